"""Host checks of bench.py's bookkeeping: the fingerprint that ties the
committed counter summaries to the kernel sources covers their code and
not their comments or layout."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_keeps_code():
    src = ('// header\nint a = 1; /* block\n comment */ int b = 2;\n'
           'const char *s = "// not a comment /* either */";\n'
           "char q = '\\''; // trailing\n"
           "#define X(y) (y) /* in a macro */\n")
    out = bench.code_only(src)
    assert "header" not in out and "block" not in out and "trailing" not in out
    assert "in a macro" not in out
    assert 'const char *s = "// not a comment /* either */";' in out
    assert "char q = '\\'';" in out
    assert "int a = 1; int b = 2;" in out
    assert "#define X(y) (y)" in out


def test_code_only_ignores_layout_and_comment_edits():
    a = "int f(int x) {\n  // doubles x\n  return 2 * x;\n}\n"
    b = "int f(int x) { /* twice x */ return 2 * x; }"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)

