"""Host checks of bench.py's bookkeeping: the fingerprint that ties the
committed counter summaries to the kernel sources covers their code and
not their comments or layout, and the timer's warm-up keeps calling until
its time floor has passed (with a stand-in for torch's device calls)."""
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



class _FakeEvent:
    def __init__(self, enable_timing=False):
        self.t = 0.0

    def record(self):
        self.t = _FakeCuda.clock

    def elapsed_time(self, other):
        return other.t - self.t


class _FakeCuda:
    clock = 0.0
    Event = _FakeEvent

    @staticmethod
    def synchronize():
        pass


class _FakeTorch:
    cuda = _FakeCuda


def _counting_call(sleep_s):
    import time
    calls = []

    def fn():
        calls.append(1)
        _FakeCuda.clock += 1.0
        time.sleep(sleep_s)
    return fn, calls


def test_timer_warms_up_for_the_time_floor():
    # 2 ms calls, 2 counted warm-up calls, a 40 ms floor: the warm-up goes
    # on past the counted calls (about 20 calls), then exactly the timed
    # steps run twice (the region and the per-call pass)
    fn, calls = _counting_call(0.002)
    r = bench.Timer(_FakeTorch, min_warm_s=0.04).run(fn, steps=5, warmup=2)
    warm = len(calls) - 2 * 5
    assert 12 <= warm
    assert warm % 2 == 0  # whole rounds of the counted warm-up
    assert r["median_ms"] == 1.0 and r["region_ms"] == 5.0


def test_timer_without_warmup_runs_only_the_timed_calls():
    fn, calls = _counting_call(0.0)
    bench.Timer(_FakeTorch, min_warm_s=10.0).run(fn, steps=3, warmup=0)
    assert len(calls) == 2 * 3
