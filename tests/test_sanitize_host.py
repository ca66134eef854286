"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the plan builders (sparse_autodiff_mesh_amd/csrc/lad_patch.cpp, driven
by tests/native/plan_check.cpp over grids and random irregular meshes) and
the CPU oracle (oracle/oracle.c, driven by tests/native/oracle_check.c over
a grid carrying every term kind, plus malformed problems).  Both are built
with the host compilers (g++ / gcc; no device code is involved) and any
sanitizer report aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, exe, expect):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert expect in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_builders_sanitized(tmp_path):
    exe = str(tmp_path / "plan_check_san")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{ROOT}/include", f"-I{ROOT}/sparse_autodiff_mesh_amd/csrc",
           f"{ROOT}/tests/native/plan_check.cpp",
           f"{ROOT}/sparse_autodiff_mesh_amd/csrc/lad_patch.cpp", "-o", exe]
    _run(cmd, exe, "all plan checks passed")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_check_san")
    cmd = ["gcc", "-std=c11", *SAN, "-ffp-contract=off", f"-I{ROOT}/oracle",
           f"{ROOT}/tests/native/oracle_check.c", f"{ROOT}/oracle/oracle.c", "-o", exe, "-lm"]
    _run(cmd, exe, "all oracle checks passed")
