"""Host logic without a GPU: the patch plan (contiguous-row patches, ribbon
vertices, per-patch element records and slots, colours, LDS budget; every
element evaluated once per patch owning one of its vertices) and the row
plan (row chunks, per-block rest lengths, per-row face incidence, rejected
inputs), checked by tests/native/plan_check.cpp against patterns and
incidences it derives itself, on grids and random irregular meshes."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    cmd = [HIPCC, "-std=c++17", "-O1", f"-I{ROOT}/include",
           f"-I{ROOT}/sparse_autodiff_mesh_amd/csrc",
           f"{ROOT}/tests/native/plan_check.cpp",
           f"{ROOT}/sparse_autodiff_mesh_amd/csrc/lad_patch.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_patch_and_row_plans(plan_check):
    r = subprocess.run([plan_check], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all plan checks passed" in r.stdout
