"""Build liblad.so (HIP kernels for gfx950 + host C++ API) in-tree.

    python -m sparse_autodiff_mesh_amd.build [--verbose]

Each source compiles to its own object under _build/, then one shared
library is linked next to this file.  Device code is built without packed
FP32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblad.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["lad_eval.hip", "lad_rows.hip", "lad_pattern.hip", "lad_insert.hip",
               "lad_solve.hip", "lad_jacobian.hip", "lad_vf.hip", "lad_terms.hip",
               "lad_noalloc.hip"]
CXX_SOURCES = ["lad_api.cpp", "lad_patch.cpp", "lad_terms_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-result"]
# Device code: no packed-FP32 instructions; finite math without signed
# zeros, so the compiler may fold the structural zeros of the dual-number
# seeds (x * 0 -> 0, x + 0 -> x).  Neither flag reassociates or changes
# rounding.
DEVICE = [f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffinite-math-only", "-fno-signed-zeros"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CXX_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
