"""The C ABI without a GPU: liblad.so loads, exports every entry point that
include/lad.h declares, and rejects bad arguments on the host before any GPU
work (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_autodiff_mesh_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lad.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lad_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("liblad.so not built")
    return binding.lib()


def test_exports_match_header(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in lad.h but not exported"
    assert set(names) == set(binding.EXPORTS)


def test_status_strings(L):
    for code, name in [(0, "LAD_OK"), (-1, "LAD_ERR_ARG"), (-2, "LAD_ERR_CAPACITY"),
                       (-3, "LAD_ERR_OOM"), (-4, "LAD_ERR_HIP"), (-5, "LAD_ERR_STATE"),
                       (-6, "LAD_ERR_PAIRS"), (-7, "LAD_ERR_NONFINITE")]:
        assert L.lad_status_string(code).decode() == name


def test_set_debug_rejects_null_context(L):
    assert L.lad_set_debug(None, binding.LAD_DEBUG_NONFINITE) == binding.LAD_ERR_ARG


def build_status(desc):
    out = ctypes.c_void_p()
    rc = binding.lib().lad_build_pattern(ctypes.byref(desc) if desc is not None else None,
                                         None, ctypes.byref(out))
    return rc, out.value, binding.lib().lad_last_error(None).decode()


def tri_desc(**kw):
    faces = np.array([[0, 1, 2]], dtype=np.int32)
    springs = np.array([[0, 1], [1, 2], [0, 2]], dtype=np.int32)
    base = dict(faces=faces, springs=springs, rest_len=np.ones(3), k=1.0)
    base.update(kw)
    return binding.make_desc(3, **base)


@pytest.mark.parametrize("mutate,msg", [
    (lambda d: setattr(d, "nv", 0), "nv"),
    (lambda d: setattr(d, "dtype", 7), "dtype"),
    (lambda d: setattr(d, "pair_capacity", -1), "pair_capacity"),
    (lambda d: setattr(d, "eval_path", 9), "eval_path"),
    (lambda d: setattr(d, "patch_lds_bytes", 1 << 20), "patch_lds_bytes"),
    (lambda d: setattr(d, "ns", -2), "ns"),
    (lambda d: (setattr(d, "eval_path", binding.LAD_PATH_PATCH_ATOMIC),
                setattr(d, "deterministic", 1)), "LAD_PATH_PATCH_ATOMIC"),
    (lambda d: (setattr(d, "eval_path", binding.LAD_PATH_PATCH_ATOMIC),
                setattr(d, "pair_capacity", 4), setattr(d, "dhat", 0.1)), "LAD_PATH_PATCH_ATOMIC"),
    (lambda d: (setattr(d, "eval_path", binding.LAD_PATH_PATCH_LDS_ATOMIC),
                setattr(d, "deterministic", 1)), "LAD_PATH_PATCH_LDS_ATOMIC"),
])
def test_bad_descriptor_fields(L, mutate, msg):
    d, keep = tri_desc()
    mutate(d)
    rc, ctx, err = build_status(d)
    assert rc == binding.LAD_ERR_ARG and ctx is None
    assert msg in err


def test_bad_indices(L):
    d, keep = tri_desc(faces=np.array([[0, 1, 5]], dtype=np.int32))
    rc, ctx, err = build_status(d)
    assert rc == binding.LAD_ERR_ARG and "out of range" in err
    d, keep = tri_desc(springs=np.array([[0, 0], [1, 2], [0, 2]], dtype=np.int32))
    rc, ctx, err = build_status(d)
    assert rc == binding.LAD_ERR_ARG and "a == b" in err
    d, keep = tri_desc(faces=np.array([[0, 1, 1]], dtype=np.int32))
    rc, ctx, err = build_status(d)
    assert rc == binding.LAD_ERR_ARG and "repeated" in err


def test_missing_arrays_and_values(L):
    d, keep = tri_desc()
    d.rest_len = ctypes.cast(None, ctypes.POINTER(ctypes.c_double))
    assert build_status(d)[0] == binding.LAD_ERR_ARG
    d, keep = tri_desc(x_tilde=None)
    d.inertia = 1
    assert build_status(d)[0] == binding.LAD_ERR_ARG
    d, keep = tri_desc(pair_capacity=4, dhat=0.0)
    assert build_status(d)[0] == binding.LAD_ERR_ARG
    d, keep = tri_desc(rest_len=np.array([1.0, np.nan, 1.0]))
    assert build_status(d)[0] == binding.LAD_ERR_ARG
    d, keep = tri_desc(face_energy=True)
    assert build_status(d)[0] == binding.LAD_ERR_ARG  # no dm_inv / area
    rc, ctx, err = build_status(None)
    assert rc == binding.LAD_ERR_ARG


def test_null_context_calls(L):
    vp = ctypes.c_void_p
    assert L.lad_eval_energy_grad_hess(None, vp(1), vp(1), vp(1), vp(1), 10, None) == binding.LAD_ERR_ARG
    assert L.lad_hvp(None, vp(1), vp(1), vp(1), None) == binding.LAD_ERR_ARG
    assert L.lad_insert_pairs(None, None, 0, None) == binding.LAD_ERR_ARG
    assert L.lad_residual_jacobian(None, vp(1), vp(1), vp(1), None) == binding.LAD_ERR_ARG
    assert L.lad_gauss_newton_product(None, vp(1), vp(1), vp(1), None) == binding.LAD_ERR_ARG
    n64 = ctypes.c_int64()
    assert L.lad_copy_jacobian_pattern(None, None, vp(1), vp(1), 10,
                                       ctypes.byref(n64)) == binding.LAD_ERR_ARG
    st = binding.lad_cg_stats()
    assert L.lad_newton_cg(None, vp(1), vp(1), vp(2), 10, 0.0, ctypes.byref(st),
                           None) == binding.LAD_ERR_ARG
    info = binding.lad_info()
    assert L.lad_get_info(None, ctypes.byref(info)) == binding.LAD_ERR_ARG
    L.lad_destroy(None)  # no-op
