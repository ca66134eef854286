"""ctypes binding of liblad.so (include/lad.h).  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and the current HIP stream.

The functions named lad_* mirror the C entry points one to one.  `Lad` is a
small convenience wrapper that owns a context and allocates outputs as torch
tensors.  There is no CPU fallback: without a built liblad.so every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblad.so")

LAD_OK = 0
LAD_ERR_ARG = -1
LAD_ERR_CAPACITY = -2
LAD_ERR_OOM = -3
LAD_ERR_HIP = -4
LAD_ERR_STATE = -5
LAD_ERR_PAIRS = -6
LAD_ERR_NONFINITE = -7
LAD_DEBUG_NONFINITE = 1
LAD_F32 = 0
LAD_F64 = 1
LAD_PATH_AUTO = 0
LAD_PATH_PATCH = 1
LAD_PATH_ROWS = 2
LAD_PATH_PATCH_ATOMIC = 3
LAD_PATH_PATCH_LDS_ATOMIC = 4
_PATHS = {"auto": LAD_PATH_AUTO, "patch": LAD_PATH_PATCH, "rows": LAD_PATH_ROWS,
          "patch_atomic": LAD_PATH_PATCH_ATOMIC, "patch_lds_atomic": LAD_PATH_PATCH_LDS_ATOMIC}

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p


class LadError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class lad_mesh_desc(ctypes.Structure):
    _fields_ = [
        ("nv", ctypes.c_int32), ("nf", ctypes.c_int32), ("faces", _i32p),
        ("dtype", ctypes.c_int32), ("deterministic", ctypes.c_int32),
        ("patch_lds_bytes", ctypes.c_int32), ("pair_capacity", ctypes.c_int32),
        ("ns", ctypes.c_int32), ("springs", _i32p), ("rest_len", _f64p),
        ("k", ctypes.c_double),
        ("inertia", ctypes.c_int32), ("c", ctypes.c_double), ("x_tilde", _f64p),
        ("face_energy", ctypes.c_int32), ("dm_inv", _f64p), ("area", _f64p),
        ("kappa", ctypes.c_double), ("dhat", ctypes.c_double),
        ("eval_path", ctypes.c_int32),
        ("vf_capacity", ctypes.c_int32),
    ]


class lad_info(ctypes.Structure):
    _fields_ = [
        ("nv", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("nnzb_base", ctypes.c_int64), ("nnzb_active", ctypes.c_int64),
        ("hvals_capacity", ctypes.c_int64), ("npairs_active", ctypes.c_int32),
        ("npatches", ctypes.c_int32), ("lds_bytes_eval", ctypes.c_int32),
        ("lds_bytes_hvp", ctypes.c_int32), ("spring_records", ctypes.c_int64),
        ("face_records", ctypes.c_int64), ("max_colors", ctypes.c_int32),
        ("active_buffer", ctypes.c_int32), ("eval_path", ctypes.c_int32),
        ("grid_eval", ctypes.c_int32), ("host_syncs", ctypes.c_int64),
        ("nvf_active", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("pattern_ms", ctypes.c_double),
    ]


class lad_cg_stats(ctypes.Structure):
    _fields_ = [
        ("iterations", ctypes.c_int32), ("reason", ctypes.c_int32),
        ("rel_residual", ctypes.c_double), ("grad_norm", ctypes.c_double),
    ]


LAD_CG_CONVERGED, LAD_CG_NEG_CURVATURE, LAD_CG_MAX_ITERS = 0, 1, 2

EXPORTS = [
    "lad_build_pattern", "lad_get_info", "lad_get_pattern", "lad_copy_pattern",
    "lad_eval_energy_grad_hess", "lad_eval_energy_grad_hess_noalloc", "lad_hvp", "lad_newton_cg", "lad_insert_pairs",
    "lad_insert_contacts",
    "lad_jacobian_pattern", "lad_copy_jacobian_pattern", "lad_residual_jacobian",
    "lad_gauss_newton_product",
    "lad_device_status", "lad_set_debug", "lad_last_error", "lad_status_string", "lad_destroy",
]

_lib = None


def lib():
    """Load liblad.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_autodiff_mesh_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.lad_build_pattern.argtypes = [ctypes.POINTER(lad_mesh_desc), _vp,
                                        ctypes.POINTER(_vp)]
        L.lad_get_info.argtypes = [_vp, ctypes.POINTER(lad_info)]
        L.lad_get_pattern.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(_vp), ctypes.POINTER(_vp)]
        L.lad_copy_pattern.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64,
                                       ctypes.POINTER(ctypes.c_int64)]
        L.lad_eval_energy_grad_hess.argtypes = [_vp, _vp, _vp, _vp, _vp,
                                                ctypes.c_int64, _vp]
        L.lad_eval_energy_grad_hess_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp,
                                                        ctypes.c_int64, _vp]
        L.lad_hvp.argtypes = [_vp, _vp, _vp, _vp, _vp]
        L.lad_newton_cg.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_double,
                                    ctypes.POINTER(lad_cg_stats), _vp]
        L.lad_jacobian_pattern.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(_vp),
                                           ctypes.POINTER(_vp)]
        L.lad_copy_jacobian_pattern.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_int64)]
        L.lad_residual_jacobian.argtypes = [_vp, _vp, _vp, _vp, _vp]
        L.lad_gauss_newton_product.argtypes = [_vp, _vp, _vp, _vp, _vp]
        L.lad_insert_pairs.argtypes = [_vp, _vp, ctypes.c_int32, _vp]
        L.lad_insert_contacts.argtypes = [_vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, _vp]
        L.lad_device_status.argtypes = [_vp, _vp, ctypes.POINTER(ctypes.c_int32)]
        L.lad_set_debug.argtypes = [_vp, ctypes.c_int32]
        L.lad_last_error.argtypes = [_vp]
        L.lad_last_error.restype = ctypes.c_char_p
        L.lad_status_string.argtypes = [ctypes.c_int]
        L.lad_status_string.restype = ctypes.c_char_p
        L.lad_destroy.argtypes = [_vp]
        L.lad_destroy.restype = None
        for name in EXPORTS:
            f = getattr(L, name)
            if f.restype is ctypes.c_int:
                f.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().lad_status_string(int(s)).decode()
    except Exception:
        return str(s)


def _check(status: int, ctx=None):
    if status != LAD_OK:
        msg = lib().lad_last_error(ctx).decode()
        raise LadError(status, msg)


# ---------------------------------------------------------------- C entry points
def lad_build_pattern(desc: lad_mesh_desc, stream=None):
    out = _vp()
    _check(lib().lad_build_pattern(ctypes.byref(desc), _vp(stream), ctypes.byref(out)), None)
    return out


def lad_get_info(ctx) -> dict:
    info = lad_info()
    _check(lib().lad_get_info(ctx, ctypes.byref(info)), ctx)
    return {name: getattr(info, name) for name, _ in lad_info._fields_}


def lad_get_pattern(ctx, stream=None):
    nnzb = ctypes.c_int64()
    rp, ci = _vp(), _vp()
    _check(lib().lad_get_pattern(ctx, _vp(stream), ctypes.byref(nnzb),
                                 ctypes.byref(rp), ctypes.byref(ci)), ctx)
    return nnzb.value, rp.value, ci.value


def lad_copy_pattern(ctx, stream, d_row_ptr, d_col_idx, col_capacity):
    nnzb = ctypes.c_int64()
    _check(lib().lad_copy_pattern(ctx, _vp(stream), _vp(d_row_ptr), _vp(d_col_idx),
                                  int(col_capacity), ctypes.byref(nnzb)), ctx)
    return nnzb.value


def lad_eval_energy_grad_hess(ctx, d_x, d_energy, d_grad, d_hvals, capacity, stream=None):
    _check(lib().lad_eval_energy_grad_hess(ctx, _vp(d_x), _vp(d_energy), _vp(d_grad),
                                           _vp(d_hvals), int(capacity), _vp(stream)), ctx)


def lad_eval_energy_grad_hess_noalloc(ctx, d_x, d_energy, d_grad, d_hvals, capacity,
                                      stream=None):
    _check(lib().lad_eval_energy_grad_hess_noalloc(ctx, _vp(d_x), _vp(d_energy), _vp(d_grad),
                                                   _vp(d_hvals), int(capacity), _vp(stream)),
           ctx)


def lad_hvp(ctx, d_x, d_v, d_y, stream=None):
    _check(lib().lad_hvp(ctx, _vp(d_x), _vp(d_v), _vp(d_y), _vp(stream)), ctx)


def lad_newton_cg(ctx, d_x, d_g, d_p, max_iters, eta=0.0, stream=None) -> dict:
    st = lad_cg_stats()
    _check(lib().lad_newton_cg(ctx, _vp(d_x), _vp(d_g), _vp(d_p), int(max_iters), float(eta),
                               ctypes.byref(st), _vp(stream)), ctx)
    return {name: getattr(st, name) for name, _ in lad_cg_stats._fields_}


def lad_jacobian_pattern(ctx, stream=None):
    nrows, nnz = ctypes.c_int64(), ctypes.c_int64()
    rp, ci = _vp(), _vp()
    _check(lib().lad_jacobian_pattern(ctx, _vp(stream), ctypes.byref(nrows), ctypes.byref(nnz),
                                      ctypes.byref(rp), ctypes.byref(ci)), ctx)
    return nrows.value, nnz.value, rp.value, ci.value


def lad_copy_jacobian_pattern(ctx, stream, d_row_ptr, d_col_idx, col_capacity):
    nnz = ctypes.c_int64()
    _check(lib().lad_copy_jacobian_pattern(ctx, _vp(stream), _vp(d_row_ptr), _vp(d_col_idx),
                                           int(col_capacity), ctypes.byref(nnz)), ctx)
    return nnz.value


def lad_residual_jacobian(ctx, d_x, d_r, d_jvals, stream=None):
    _check(lib().lad_residual_jacobian(ctx, _vp(d_x), _vp(d_r), _vp(d_jvals), _vp(stream)), ctx)


def lad_gauss_newton_product(ctx, d_x, d_v, d_y, stream=None):
    _check(lib().lad_gauss_newton_product(ctx, _vp(d_x), _vp(d_v), _vp(d_y), _vp(stream)), ctx)


def lad_insert_contacts(ctx, d_pairs, npairs, d_vf, nvf, stream=None):
    _check(lib().lad_insert_contacts(ctx, _vp(d_pairs), int(npairs), _vp(d_vf), int(nvf),
                                     _vp(stream)), ctx)


def lad_insert_pairs(ctx, d_pairs, npairs, stream=None):
    _check(lib().lad_insert_pairs(ctx, _vp(d_pairs), int(npairs), _vp(stream)), ctx)


def lad_device_status(ctx, stream=None) -> int:
    st = ctypes.c_int32()
    _check(lib().lad_device_status(ctx, _vp(stream), ctypes.byref(st)), ctx)
    return st.value


def lad_destroy(ctx):
    lib().lad_destroy(ctx)


# ---------------------------------------------------------------- convenience
def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a, t):
    return ctypes.cast(None, t) if a is None else a.ctypes.data_as(t)


def make_desc(nv, faces=None, springs=None, rest_len=None, k=0.0, x_tilde=None, c=0.0,
              face_energy=False, dm_inv=None, area=None, pair_capacity=0, kappa=0.0,
              dhat=0.0, dtype="f32", deterministic=False, patch_lds_bytes=0, path="auto",
              vf_capacity=0):
    """Fill a lad_mesh_desc from numpy arrays.  Returns (desc, keepalive)."""
    keep = {
        "faces": _i32(faces if faces is not None else np.zeros((0, 3))),
        "springs": _i32(springs) if springs is not None else None,
        "rest_len": _f64(rest_len),
        "x_tilde": _f64(x_tilde),
        "dm_inv": _f64(dm_inv),
        "area": _f64(area),
    }
    d = lad_mesh_desc()
    d.nv = int(nv)
    d.nf = keep["faces"].reshape(-1, 3).shape[0]
    d.faces = _ptr(keep["faces"], _i32p)
    d.dtype = LAD_F64 if dtype in ("f64", "float64", np.float64) else LAD_F32
    d.deterministic = 1 if deterministic else 0
    d.patch_lds_bytes = int(patch_lds_bytes)
    d.pair_capacity = int(pair_capacity)
    d.ns = 0 if springs is None else keep["springs"].reshape(-1, 2).shape[0]
    d.springs = _ptr(keep["springs"], _i32p)
    d.rest_len = _ptr(keep["rest_len"], _f64p)
    d.k = float(k)
    d.inertia = 0 if x_tilde is None else 1
    d.c = float(c)
    d.x_tilde = _ptr(keep["x_tilde"], _f64p)
    d.face_energy = 1 if face_energy else 0
    d.dm_inv = _ptr(keep["dm_inv"], _f64p)
    d.area = _ptr(keep["area"], _f64p)
    d.kappa = float(kappa)
    d.dhat = float(dhat)
    d.eval_path = _PATHS[path] if isinstance(path, str) else int(path)
    d.vf_capacity = int(vf_capacity)
    return d, keep


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


class Lad:
    """One context on the current device; outputs as torch tensors."""

    def __init__(self, nv, dtype="f32", **terms):
        import torch
        self.torch = torch
        self.nv = int(nv)
        self.dtype = torch.float64 if dtype in ("f64", "float64") else torch.float32
        desc, self._keep = make_desc(nv, dtype=dtype, **terms)
        self.ctx = lad_build_pattern(desc, _stream())
        self.info = lad_get_info(self.ctx)
        self.capacity = self.info["hvals_capacity"]
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self):
        if getattr(self, "ctx", None) is not None:
            lad_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_outputs(self):
        t = self.torch
        E = t.empty(1, dtype=t.float64, device=self.device)
        g = t.empty((self.nv, 3), dtype=self.dtype, device=self.device)
        H = t.empty((self.capacity, 3, 3), dtype=self.dtype, device=self.device)
        return E, g, H

    def eval(self, x, out=None, energy=True):
        """(energy[1] fp64, g (nv,3), hvals (capacity,3,3)); the first
        nnzb_active blocks of hvals are valid.  With energy=False the energy
        is not computed (NULL is passed) and E is left untouched."""
        assert x.dtype == self.dtype and x.is_cuda and x.is_contiguous()
        E, g, H = out if out is not None else self.alloc_outputs()
        lad_eval_energy_grad_hess(self.ctx, x.data_ptr(), E.data_ptr() if energy else None,
                                  g.data_ptr(), H.data_ptr(), H.shape[0], _stream())
        return E, g, H

    def hvp(self, x, v, out=None):
        assert x.dtype == self.dtype and v.dtype == self.dtype
        y = out if out is not None else self.torch.empty_like(v)
        lad_hvp(self.ctx, x.data_ptr(), v.data_ptr(), y.data_ptr(), _stream())
        return y

    def newton_cg(self, x, g, out=None, max_iters=100, eta=0.0):
        """Truncated Newton-CG direction p (H(x) p ~ -g); returns (p, stats)."""
        assert x.dtype == self.dtype and g.dtype == self.dtype
        assert x.is_contiguous() and g.is_contiguous()
        p = out if out is not None else self.torch.empty_like(g)
        stats = lad_newton_cg(self.ctx, x.data_ptr(), g.data_ptr(), p.data_ptr(), max_iters,
                              eta, _stream())
        return p, stats

    def jacobian_pattern(self):
        """(row_ptr, col_idx) of the vector objective's Jacobian, copied into
        new int32 tensors."""
        t = self.torch
        nrows, nnz, _, _ = lad_jacobian_pattern(self.ctx, _stream())
        row_ptr = t.empty(nrows + 1, dtype=t.int32, device=self.device)
        col_idx = t.empty(max(nnz, 1), dtype=t.int32, device=self.device)
        lad_copy_jacobian_pattern(self.ctx, _stream(), row_ptr.data_ptr(), col_idx.data_ptr(),
                                  col_idx.numel())
        return row_ptr, col_idx[:nnz]

    def residual_jacobian(self, x, out=None):
        """(R [nrows], J values [nnz]) at x."""
        assert x.dtype == self.dtype and x.is_contiguous()
        if out is None:
            nrows, nnz, _, _ = lad_jacobian_pattern(self.ctx, _stream())
            out = (self.torch.empty(nrows, dtype=self.dtype, device=self.device),
                   self.torch.empty(max(nnz, 1), dtype=self.dtype, device=self.device))
        R, Jv = out
        lad_residual_jacobian(self.ctx, x.data_ptr(), R.data_ptr(), Jv.data_ptr(), _stream())
        return R, Jv

    def gauss_newton(self, x, v, out=None):
        assert x.dtype == self.dtype and v.dtype == self.dtype
        y = out if out is not None else self.torch.empty_like(v)
        lad_gauss_newton_product(self.ctx, x.data_ptr(), v.data_ptr(), y.data_ptr(), _stream())
        return y

    def insert_contacts(self, pairs=None, vf=None):
        """pairs: int32 cuda tensor (P, 2) or None; vf: int32 cuda tensor
        (Q, 2) of (vertex, face id) or None.  Both empty restores the
        topology pattern."""
        np_ = 0 if pairs is None else pairs.shape[0]
        nvf = 0 if vf is None else vf.shape[0]
        for t in (pairs, vf):
            if t is not None and t.numel():
                assert t.dtype == self.torch.int32 and t.is_cuda and t.is_contiguous()
        lad_insert_contacts(self.ctx, pairs.data_ptr() if np_ else None, np_,
                            vf.data_ptr() if nvf else None, nvf, _stream())

    def insert_pairs(self, pairs):
        """pairs: int32 cuda tensor (P, 2), or None / empty for no pairs."""
        if pairs is None or pairs.numel() == 0:
            lad_insert_pairs(self.ctx, None, 0, _stream())
            return
        assert pairs.dtype == self.torch.int32 and pairs.is_cuda and pairs.is_contiguous()
        lad_insert_pairs(self.ctx, pairs.data_ptr(), pairs.shape[0], _stream())

    def pattern(self):
        t = self.torch
        rp = t.empty(self.nv + 1, dtype=t.int32, device=self.device)
        ci = t.empty(max(self.capacity, 1), dtype=t.int32, device=self.device)
        nnzb = lad_copy_pattern(self.ctx, _stream(), rp.data_ptr(), ci.data_ptr(), ci.numel())
        return rp, ci[:nnzb]

    def device_status(self) -> int:
        return lad_device_status(self.ctx, _stream())

    def set_debug(self, flags: int) -> None:
        _check(lib().lad_set_debug(self.ctx, int(flags)), self.ctx)

    def get_info(self) -> dict:
        return lad_get_info(self.ctx)


def mesh_terms(mesh, springs=True, inertia=True, faces=False, pair_capacity=0,
               kappa=0.0, dhat=0.0, vf_capacity=0):
    """Keyword arguments of Lad(...) for a generated grid bundle."""
    kw = {"faces": mesh.faces}
    if springs:
        kw.update(springs=mesh.springs, rest_len=mesh.rest_len, k=mesh.params.get("k", 0.0))
    if inertia:
        kw.update(x_tilde=mesh.X, c=mesh.params.get("c", 0.0))
    if faces:
        kw.update(face_energy=True, dm_inv=mesh.dm_inv, area=mesh.area)
    if pair_capacity or vf_capacity:
        kw.update(pair_capacity=pair_capacity, vf_capacity=vf_capacity, kappa=kappa, dhat=dhat)
    return kw
