"""ctypes binding of the term front end (include/lad_terms.h): argument
marshalling only.  Every step of the evaluation runs in liblad.so's
kernels; there is no CPU fallback, and every call raises if the library is
missing."""
from __future__ import annotations

import ctypes

import numpy as np

from . import binding
from .binding import LadError, _stream

SETS = {"cloth": 1, "arap": 2, "symdir": 3, "arap_cloth": 4, "cloth_quad": 5}

TERMS_EXPORTS = [
    "lad_terms_describe", "lad_terms_build", "lad_terms_eval", "lad_terms_hvp",
    "lad_terms_get_pattern", "lad_terms_copy_pattern", "lad_terms_last_error",
    "lad_terms_host_syncs", "lad_terms_destroy",
]

_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


class lad_term_block(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("elems", _i32p), ("consts", _f64p)]


class lad_terms_desc(ctypes.Structure):
    _fields_ = [
        ("nv", ctypes.c_int32), ("dtype", ctypes.c_int32), ("set", ctypes.c_int32),
        ("fused", ctypes.c_int32), ("nblocks", ctypes.c_int32),
        ("blocks", ctypes.POINTER(lad_term_block)),
    ]


_typed = False


def lib():
    global _typed
    L = binding.lib()
    if not _typed:
        L.lad_terms_describe.argtypes = [ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p,
                                         ctypes.POINTER(ctypes.c_char_p)]
        L.lad_terms_build.argtypes = [ctypes.POINTER(lad_terms_desc), _vp, ctypes.POINTER(_vp)]
        L.lad_terms_eval.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _vp]
        L.lad_terms_hvp.argtypes = [_vp, _vp, _vp, _vp, _vp]
        L.lad_terms_get_pattern.argtypes = [_vp, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(_vp), ctypes.POINTER(_vp)]
        L.lad_terms_copy_pattern.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64,
                                             ctypes.POINTER(ctypes.c_int64)]
        L.lad_terms_last_error.argtypes = [_vp]
        L.lad_terms_last_error.restype = ctypes.c_char_p
        L.lad_terms_host_syncs.argtypes = [_vp]
        L.lad_terms_host_syncs.restype = ctypes.c_int64
        L.lad_terms_destroy.argtypes = [_vp]
        L.lad_terms_destroy.restype = None
        _typed = True
    return L


def _check(status: int, ctx=None):
    if status != 0:
        raise LadError(status, lib().lad_terms_last_error(ctx).decode())


def describe(set_id) -> list:
    """[(name, arity, nconst)] of the set's terms, in order."""
    s = SETS.get(set_id, set_id)
    n = ctypes.c_int32()
    st = lib().lad_terms_describe(int(s), -1, ctypes.byref(n), None, None, None)
    if st != 0:
        raise LadError(st, f"unknown term set {set_id}")
    out = []
    for t in range(n.value):
        ar, nc, nm = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_char_p()
        _check(lib().lad_terms_describe(int(s), t, None, ctypes.byref(ar), ctypes.byref(nc),
                                        ctypes.byref(nm)))
        out.append((nm.value.decode(), ar.value, nc.value))
    return out


def make_desc(nv, set_id, blocks, dtype="f32", fused=True):
    """Descriptor for `blocks` = [(elems int (count, arity), consts float
    (count, nconst)), ...] in the set's term order; returns (desc, keep)."""
    keep = []
    arr = (lad_term_block * max(len(blocks), 1))()
    for i, (el, cs) in enumerate(blocks):
        el = np.ascontiguousarray(el, dtype=np.int32)
        cs = np.ascontiguousarray(cs, dtype=np.float64)
        keep += [el, cs]
        arr[i].count = el.shape[0] if el.ndim > 1 else (0 if el.size == 0 else 1)
        arr[i].elems = el.ctypes.data_as(_i32p) if el.size else None
        arr[i].consts = cs.ctypes.data_as(_f64p) if cs.size else None
    keep.append(arr)
    d = lad_terms_desc()
    d.nv = int(nv)
    d.dtype = 1 if dtype in ("f64", "float64") else 0
    d.set = int(SETS.get(set_id, set_id))
    d.fused = 1 if fused else 0
    d.nblocks = len(blocks)
    d.blocks = ctypes.cast(arr, ctypes.POINTER(lad_term_block))
    return d, keep


def build(desc, stream=None):
    out = _vp()
    _check(lib().lad_terms_build(ctypes.byref(desc), _vp(stream), ctypes.byref(out)), None)
    return out


class Terms:
    """One term-set context on the current device; outputs as torch tensors."""

    def __init__(self, nv, set_id, blocks, dtype="f32", fused=True):
        import torch
        self.torch = torch
        self.nv = int(nv)
        self.dtype = torch.float64 if dtype in ("f64", "float64") else torch.float32
        desc, self._keep = make_desc(nv, set_id, blocks, dtype=dtype, fused=fused)
        self.ctx = build(desc, _stream())
        n = ctypes.c_int64()
        rp, ci = _vp(), _vp()
        _check(lib().lad_terms_get_pattern(self.ctx, ctypes.byref(n), ctypes.byref(rp),
                                           ctypes.byref(ci)), self.ctx)
        self.nnzb = n.value
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self):
        if getattr(self, "ctx", None) is not None:
            lib().lad_terms_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_outputs(self):
        t = self.torch
        return (t.empty(1, dtype=t.float64, device=self.device),
                t.empty((self.nv, 3), dtype=self.dtype, device=self.device),
                t.empty((self.nnzb, 3, 3), dtype=self.dtype, device=self.device))

    def eval(self, x, out=None, energy=True):
        assert x.dtype == self.dtype and x.is_cuda and x.is_contiguous()
        E, g, H = out if out is not None else self.alloc_outputs()
        _check(lib().lad_terms_eval(self.ctx, x.data_ptr(), E.data_ptr() if energy else None,
                                    g.data_ptr(), H.data_ptr(), H.shape[0], _stream()), self.ctx)
        return E, g, H

    def hvp(self, x, v, out=None):
        assert x.dtype == self.dtype and v.dtype == self.dtype
        assert x.is_contiguous() and v.is_contiguous()
        y = out if out is not None else self.torch.empty_like(v)
        _check(lib().lad_terms_hvp(self.ctx, x.data_ptr(), v.data_ptr(), y.data_ptr(),
                                   _stream()), self.ctx)
        return y

    def host_syncs(self) -> int:
        return int(lib().lad_terms_host_syncs(self.ctx))

    def pattern(self):
        t = self.torch
        rp = t.empty(self.nv + 1, dtype=t.int32, device=self.device)
        ci = t.empty(max(self.nnzb, 1), dtype=t.int32, device=self.device)
        n = ctypes.c_int64()
        _check(lib().lad_terms_copy_pattern(self.ctx, _stream(), rp.data_ptr(), ci.data_ptr(),
                                            ci.numel(), ctypes.byref(n)), self.ctx)
        return rp, ci[: n.value]


def mesh_blocks(mesh, set_id, k=None, c=None, kq=1.0):
    """Term blocks of a generated grid bundle for one of the compiled sets:
    springs with (rest length, k), one inertia element per vertex with
    (rest position, c), faces with (Dm^-1, rest area), grid cells as
    planarity quads with (kq)."""
    kk = mesh.params.get("k", 0.0) if k is None else k
    cc = mesh.params.get("c", 0.0) if c is None else c
    spring = (mesh.springs, np.stack([mesh.rest_len, np.full(len(mesh.rest_len), kk)], axis=1))
    inertia = (np.arange(mesh.nv, dtype=np.int32).reshape(-1, 1),
               np.concatenate([mesh.X, np.full((mesh.nv, 1), cc)], axis=1))
    face = (mesh.faces, np.concatenate([mesh.dm_inv, mesh.area.reshape(-1, 1)], axis=1))
    name = {v: k_ for k_, v in SETS.items()}.get(set_id, set_id)
    if name == "cloth_quad":
        from .inputs import grid_quads
        q = grid_quads(mesh.n)
        return [spring, inertia, (q, np.full((len(q), 1), float(kq)))]
    return {"cloth": [spring, inertia], "arap": [face], "symdir": [face],
            "arap_cloth": [face, spring, inertia]}[name]
