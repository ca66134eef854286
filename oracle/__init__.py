"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library and its binding never import it.

What it computes follows the page "Locality-Aware Automatic Differentiation on
the GPU for Mesh-Based Computations", section "Method" (F(x) = sum_j f_j(x_j),
g = sum_j S_j^T g_j, H = sum_j S_j^T H_j S_j) and key designs 3 and 4
(block-CSR pattern from the mesh topology plus runtime vertex-vertex pairs).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


class OracleProblem(ctypes.Structure):
    _fields_ = [
        ("nv", ctypes.c_int32), ("nf", ctypes.c_int32), ("faces", _i32p),
        ("ns", ctypes.c_int32), ("springs", _i32p), ("rest_len", _f64p),
        ("k", ctypes.c_double),
        ("inertia", ctypes.c_int32), ("c", ctypes.c_double), ("x_tilde", _f64p),
        ("face_energy", ctypes.c_int32), ("dm_inv", _f64p), ("area", _f64p),
        ("np", ctypes.c_int32), ("pairs", _i32p),
        ("kappa", ctypes.c_double), ("dhat", ctypes.c_double),
        ("nvf", ctypes.c_int32), ("vf", _i32p),
        ("nq", ctypes.c_int32), ("quads", _i32p), ("kq", ctypes.c_double),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.oracle_pattern_nnzb.restype = ctypes.c_int64
        L.oracle_pattern_nnzb.argtypes = [ctypes.POINTER(OracleProblem)]
        L.oracle_pattern.argtypes = [ctypes.POINTER(OracleProblem), _i32p, _i32p]
        L.oracle_eval.argtypes = [ctypes.POINTER(OracleProblem), _i32p, _i32p,
                                  _f64p, _f64p, _f64p, _f64p]
        L.oracle_hvp.argtypes = [ctypes.POINTER(OracleProblem), _i32p, _i32p,
                                 _f64p, _f64p, _f64p]
        L.oracle_bsr_spmv.argtypes = [ctypes.c_int32, _i32p, _i32p, _f64p, _f64p, _f64p]
        L.oracle_spring_local.argtypes = [_f64p, _f64p, ctypes.c_double,
                                          ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_spring_local.restype = None
        L.oracle_barrier_local.argtypes = [_f64p, _f64p, ctypes.c_double,
                                           ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_barrier_local.restype = None
        L.oracle_barrier_scalar.argtypes = [ctypes.c_double, ctypes.c_double,
                                            ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_barrier_scalar.restype = None
        L.oracle_inertia_local.argtypes = [_f64p, _f64p, ctypes.c_double,
                                           _f64p, _f64p, _f64p]
        L.oracle_inertia_local.restype = None
        L.oracle_face_local.argtypes = [_f64p, _f64p, _f64p, _f64p,
                                        ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_face_local.restype = None
        L.oracle_quad_local.argtypes = [_f64p, _f64p, _f64p, _f64p, ctypes.c_double,
                                        _f64p, _f64p, _f64p]
        L.oracle_quad_local.restype = None
        L.oracle_arap_local.argtypes = [_f64p, _f64p, _f64p, _f64p,
                                        ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_arap_local.restype = None
        L.oracle_face_grad_hyperdual.argtypes = [_f64p, _f64p, _f64p, _f64p,
                                                 ctypes.c_double, _f64p]
        L.oracle_face_grad_hyperdual.restype = None
        L.oracle_vf_local.argtypes = [_f64p, _f64p, _f64p, _f64p, ctypes.c_double,
                                      ctypes.c_double, _f64p, _f64p, _f64p]
        L.oracle_vf_local.restype = None
        L.oracle_vf_distance_type.argtypes = [_f64p, _f64p, _f64p, _f64p]
        L.oracle_vf_distance_type.restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else ctypes.cast(None, t)


class Problem:
    """Energy terms of one evaluation.  Arrays are copied to contiguous fp64 /
    int32 and kept alive for the lifetime of the object."""

    def __init__(self, nv, faces=None, springs=None, rest_len=None, k=0.0,
                 x_tilde=None, c=0.0, face_energy=False, dm_inv=None, area=None,
                 pairs=None, kappa=0.0, dhat=0.0, vf=None, quads=None, kq=0.0):
        self.nv = int(nv)
        self.faces = _i32(faces if faces is not None else np.zeros((0, 3))).reshape(-1, 3)
        self.springs = _i32(springs if springs is not None else np.zeros((0, 2))).reshape(-1, 2)
        self.rest_len = _f64(rest_len if rest_len is not None else np.zeros(0))
        self.k = float(k)
        self.inertia = x_tilde is not None
        self.x_tilde = _f64(x_tilde).reshape(-1, 3) if x_tilde is not None else None
        self.c = float(c)
        # face term: False/None/0 none, True/1/"sd" symmetric Dirichlet, 2/"arap"
        self.face_energy = {None: 0, False: 0, 0: 0, True: 1, 1: 1, "sd": 1, 2: 2,
                            "arap": 2}[face_energy]
        self.dm_inv = _f64(dm_inv).reshape(-1, 4) if dm_inv is not None else None
        self.area = _f64(area) if area is not None else None
        self.pairs = _i32(pairs if pairs is not None else np.zeros((0, 2))).reshape(-1, 2)
        self.kappa = float(kappa)
        self.dhat = float(dhat)
        self.vf = _i32(vf if vf is not None else np.zeros((0, 2))).reshape(-1, 2)
        self.quads = _i32(quads if quads is not None else np.zeros((0, 4))).reshape(-1, 4)
        self.kq = float(kq)

    def with_pairs(self, pairs, kappa=None, dhat=None):
        import copy
        q = copy.copy(self)
        q.pairs = _i32(pairs).reshape(-1, 2)
        if kappa is not None:
            q.kappa = float(kappa)
        if dhat is not None:
            q.dhat = float(dhat)
        return q

    def struct(self) -> OracleProblem:
        s = OracleProblem()
        s.nv = self.nv
        s.nf = self.faces.shape[0]
        s.faces = _p(self.faces, _i32p)
        s.ns = self.springs.shape[0]
        s.springs = _p(self.springs, _i32p)
        s.rest_len = _p(self.rest_len, _f64p)
        s.k = self.k
        s.inertia = 1 if self.inertia else 0
        s.c = self.c
        s.x_tilde = _p(self.x_tilde, _f64p)
        s.face_energy = self.face_energy
        s.dm_inv = _p(self.dm_inv, _f64p)
        s.area = _p(self.area, _f64p)
        s.np = self.pairs.shape[0]
        s.pairs = _p(self.pairs, _i32p)
        s.kappa = self.kappa
        s.dhat = self.dhat
        s.nvf = self.vf.shape[0]
        s.vf = _p(self.vf, _i32p)
        s.nq = self.quads.shape[0]
        s.quads = _p(self.quads, _i32p)
        s.kq = self.kq
        return s


def pattern(prob: Problem):
    s = prob.struct()
    nnzb = lib().oracle_pattern_nnzb(ctypes.byref(s))
    if nnzb < 0:
        raise ValueError(f"oracle_pattern_nnzb failed ({nnzb})")
    row_ptr = np.zeros(prob.nv + 1, dtype=np.int32)
    col_idx = np.zeros(max(nnzb, 1), dtype=np.int32)
    rc = lib().oracle_pattern(ctypes.byref(s), _p(row_ptr, _i32p), _p(col_idx, _i32p))
    if rc:
        raise ValueError(f"oracle_pattern failed ({rc})")
    return row_ptr, col_idx[:nnzb]


def evaluate(prob: Problem, row_ptr, col_idx, x):
    """Returns (energy, g (nv, 3), hvals (nnzb, 3, 3))."""
    s = prob.struct()
    row_ptr = _i32(row_ptr)
    col_idx = _i32(col_idx)
    x = _f64(x).reshape(-1, 3)
    nnzb = int(row_ptr[-1])
    E = np.zeros(1)
    g = np.zeros((prob.nv, 3))
    H = np.zeros((max(nnzb, 1), 3, 3))
    rc = lib().oracle_eval(ctypes.byref(s), _p(row_ptr, _i32p), _p(col_idx, _i32p),
                           _p(x, _f64p), _p(E, _f64p), _p(g, _f64p), _p(H, _f64p))
    if rc:
        raise ValueError(f"oracle_eval failed ({rc})")
    return float(E[0]), g, H[:nnzb]


def hvp(prob: Problem, row_ptr, col_idx, x, v):
    s = prob.struct()
    row_ptr = _i32(row_ptr)
    col_idx = _i32(col_idx)
    x = _f64(x).reshape(-1, 3)
    v = _f64(v).reshape(-1, 3)
    y = np.zeros((prob.nv, 3))
    rc = lib().oracle_hvp(ctypes.byref(s), _p(row_ptr, _i32p), _p(col_idx, _i32p),
                          _p(x, _f64p), _p(v, _f64p), _p(y, _f64p))
    if rc:
        raise ValueError(f"oracle_hvp failed ({rc})")
    return y


def bsr_spmv(row_ptr, col_idx, hvals, v):
    row_ptr = _i32(row_ptr)
    col_idx = _i32(col_idx)
    hvals = _f64(hvals)
    v = _f64(v).reshape(-1, 3)
    nv = row_ptr.size - 1
    y = np.zeros((nv, 3))
    rc = lib().oracle_bsr_spmv(nv, _p(row_ptr, _i32p), _p(col_idx, _i32p),
                               _p(hvals, _f64p), _p(v, _f64p), _p(y, _f64p))
    if rc:
        raise ValueError("oracle_bsr_spmv failed")
    return y


def _local(fn, m, *args):
    E = np.zeros(1)
    g = np.zeros(3 * m)
    H = np.zeros((3 * m, 3 * m))
    fn(*args, _p(E, _f64p), _p(g, _f64p), _p(H, _f64p))
    return float(E[0]), g, H


def spring_local(xa, xb, rest, k):
    xa, xb = _f64(xa), _f64(xb)
    return _local(lib().oracle_spring_local, 2, _p(xa, _f64p), _p(xb, _f64p),
                  float(rest), float(k))


def barrier_local(xa, xb, kappa, dhat):
    xa, xb = _f64(xa), _f64(xb)
    return _local(lib().oracle_barrier_local, 2, _p(xa, _f64p), _p(xb, _f64p),
                  float(kappa), float(dhat))


def barrier_scalar(d, kappa, dhat):
    out = np.zeros(3)
    lib().oracle_barrier_scalar(float(d), float(kappa), float(dhat),
                                _p(out[0:1], _f64p), _p(out[1:2], _f64p),
                                _p(out[2:3], _f64p))
    return tuple(out)


def inertia_local(xv, xt, c):
    xv, xt = _f64(xv), _f64(xt)
    return _local(lib().oracle_inertia_local, 1, _p(xv, _f64p), _p(xt, _f64p), float(c))


def face_local(x0, x1, x2, dm_inv, area):
    x0, x1, x2, dm = _f64(x0), _f64(x1), _f64(x2), _f64(dm_inv)
    return _local(lib().oracle_face_local, 3, _p(x0, _f64p), _p(x1, _f64p),
                  _p(x2, _f64p), _p(dm, _f64p), float(area))


def quad_local(x0, x1, x2, x3, kq):
    x0, x1, x2, x3 = _f64(x0), _f64(x1), _f64(x2), _f64(x3)
    return _local(lib().oracle_quad_local, 4, _p(x0, _f64p), _p(x1, _f64p), _p(x2, _f64p),
                  _p(x3, _f64p), float(kq))


def arap_local(x0, x1, x2, dm_inv, area):
    x0, x1, x2, dm = _f64(x0), _f64(x1), _f64(x2), _f64(dm_inv)
    return _local(lib().oracle_arap_local, 3, _p(x0, _f64p), _p(x1, _f64p),
                  _p(x2, _f64p), _p(dm, _f64p), float(area))


def face_grad_hyperdual(x0, x1, x2, dm_inv, area):
    x0, x1, x2, dm = _f64(x0), _f64(x1), _f64(x2), _f64(dm_inv)
    g = np.zeros(9)
    lib().oracle_face_grad_hyperdual(_p(x0, _f64p), _p(x1, _f64p), _p(x2, _f64p),
                                     _p(dm, _f64p), float(area), _p(g, _f64p))
    return g


def vf_local(p, t0, t1, t2, kappa, dhat):
    """Vertex-face barrier: (E, g (12,), H (12, 12)), local order p, t0, t1, t2."""
    p, t0, t1, t2 = _f64(p), _f64(t0), _f64(t1), _f64(t2)
    E = np.zeros(1)
    g = np.zeros(12)
    H = np.zeros((12, 12))
    lib().oracle_vf_local(_p(p, _f64p), _p(t0, _f64p), _p(t1, _f64p), _p(t2, _f64p),
                          float(kappa), float(dhat), _p(E, _f64p), _p(g, _f64p), _p(H, _f64p))
    return float(E[0]), g, H


def vf_distance_type(p, t0, t1, t2):
    p, t0, t1, t2 = _f64(p), _f64(t0), _f64(t1), _f64(t2)
    return int(lib().oracle_vf_distance_type(_p(p, _f64p), _p(t0, _f64p), _p(t1, _f64p),
                                             _p(t2, _f64p)))


def problem_from_mesh(mesh, springs=True, inertia=True, faces=False, pairs=None,
                      kappa=0.0, dhat=0.0, k=None, c=None, f32=False, vf=None, quads=None,
                      kq=0.0):
    """Build a Problem from a generated mesh bundle.  With f32=True every real
    input is rounded to fp32 first (the inputs an fp32 evaluation sees)."""
    r = (lambda a: np.asarray(a, dtype=np.float32).astype(np.float64)) if f32 else (lambda a: a)
    rs = (lambda a: float(np.float32(a))) if f32 else float
    kk = mesh.params.get("k", 0.0) if k is None else k
    cc = mesh.params.get("c", 0.0) if c is None else c
    return Problem(
        nv=mesh.nv, faces=mesh.faces,
        springs=mesh.springs if springs else None,
        rest_len=r(mesh.rest_len) if springs else None, k=rs(kk),
        x_tilde=r(mesh.X) if inertia else None, c=rs(cc),
        face_energy=faces, dm_inv=r(mesh.dm_inv) if faces else None,
        area=r(mesh.area) if faces else None,
        pairs=pairs, kappa=rs(kappa), dhat=rs(dhat), vf=vf, quads=quads, kq=rs(kq))
