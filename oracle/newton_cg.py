"""Truncated Newton-CG direction, fp64, on the oracle's matrix-free HVP.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
it; the GPU library and its binding never import it.

Why: the page "Locality-Aware Automatic Differentiation on the GPU for
Mesh-Based Computations" (introduction and closing discussion) presents fast
gradients, Hessians and Hessian-vector products as what makes Newton-type
methods practical on large meshes, with the linear solve as the next
bottleneck.  The page does not fix a solver.  This module takes the standard
matrix-free choice for a possibly indefinite Hessian: the inner iteration of
line-search Newton-CG (Nocedal and Wright, Numerical Optimization, 2nd ed.,
section 7.1, Algorithm 7.1), i.e. conjugate gradients on H p = -g started at
p = 0 and stopped either when the residual is small enough or at the first
direction of non-positive curvature.

Steps, in that algorithm's notation (B = H(x), r = B z + g):
    z = 0, r = g, d = -r
    repeat:  if d.B d <= 0: return -g on the first step, else z
             alpha = r.r / d.B d;  z += alpha d;  r += alpha B d
             if |r| < eps: return z
             beta = r.r (new) / r.r (old);  d = -r + beta d
eps = eta |g| for a caller-given eta > 0, else the algorithm's own forcing
term min(0.5, sqrt|g|) |g|.  Added here: an iteration cap (returns the last
z) and an initial test |g| <= eps (returns p = 0).

Every vector operation and dot product is a plain numpy call on (nv, 3) fp64
arrays; B d is the oracle's fp64 Hessian-vector product.
"""
from __future__ import annotations

import math

import numpy as np

from . import hvp

CONVERGED, NEG_CURVATURE, MAX_ITERS = 0, 1, 2


def forcing_eps(gnorm: float, eta: float) -> float:
    """Residual threshold: eta |g| if eta > 0, else min(0.5, sqrt|g|) |g|."""
    if eta > 0.0:
        return eta * gnorm
    return min(0.5, math.sqrt(gnorm)) * gnorm


def newton_cg(prob, row_ptr, col_idx, x, g, max_iters: int, eta: float = 0.0,
              operator=None):
    """Returns (p (nv, 3), iterations, reason, |r| / |g|).

    `operator(d)` overrides B d (default: the oracle HVP at x).  iterations
    counts completed CG updates; reason is CONVERGED, NEG_CURVATURE or
    MAX_ITERS.
    """
    g = np.asarray(g, dtype=np.float64).reshape(-1, 3)
    if operator is None:
        def operator(d):
            return hvp(prob, row_ptr, col_idx, x, d)
    gnorm = float(np.sqrt(np.vdot(g, g)))
    eps = forcing_eps(gnorm, eta)
    z = np.zeros_like(g)
    r = g.copy()
    d = -r
    rr = float(np.vdot(r, r))
    if rr <= eps * eps:
        return z, 0, CONVERGED, (0.0 if gnorm == 0.0 else math.sqrt(rr) / gnorm)
    for j in range(max_iters):
        Bd = np.asarray(operator(d), dtype=np.float64).reshape(-1, 3)
        dBd = float(np.vdot(d, Bd))
        if dBd <= 0.0:
            p = -g if j == 0 else z
            return p.copy(), j, NEG_CURVATURE, math.sqrt(rr) / gnorm
        alpha = rr / dBd
        z = z + alpha * d
        r = r + alpha * Bd
        rr_new = float(np.vdot(r, r))
        if rr_new < eps * eps:
            return z, j + 1, CONVERGED, math.sqrt(rr_new) / gnorm
        beta = rr_new / rr
        d = -r + beta * d
        rr = rr_new
    return z, max_iters, MAX_ITERS, math.sqrt(rr) / gnorm
