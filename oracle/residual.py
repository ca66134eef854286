"""Vector objective of the mass-spring cloth: residuals, sparse Jacobian and
Gauss-Newton product, fp64.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
it; the GPU library and its binding never import it.

Source: page "Locality-Aware Automatic Differentiation on the GPU for
Mesh-Based Computations", section "Method": for a vector-valued objective
the local terms produce small dense Jacobians J_j that are assembled into
the global sparse Jacobian J = sum_j P_j^T J_j S_j (P_j places term j's
residual rows, S_j selects its variables); its closing discussion argues
that materialising J explicitly pays off at scale.

The residual vector is the least-squares form of the cloth energy
(F = 0.5 |R|^2 is exactly the spring + inertia energy):
    spring s = (a, b):   R_s = sqrt(k) (|x_a - x_b| - L_s)         rows 0 .. S-1
    vertex v, coord c:   R_(S + 3v + c) = sqrt(c_in) (x_v - xt_v)_c  rows S .. S+3V-1
Row s of J holds d R_s / d x_a = sqrt(k) n^T and d R_s / d x_b = -sqrt(k) n^T
(n = (x_a - x_b) / |x_a - x_b|), its six columns in ascending order; an
inertia row holds sqrt(c_in) in its single column.  The Gauss-Newton
product is y = J^T (J v).  All of it is written out from these definitions
with numpy and scipy.sparse (no blocking, no fusion).
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sps


def residual_jacobian(springs, rest_len, k, x, x_tilde=None, c=0.0):
    """Returns (R (m,), J as scipy CSR (m, 3V)) at positions x (V, 3)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, 3)
    V = x.shape[0]
    sp = np.asarray(springs, dtype=np.int64).reshape(-1, 2)
    S = sp.shape[0]
    L = np.asarray(rest_len, dtype=np.float64).reshape(-1)
    sk = np.sqrt(float(k))
    d = x[sp[:, 0]] - x[sp[:, 1]]
    ell = np.linalg.norm(d, axis=1)
    n = d / ell[:, None]
    R_s = sk * (ell - L)
    # J_j S_j for a spring: sqrt(k) [n^T, -n^T] on the DOFs of a and b
    rows = np.repeat(np.arange(S), 6)
    cols = np.concatenate([3 * sp[:, :1] + np.arange(3), 3 * sp[:, 1:] + np.arange(3)], axis=1)
    vals = np.concatenate([sk * n, -sk * n], axis=1)
    blocks = [(rows, cols.reshape(-1), vals.reshape(-1))]
    R = [R_s]
    if x_tilde is not None:
        xt = np.asarray(x_tilde, dtype=np.float64).reshape(-1, 3)
        sc = np.sqrt(float(c))
        R.append(sc * (x - xt).reshape(-1))
        i = np.arange(3 * V)
        blocks.append((S + i, i, np.full(3 * V, sc)))
    m = S + (3 * V if x_tilde is not None else 0)
    r = np.concatenate([b[0] for b in blocks])
    cc = np.concatenate([b[1] for b in blocks])
    v = np.concatenate([b[2] for b in blocks])
    J = sps.csr_matrix((v, (r, cc)), shape=(m, 3 * V))
    J.sort_indices()
    return np.concatenate(R), J


def gauss_newton_product(J, v):
    """y = J^T (J v) for v of shape (V, 3); returns (V, 3)."""
    v = np.asarray(v, dtype=np.float64).reshape(-1)
    return (J.T @ (J @ v)).reshape(-1, 3)
