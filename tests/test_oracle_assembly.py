"""Pins of the oracle's pattern, assembly, Hessian-vector product and pair
insertion: brute force on tiny grids (explicit selection matrices), closed-form
counts, finite differences, symmetry and the translation null space."""
import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from test_oracle_elements import fd_grad, fd_jac


def dense_from_bsr(row_ptr, col_idx, hvals, nv):
    D = np.zeros((3 * nv, 3 * nv))
    for a in range(nv):
        for k in range(row_ptr[a], row_ptr[a + 1]):
            b = col_idx[k]
            D[3 * a:3 * a + 3, 3 * b:3 * b + 3] = hvals[k]
    return D


def all_terms(mesh, pairs=None, dhat=None):
    return oracle.problem_from_mesh(mesh, springs=True, inertia=True, faces=True,
                                    pairs=pairs, kappa=100.0,
                                    dhat=dhat if dhat is not None else 0.5 * mesh.h)


# ---------------------------------------------------------------- pattern
@pytest.mark.parametrize("n,nnzb", [(3, 41), (10, 622), (100, 69_202)])
def test_pattern_counts(n, nnzb):
    m = inputs.cloth(n)
    c = inputs.grid_counts(n)
    rp, ci = oracle.pattern(oracle.problem_from_mesh(m))
    assert rp[-1] == nnzb == c["V"] + 2 * c["S"]
    # row length = 1 + valence (springs are the unique triangle edges)
    val = np.bincount(m.springs.reshape(-1), minlength=m.nv)
    assert np.array_equal(np.diff(rp), 1 + val)


@pytest.mark.parametrize("n", [3, 4, 7])
def test_pattern_brute_force(n):
    m = inputs.cloth(n)
    adj = np.eye(m.nv, dtype=bool)
    for t in m.faces:
        for i in t:
            for j in t:
                adj[i, j] = True
    rp, ci = oracle.pattern(oracle.problem_from_mesh(m))
    for a in range(m.nv):
        row = ci[rp[a]:rp[a + 1]]
        assert np.array_equal(row, np.nonzero(adj[a])[0])


def test_pattern_with_pairs_is_sorted_union():
    m = inputs.cloth(12)
    pairs, _ = inputs.contact_pairs(m, m.x, step=3, frac=0.05)
    base = oracle.problem_from_mesh(m)
    rp0, ci0 = oracle.pattern(base)
    rp, ci = oracle.pattern(base.with_pairs(pairs))
    # non-adjacent, pairwise-distinct pairs add exactly two blocks each
    assert rp[-1] == rp0[-1] + 2 * pairs.shape[0]
    for a in range(m.nv):
        s = set(ci0[rp0[a]:rp0[a + 1]].tolist())
        s |= {int(b) for (i, b) in pairs if i == a} | {int(i) for (i, b) in pairs if b == a}
        assert ci[rp[a]:rp[a + 1]].tolist() == sorted(s)


def test_pattern_duplicate_and_adjacent_pairs_add_nothing():
    m = inputs.cloth(6)
    base = oracle.problem_from_mesh(m)
    rp0, _ = oracle.pattern(base)
    # (0,1) is an edge; (0,7) is the +x+y diagonal; duplicates and reversed
    pairs = np.array([[0, 1], [1, 0], [0, 7], [0, 20], [20, 0], [0, 20]])
    rp, ci = oracle.pattern(base.with_pairs(pairs))
    assert rp[-1] == rp0[-1] + 2
    assert 20 in ci[rp[0]:rp[1]] and 0 in ci[rp[20]:rp[21]]


def test_pattern_isolated_and_empty():
    p = oracle.Problem(nv=4, faces=np.array([[0, 1, 2]]))
    rp, ci = oracle.pattern(p)
    assert rp.tolist() == [0, 3, 6, 9, 10] and ci[-1] == 3
    rp, ci = oracle.pattern(oracle.Problem(nv=0))
    assert rp.tolist() == [0] and ci.size == 0


def test_pattern_rejects_bad_index():
    with pytest.raises(ValueError):
        oracle.pattern(oracle.Problem(nv=3, faces=np.array([[0, 1, 3]])))


# ---------------------------------------------------------------- assembly
def test_dense_assembly_brute_force_3x3():
    """H = sum_j S_j^T H_j S_j with explicit selection matrices equals the
    dense expansion of the oracle's block CSR, bit for bit."""
    m = inputs.cloth(3)
    pairs = np.array([[0, 8], [2, 6]])
    x = m.x.copy()
    x[8] = x[0] + np.array([0.1, 0.05, 0.02])
    x[6] = x[2] + np.array([-0.05, 0.1, 0.0])
    dhat = 0.5 * m.h
    prob = all_terms(m, pairs, dhat)
    rp, ci = oracle.pattern(prob)
    E, g, Hv = oracle.evaluate(prob, rp, ci, x)
    N = 3 * m.nv
    Hd = np.zeros((N, N))
    gd = np.zeros(N)
    Ed = 0.0

    def S_of(verts):
        S = np.zeros((3 * len(verts), N))
        for i, v in enumerate(verts):
            S[3 * i:3 * i + 3, 3 * v:3 * v + 3] = np.eye(3)
        return S

    def add(verts, e, gl, Hl):
        nonlocal Ed, gd, Hd
        S = S_of(verts)
        Ed += e
        gd = gd + S.T @ gl
        Hd = Hd + S.T @ Hl @ S

    for s, (a, b) in enumerate(m.springs):
        add([a, b], *oracle.spring_local(x[a], x[b], m.rest_len[s], prob.k))
    for v in range(m.nv):
        add([v], *oracle.inertia_local(x[v], m.X[v], prob.c))
    for f, t in enumerate(m.faces):
        add(list(t), *oracle.face_local(x[t[0]], x[t[1]], x[t[2]], m.dm_inv[f], m.area[f]))
    for a, b in pairs:
        add([a, b], *oracle.barrier_local(x[a], x[b], 100.0, dhat))
    assert E == Ed
    assert np.array_equal(g.reshape(-1), gd)
    assert np.array_equal(dense_from_bsr(rp, ci, Hv, m.nv), Hd)
    # the pairs are active (inside the barrier support)
    assert np.any(Hd[0:3, 24:27] != 0)


@pytest.mark.parametrize("n", [3, 4])
def test_full_finite_differences(n):
    m = inputs.cloth(n)
    pairs = np.array([[0, m.nv - 1]])
    x = m.x.copy()
    x[-1] = x[0] + np.array([0.2, 0.1, -0.1]) * m.h
    prob = all_terms(m, pairs)
    rp, ci = oracle.pattern(prob)
    Ef = lambda z: oracle.evaluate(prob, rp, ci, z.reshape(-1, 3))[0]
    gf = lambda z: oracle.evaluate(prob, rp, ci, z.reshape(-1, 3))[1].reshape(-1)
    E, g, Hv = oracle.evaluate(prob, rp, ci, x)
    z = x.reshape(-1)
    assert np.allclose(g.reshape(-1), fd_grad(Ef, z, 1e-7), rtol=1e-6, atol=1e-5)
    Hd = dense_from_bsr(rp, ci, Hv, m.nv)
    Hfd = fd_jac(gf, z, 1e-7)
    assert np.allclose(Hd, Hfd, rtol=1e-5, atol=1e-3)


def test_symmetry_exact():
    m = inputs.cloth(8)
    prob = all_terms(m)
    rp, ci = oracle.pattern(prob)
    _, _, Hv = oracle.evaluate(prob, rp, ci, m.x)
    Hd = dense_from_bsr(rp, ci, Hv, m.nv)
    assert np.array_equal(Hd, Hd.T)


@pytest.mark.parametrize("kind", ["springs", "faces", "pairs"])
def test_translation_null_space(kind):
    m = inputs.cloth(9)
    pairs = None
    x = m.x.copy()
    if kind == "pairs":
        pairs, x = inputs.contact_pairs(m, m.x, step=0, frac=0.05)
    prob = oracle.problem_from_mesh(m, springs=kind == "springs", inertia=False,
                                    faces=kind == "faces", pairs=pairs,
                                    kappa=100.0, dhat=0.5 * m.h)
    rp, ci = oracle.pattern(prob)
    E, g, Hv = oracle.evaluate(prob, rp, ci, x)
    scale = np.abs(Hv).max()
    assert scale > 0
    assert np.allclose(g.sum(axis=0), 0, atol=1e-12 * np.abs(g).sum())
    for a in range(m.nv):
        assert np.allclose(Hv[rp[a]:rp[a + 1]].sum(axis=0), 0, atol=1e-12 * scale)


def test_inertia_gradient_sum():
    m = inputs.cloth(7)
    prob = oracle.problem_from_mesh(m)
    rp, ci = oracle.pattern(prob)
    _, g, _ = oracle.evaluate(prob, rp, ci, m.x)
    assert np.allclose(g.sum(axis=0), prob.c * (m.x - m.X).sum(axis=0), rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("s", [0.8, 1.1])
def test_total_energy_closed_form_under_scaling(s):
    n = 5
    m = inputs.cloth(n)
    prob = all_terms(m)
    rp, ci = oracle.pattern(prob)
    x = s * m.X
    E, _, _ = oracle.evaluate(prob, rp, ci, x)
    h = m.h
    axis_edges, diag_edges = 2 * n * (n - 1), (n - 1) ** 2
    sumL2 = axis_edges * h * h + diag_edges * 2 * h * h
    Espring = 0.5 * prob.k * (s - 1) ** 2 * sumL2
    Einertia = 0.5 * prob.c * (s - 1) ** 2 * np.sum(m.X ** 2)
    nf = 2 * (n - 1) ** 2
    Eface = nf * (0.5 * h * h) * (2 * s * s + 2 / (s * s))
    assert E == pytest.approx(Espring + Einertia + Eface, rel=1e-12)


def test_missing_block_is_an_error():
    m = inputs.cloth(5)
    prob = oracle.problem_from_mesh(m)
    rp, ci = oracle.pattern(prob)
    with pytest.raises(ValueError):
        oracle.evaluate(prob.with_pairs(np.array([[0, 24]]), 100.0, 0.5), rp, ci, m.x)


# ---------------------------------------------------------------- HVP
@pytest.mark.parametrize("n", [4, 12])
def test_hvp_matches_fd_and_dense(n):
    m = inputs.face_grid(n)
    prob = oracle.problem_from_mesh(m, springs=False, inertia=False, faces=True)
    rp, ci = oracle.pattern(prob)
    v = inputs.hvp_direction(m.nv)
    y = oracle.hvp(prob, rp, ci, m.x, v)
    _, _, Hv = oracle.evaluate(prob, rp, ci, m.x)
    Hd = dense_from_bsr(rp, ci, Hv, m.nv)
    assert np.allclose(y.reshape(-1), Hd @ v.reshape(-1), rtol=1e-12, atol=1e-12 * np.abs(Hd).max())
    d = 1e-6
    gp = oracle.evaluate(prob, rp, ci, m.x + d * v)[1]
    gm = oracle.evaluate(prob, rp, ci, m.x - d * v)[1]
    assert np.allclose(y, (gp - gm) / (2 * d), rtol=1e-5, atol=1e-6 * np.abs(y).max())


def test_bsr_spmv_matches_dense():
    m = inputs.cloth(6)
    prob = all_terms(m)
    rp, ci = oracle.pattern(prob)
    _, _, Hv = oracle.evaluate(prob, rp, ci, m.x)
    v = np.random.default_rng(1).normal(size=(m.nv, 3))
    y = oracle.bsr_spmv(rp, ci, Hv, v)
    assert np.allclose(y.reshape(-1), dense_from_bsr(rp, ci, Hv, m.nv) @ v.reshape(-1),
                       rtol=1e-13, atol=1e-10)
