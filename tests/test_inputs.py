"""Input generator: grid counts, seeds and contact-pair construction."""
import math

import numpy as np
import pytest

from sparse_autodiff_mesh_amd import inputs


@pytest.mark.parametrize("n,V,F,S", [(3, 9, 8, 16), (10, 100, 162, 261),
                                     (100, 10_000, 19_602, 29_601)])
def test_grid_counts(n, V, F, S):
    m = inputs.make_grid(n)
    assert m.nv == V and m.faces.shape == (F, 3) and m.springs.shape == (S, 2)
    assert inputs.grid_counts(n) == {"V": V, "F": F, "S": S}
    # Euler characteristic of a disc: V - E + F = 1.
    assert V - S + F == 1


def test_headline_grid_counts():
    c = inputs.grid_counts(1000)
    assert c["V"] == 1_000_000 and c["S"] == 2_996_001 and c["F"] == 1_996_002


def test_grid_geometry():
    m = inputs.make_grid(10)
    assert math.isclose(m.h, 1.0 / 9.0)
    # rest lengths are h (axis edges) or sqrt(2) h (diagonals)
    L = np.unique(np.round(m.rest_len / m.h, 12))
    assert np.allclose(L, [1.0, math.sqrt(2.0)])
    assert np.all(m.springs[:, 0] < m.springs[:, 1])
    key = m.springs[:, 0].astype(np.int64) * m.nv + m.springs[:, 1]
    assert np.all(np.diff(key) > 0)
    # faces are counter-clockwise in the xy plane and have area h^2/2
    assert np.allclose(m.area, 0.5 * m.h ** 2)
    X = m.X
    e1 = X[m.faces[:, 1]] - X[m.faces[:, 0]]
    e2 = X[m.faces[:, 2]] - X[m.faces[:, 0]]
    assert np.all(e1[:, 0] * e2[:, 1] - e1[:, 1] * e2[:, 0] > 0)
    # perturbation bounded by amp * h per axis
    assert np.max(np.abs(m.x - m.X)) <= 0.1 * m.h + 1e-15


def test_dm_inv_is_inverse():
    m = inputs.make_grid(5)
    X = m.X
    for f in range(m.faces.shape[0]):
        t = m.faces[f]
        Dm = np.stack([X[t[1], :2] - X[t[0], :2], X[t[2], :2] - X[t[0], :2]], axis=1)
        assert np.allclose(Dm @ m.dm_inv[f].reshape(2, 2), np.eye(2), atol=1e-12)


def test_splitmix_scalar_matches_block():
    s = inputs.SplitMix64(12345)
    seq = [s.next_u64() for _ in range(20)]
    blk = inputs.splitmix64_block(12345, 20)
    assert seq == [int(v) for v in blk]
    # uniform draws lie in [0, 1)
    u = inputs.uniform_block(7, 10000)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.02


def test_seeded_reproducible():
    a = inputs.make_grid(20, seed=3).x
    b = inputs.make_grid(20, seed=3).x
    c = inputs.make_grid(20, seed=4).x
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_hvp_direction_unit():
    v = inputs.hvp_direction(100)
    assert v.shape == (100, 3)
    assert math.isclose(np.linalg.norm(v), 1.0, rel_tol=1e-14)


def test_contact_pairs():
    m = inputs.cloth(30)
    dhat = 0.5 * m.h
    pairs, xn = inputs.contact_pairs(m, m.x, step=0)
    P = pairs.shape[0]
    assert P == round(0.02 * m.nv)
    flat = pairs.reshape(-1)
    assert np.unique(flat).size == 2 * P          # all 2P vertices distinct
    for a, b in pairs:
        assert not inputs.grid_adjacent(m.n, int(a), int(b))
    d = np.linalg.norm(xn[pairs[:, 0]] - xn[pairs[:, 1]], axis=1)
    assert np.all(d > 0.1 * dhat * (1 - 1e-12)) and np.all(d < dhat)
    # only the partners moved
    moved = np.any(xn != m.x, axis=1)
    assert set(np.nonzero(moved)[0]) <= set(pairs[:, 1].tolist())
    p2, x2 = inputs.contact_pairs(m, m.x, step=0)
    assert np.array_equal(p2, pairs) and np.array_equal(x2, xn)
    p3, _ = inputs.contact_pairs(m, m.x, step=1)
    assert not np.array_equal(p3, pairs)
