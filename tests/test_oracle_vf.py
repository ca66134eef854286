"""Pins of the oracle's vertex-face contact element (point-triangle distance
barrier) and its assembly: closed-form distances in every closest-point
region, the barrier's own scalar form, central finite differences of E -> g
and g -> H, the translation null space, rotation invariance, continuity
across a region boundary, zero beyond the support, and the pattern blocks
the contacts add (brute force)."""
import math

import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from test_oracle_elements import fd_grad, fd_jac

T0, T1, T2 = np.array([0.0, 0.0, 0.0]), np.array([1.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0])
KAPPA, DHAT = 2.0, 1.0

# (point, region, distance) on the triangle (0,0,0), (1,0,0), (0,1,0)
CASES = [
    ((0.25, 0.25, 0.3), 6, 0.3),
    ((0.2, 0.3, -0.45), 6, 0.45),
    ((0.5, -0.2, 0.1), 3, math.hypot(0.2, 0.1)),
    ((0.7, 0.7, 0.1), 4, math.hypot(0.4 / math.sqrt(2.0), 0.1)),
    ((-0.3, 0.4, 0.2), 5, math.hypot(0.3, 0.2)),
    ((-0.3, -0.4, 0.2), 0, math.sqrt(0.09 + 0.16 + 0.04)),
    ((1.5, -0.3, 0.0), 1, math.hypot(0.5, 0.3)),
    ((-0.2, 1.4, 0.3), 2, math.sqrt(0.04 + 0.16 + 0.09)),
]


def local(p, t=(T0, T1, T2)):
    return oracle.vf_local(p, t[0], t[1], t[2], KAPPA, DHAT)


@pytest.mark.parametrize("p,region,d", CASES)
def test_distance_region_and_value(p, region, d):
    p = np.array(p)
    assert oracle.vf_distance_type(p, T0, T1, T2) == region
    E, g, H = local(p)
    b, _, _ = oracle.barrier_scalar(d, KAPPA, DHAT)
    assert E == pytest.approx(b, rel=1e-12)


@pytest.mark.parametrize("p,region,d", CASES)
def test_finite_differences(p, region, d):
    x0 = np.concatenate([np.array(p), T0, T1, T2])

    def energy(x):
        return local(x[:3], (x[3:6], x[6:9], x[9:]))[0]

    def grad(x):
        return local(x[:3], (x[3:6], x[6:9], x[9:]))[1]

    E, g, H = local(x0[:3], (x0[3:6], x0[6:9], x0[9:]))
    np.testing.assert_allclose(g, fd_grad(energy, x0), rtol=0, atol=1e-6 * max(1.0, np.abs(g).max()))
    np.testing.assert_allclose(H, fd_jac(grad, x0), rtol=0, atol=1e-5 * max(1.0, np.abs(H).max()))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("p,region,d", CASES)
def test_translation_null_space_and_rotation(p, region, d):
    p = np.array(p)
    E, g, H = local(p)
    np.testing.assert_allclose(g.reshape(4, 3).sum(axis=0), 0.0, atol=1e-12 * max(1, abs(g).max()))
    np.testing.assert_allclose(H.reshape(12, 4, 3).sum(axis=1), 0.0, atol=1e-11 * max(1, abs(H).max()))
    c, s = math.cos(0.7), math.sin(0.7)
    R = np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]]) @ \
        np.array([[1.0, 0.0, 0.0], [0.0, c, s], [0.0, -s, c]])
    Er, gr, Hr = oracle.vf_local(R @ p, R @ T0, R @ T1, R @ T2, KAPPA, DHAT)
    assert Er == pytest.approx(E, rel=1e-12)
    Rb = np.kron(np.eye(4), R)
    np.testing.assert_allclose(gr, Rb @ g, atol=1e-12 * max(1, abs(g).max()))
    np.testing.assert_allclose(Hr, Rb @ H @ Rb.T, atol=1e-10 * max(1, abs(H).max()))


def test_continuous_across_the_face_edge_boundary():
    # just inside the face region over edge (t0,t1) and just outside it
    eps = 1e-7
    pin = np.array([0.4, eps, 0.3])
    pout = np.array([0.4, -eps, 0.3])
    assert oracle.vf_distance_type(pin, T0, T1, T2) == 6
    assert oracle.vf_distance_type(pout, T0, T1, T2) == 3
    Ei, gi, _ = local(pin)
    Eo, go, _ = local(pout)
    assert Ei == pytest.approx(Eo, rel=1e-6)
    np.testing.assert_allclose(gi, go, rtol=0, atol=1e-5 * abs(gi).max())


def test_zero_beyond_the_support():
    E, g, H = local(np.array([0.2, 0.2, 1.5]))
    assert E == 0.0 and not g.any() and not H.any()


def test_pattern_blocks_and_assembly():
    # VF contacts add the (v, t_i) and (t_i, v) blocks; the assembled g of a
    # contact-only energy is the sum of the element gradients
    m = inputs.cloth(8)
    vf, x = inputs.vf_contacts(m, m.x, 3, frac=0.05)
    prob = oracle.Problem(nv=m.nv, faces=m.faces, springs=m.springs, rest_len=m.rest_len,
                          k=0.0, vf=vf, kappa=KAPPA, dhat=0.5 * m.h)
    rp, ci = oracle.pattern(prob)
    want = {(a, a) for a in range(m.nv)}
    for t in m.faces:
        want |= {(int(a), int(b)) for a in t for b in t}
    for a, b in m.springs:
        want |= {(int(a), int(b)), (int(b), int(a))}
    for v, f in vf:
        for t in m.faces[f]:
            want |= {(int(v), int(t)), (int(t), int(v))}
    got = {(a, int(ci[k])) for a in range(m.nv) for k in range(rp[a], rp[a + 1])}
    assert got == want
    E, g, H = oracle.evaluate(prob, rp, ci, x)
    gs = np.zeros_like(g)
    Es = 0.0
    for v, f in vf:
        ids = [int(v)] + [int(t) for t in m.faces[f]]
        e, gl, _ = oracle.vf_local(x[ids[0]], x[ids[1]], x[ids[2]], x[ids[3]], KAPPA, 0.5 * m.h)
        Es += e
        for i, a in enumerate(ids):
            gs[a] += gl[3 * i:3 * i + 3]
    assert E == pytest.approx(Es, rel=1e-12) and Es > 0.0
    np.testing.assert_allclose(g, gs, rtol=0, atol=1e-12 * np.abs(gs).max())


def test_generator_places_each_region_at_its_distance():
    m = inputs.cloth(30)
    dh = 0.5 * m.h
    vf, x = inputs.vf_contacts(m, m.x, 0, dhat=dh)
    for k, (v, f) in enumerate(vf):
        t = x[m.faces[f]]
        typ = oracle.vf_distance_type(x[v], t[0], t[1], t[2])
        assert (typ == 6) == (k % 3 == 0) and (3 <= typ <= 5) == (k % 3 == 1)
        assert (typ <= 2) == (k % 3 == 2)
        E, _, _ = oracle.vf_local(x[v], t[0], t[1], t[2], 1.0, dh)
        assert E > 0.0  # inside the support
