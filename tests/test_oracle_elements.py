"""Pins of the oracle's element routines against values fixed by the
mathematics: hand-computed values, closed forms, invariances and central
finite differences.  (The page prints no worked values for these terms.)"""
import math

import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

RNG = np.random.default_rng(0)


def fd_grad(f, x, h=1e-6):
    x = np.array(x, dtype=np.float64)
    g = np.zeros_like(x)
    for i in range(x.size):
        xp, xm = x.copy(), x.copy()
        xp.flat[i] += h
        xm.flat[i] -= h
        g.flat[i] = (f(xp) - f(xm)) / (2 * h)
    return g


def fd_jac(fg, x, h=1e-6):
    x = np.array(x, dtype=np.float64)
    cols = []
    for i in range(x.size):
        xp, xm = x.copy(), x.copy()
        xp.flat[i] += h
        xm.flat[i] -= h
        cols.append((fg(xp) - fg(xm)) / (2 * h))
    return np.stack(cols, axis=1)


# ---------------------------------------------------------------- springs
def test_spring_hand_values():
    # |xa - xb| = 5, L = 2, k = 2: E = 0.5*2*3^2 = 9, force 6 along n.
    E, g, H = oracle.spring_local([0, 0, 0], [3, 4, 0], 2.0, 2.0)
    assert E == pytest.approx(9.0, rel=1e-15)
    assert np.allclose(g, [-3.6, -4.8, 0, 3.6, 4.8, 0], rtol=1e-14)
    # along n the stiffness is k = 2; across n it is tension/length = 6/5
    K = np.array([[1.488, 0.384, 0.0], [0.384, 1.712, 0.0], [0.0, 0.0, 1.2]])
    assert np.allclose(H[:3, :3], K, rtol=1e-13)
    assert np.allclose(H[:3, 3:], -K, rtol=1e-13)
    assert np.allclose(H[3:, 3:], K, rtol=1e-13)


def test_spring_at_rest_length():
    d = np.array([0.3, -0.2, 0.5])
    L = np.linalg.norm(d)
    E, g, H = oracle.spring_local(d, [0, 0, 0], L, 7.0)
    n = d / L
    assert E == 0.0 or abs(E) < 1e-30
    assert np.allclose(g, 0.0, atol=1e-14)
    K = 7.0 * np.outer(n, n)
    assert np.allclose(H[:3, :3], K, atol=1e-13)
    assert np.allclose(H[:3, 3:], -K, atol=1e-13)


@pytest.mark.parametrize("trial", range(5))
def test_spring_finite_differences(trial):
    x = RNG.normal(size=6)
    L, k = 0.7, 13.0
    f = lambda z: oracle.spring_local(z[:3], z[3:], L, k)[0]
    gf = lambda z: oracle.spring_local(z[:3], z[3:], L, k)[1]
    E, g, H = oracle.spring_local(x[:3], x[3:], L, k)
    assert np.allclose(g, fd_grad(f, x), rtol=1e-7, atol=1e-8)
    assert np.allclose(H, fd_jac(gf, x), rtol=1e-6, atol=1e-6)
    assert np.allclose(H, H.T, atol=0)
    # translation invariance: g_a + g_b = 0 and H annihilates translations
    assert np.allclose(g[:3] + g[3:], 0, atol=1e-12)
    assert np.allclose(H[:, :3] + H[:, 3:], 0, atol=1e-11)


# ---------------------------------------------------------------- inertia
def test_inertia_hand_values():
    E, g, H = oracle.inertia_local([1, 2, 3], [0, 0, 1], 4.0)
    assert E == 18.0
    assert np.array_equal(g, [4.0, 8.0, 8.0])
    assert np.array_equal(H, 4.0 * np.eye(3))


# ---------------------------------------------------------------- barrier
def test_barrier_vanishes_at_support():
    b, db, ddb = oracle.barrier_scalar(0.5, 100.0, 0.5)
    assert (b, db, ddb) == (0.0, 0.0, 0.0)
    # C^2 from the inside: all three tend to 0 as d -> dhat
    b, db, ddb = oracle.barrier_scalar(0.5 * (1 - 1e-7), 100.0, 0.5)
    assert abs(b) < 1e-15 and abs(db) < 1e-11 and abs(ddb) < 1e-4
    assert oracle.barrier_scalar(0.9, 100.0, 0.5) == (0.0, 0.0, 0.0)


def test_barrier_hand_value():
    # d = dhat/2: b = kappa (dhat/2)^2 ln 2
    b, _, _ = oracle.barrier_scalar(0.25, 100.0, 0.5)
    assert b == pytest.approx(100.0 * 0.0625 * math.log(2.0), rel=1e-14)


@pytest.mark.parametrize("d", [0.06, 0.2, 0.33, 0.49])
def test_barrier_scalar_fd(d):
    kappa, dhat, h = 100.0, 0.5, 1e-7
    b, db, ddb = oracle.barrier_scalar(d, kappa, dhat)
    bp = oracle.barrier_scalar(d + h, kappa, dhat)
    bm = oracle.barrier_scalar(d - h, kappa, dhat)
    assert db == pytest.approx((bp[0] - bm[0]) / (2 * h), rel=1e-6)
    assert ddb == pytest.approx((bp[1] - bm[1]) / (2 * h), rel=1e-6)
    assert b > 0 and db < 0  # repulsive


@pytest.mark.parametrize("trial", range(4))
def test_barrier_local_fd(trial):
    dhat = 0.5
    u = RNG.normal(size=3)
    u /= np.linalg.norm(u)
    xa = RNG.normal(size=3)
    xb = xa + (0.1 + 0.8 * RNG.random()) * dhat * u
    x = np.concatenate([xa, xb])
    f = lambda z: oracle.barrier_local(z[:3], z[3:], 100.0, dhat)[0]
    gf = lambda z: oracle.barrier_local(z[:3], z[3:], 100.0, dhat)[1]
    E, g, H = oracle.barrier_local(xa, xb, 100.0, dhat)
    assert np.allclose(g, fd_grad(f, x), rtol=1e-6, atol=1e-8)
    assert np.allclose(H, fd_jac(gf, x), rtol=1e-5, atol=1e-5)
    assert np.allclose(g[:3] + g[3:], 0, atol=1e-12)


def test_barrier_outside_support_is_zero():
    E, g, H = oracle.barrier_local([0, 0, 0], [0.6, 0, 0], 100.0, 0.5)
    assert E == 0.0 and not g.any() and not H.any()


# ---------------------------------------------------------------- faces
def _rest_triangle():
    m = inputs.make_grid(4)
    f = 5
    t = m.faces[f]
    return m.X[t[0]], m.X[t[1]], m.X[t[2]], m.dm_inv[f], m.area[f]


def test_face_rest_energy_and_zero_gradient():
    X0, X1, X2, Mi, A = _rest_triangle()
    E, g, H = oracle.face_local(X0, X1, X2, Mi, A)
    assert E == pytest.approx(4.0 * A, rel=1e-14)  # tr C = 2, det C = 1
    assert np.allclose(g, 0.0, atol=1e-12)


def test_face_rigid_motion_invariance():
    X0, X1, X2, Mi, A = _rest_triangle()
    q, _ = np.linalg.qr(RNG.normal(size=(3, 3)))
    t = RNG.normal(size=3)
    xs = [q @ X + t for X in (X0, X1, X2)]
    E, g, H = oracle.face_local(*xs, Mi, A)
    assert E == pytest.approx(4.0 * A, rel=1e-12)
    assert np.allclose(g, 0.0, atol=1e-10)


@pytest.mark.parametrize("s", [0.5, 0.9, 1.3, 2.0])
def test_face_uniform_scaling(s):
    X0, X1, X2, Mi, A = _rest_triangle()
    E, g, H = oracle.face_local(s * X0, s * X1, s * X2, Mi, A)
    assert E == pytest.approx(A * (2 * s * s + 2 / (s * s)), rel=1e-13)
    dEds = float(g @ np.concatenate([X0, X1, X2]))
    assert dEds == pytest.approx(A * (4 * s - 4 / s ** 3), rel=1e-11, abs=1e-13)


@pytest.mark.parametrize("s1,s2", [(1.5, 0.8), (0.7, 1.1)])
def test_face_anisotropic_stretch(s1, s2):
    X0, X1, X2, Mi, A = _rest_triangle()
    S = np.diag([s1, s2, 1.0])
    E, _, _ = oracle.face_local(S @ X0, S @ X1, S @ X2, Mi, A)
    expect = A * (s1 ** 2 + s2 ** 2 + 1 / s1 ** 2 + 1 / s2 ** 2)
    assert E == pytest.approx(expect, rel=1e-13)


@pytest.mark.parametrize("trial", range(5))
def test_face_finite_differences_and_structure(trial):
    X0, X1, X2, Mi, A = _rest_triangle()
    x = np.concatenate([X0, X1, X2]) + 0.05 * RNG.normal(size=9)
    f = lambda z: oracle.face_local(z[:3], z[3:6], z[6:], Mi, A)[0]
    gf = lambda z: oracle.face_local(z[:3], z[3:6], z[6:], Mi, A)[1]
    E, g, H = oracle.face_local(x[:3], x[3:6], x[6:], Mi, A)
    # closed-form gradient vs FD of the energy
    assert np.allclose(g, fd_grad(f, x, 1e-7), rtol=1e-6, atol=1e-7)
    # hyper-dual Hessian vs FD of the closed-form gradient
    assert np.allclose(H, fd_jac(gf, x, 1e-7), rtol=1e-5, atol=1e-4)
    # closed-form gradient vs the hyper-dual gradient (two algorithms)
    gh = oracle.face_grad_hyperdual(x[:3], x[3:6], x[6:], Mi, A)
    assert np.allclose(g, gh, rtol=1e-12, atol=1e-12)
    assert np.array_equal(H, H.T)
    # translation: sum of vertex gradients and of H column blocks vanish
    assert np.allclose(g[:3] + g[3:6] + g[6:], 0, atol=1e-10)
    T = H[:, 0:3] + H[:, 3:6] + H[:, 6:9]
    assert np.allclose(T, 0, atol=1e-8 * np.abs(H).max())
    # rotation: g is orthogonal to every infinitesimal rotation w x x_i
    P = x.reshape(3, 3)
    for w in np.eye(3):
        rot = np.cross(w, P).reshape(-1)
        assert abs(g @ rot) < 1e-10 * (1 + np.abs(g).max())


def test_face_hessian_rotation_nullspace_at_rest():
    X0, X1, X2, Mi, A = _rest_triangle()
    E, g, H = oracle.face_local(X0, X1, X2, Mi, A)
    P = np.stack([X0, X1, X2])
    for w in np.eye(3):
        rot = np.cross(w, P).reshape(-1)
        assert np.allclose(H @ rot, 0, atol=1e-9 * np.abs(H).max())
