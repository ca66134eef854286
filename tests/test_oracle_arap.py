"""Pins of the oracle's as-rigid-as-possible face term
E = A sum_i (sigma_i - 1)^2 (sigma_i the singular values of
F = [x1 - x0, x2 - x0] Dm^-1): the definition through numpy's SVD, zero
energy and gradient under rigid motion, the closed form under uniform
scaling, central finite differences of E -> g and g -> H, symmetry, the
translation and (at rest) rotation null spaces, and the assembly of the
per-face terms."""
import math

import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from test_oracle_elements import fd_grad, fd_jac

# rest triangle in its plane (z = 0) and its constants
REST = np.array([[0.0, 0.0, 0.0], [1.3, 0.1, 0.0], [0.4, 0.9, 0.0]])
DM = np.array([[REST[1, 0] - REST[0, 0], REST[2, 0] - REST[0, 0]],
               [REST[1, 1] - REST[0, 1], REST[2, 1] - REST[0, 1]]])
DM_INV = np.linalg.inv(DM).reshape(-1)
AREA = 0.5 * abs(np.linalg.det(DM))


def local(x):
    x = np.asarray(x, dtype=np.float64).reshape(3, 3)
    return oracle.arap_local(x[0], x[1], x[2], DM_INV, AREA)


def energy_by_svd(x):
    x = np.asarray(x, dtype=np.float64).reshape(3, 3)
    Ds = np.stack([x[1] - x[0], x[2] - x[0]], axis=1)          # 3 x 2
    F = Ds @ DM_INV.reshape(2, 2)
    s = np.linalg.svd(F, compute_uv=False)
    return AREA * float(np.sum((s - 1.0) ** 2))


def rotation(a, b, c):
    ca, sa, cb, sb = math.cos(a), math.sin(a), math.cos(b), math.sin(b)
    cc, sc = math.cos(c), math.sin(c)
    Rz = np.array([[ca, -sa, 0], [sa, ca, 0], [0, 0, 1]])
    Ry = np.array([[cb, 0, sb], [0, 1, 0], [-sb, 0, cb]])
    Rx = np.array([[1, 0, 0], [0, cc, -sc], [0, sc, cc]])
    return Rz @ Ry @ Rx


def deformed(seed, amp=0.3):
    rng = np.random.default_rng(seed)
    return REST + amp * rng.normal(size=(3, 3))


@pytest.mark.parametrize("seed", range(6))
def test_energy_is_the_svd_definition(seed):
    x = deformed(seed)
    E, _, _ = local(x)
    assert E == pytest.approx(energy_by_svd(x), rel=1e-12, abs=1e-14)


def test_rigid_motion_has_zero_energy_and_gradient():
    R = rotation(0.3, -1.1, 2.0)
    x = REST @ R.T + np.array([0.5, -2.0, 3.0])
    E, g, _ = local(x)
    assert abs(E) < 1e-14 and np.abs(g).max() < 1e-12


@pytest.mark.parametrize("s", [0.5, 1.0, 1.7, 3.0])
def test_uniform_scaling_closed_form(s):
    E, _, _ = local(s * REST @ rotation(0.2, 0.4, -0.3).T)
    assert E == pytest.approx(2.0 * AREA * (s - 1.0) ** 2, rel=1e-12, abs=1e-14)


def test_anisotropic_stretch_closed_form():
    # F = diag(a, b) in the rest frame: sigma = (a, b)
    a, b = 1.6, 0.7
    x = REST.copy()
    x[:, 0] *= a
    x[:, 1] *= b
    E, _, _ = local(x)
    assert E == pytest.approx(AREA * ((a - 1) ** 2 + (b - 1) ** 2), rel=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_finite_differences_symmetry_translation(seed):
    x0 = deformed(10 + seed).reshape(-1)
    E, g, H = local(x0)
    gf = fd_grad(lambda y: local(y)[0], x0)
    Hf = fd_jac(lambda y: local(y)[1], x0)
    np.testing.assert_allclose(g, gf, rtol=0, atol=1e-6 * max(1.0, np.abs(g).max()))
    np.testing.assert_allclose(H, Hf, rtol=0, atol=1e-5 * max(1.0, np.abs(H).max()))
    assert np.array_equal(H, H.T)
    np.testing.assert_allclose(g.reshape(3, 3).sum(axis=0), 0.0, atol=1e-12 * max(1, abs(g).max()))
    np.testing.assert_allclose(H.reshape(9, 3, 3).sum(axis=1), 0.0, atol=1e-11 * max(1, abs(H).max()))


def test_rest_hessian_psd_with_rotation_null_space():
    _, _, H = local(REST)
    w = np.linalg.eigvalsh(H)
    assert w.min() > -1e-10 * w.max()
    for axis in np.eye(3):
        d = np.cross(axis, REST).reshape(-1)      # infinitesimal rotation
        assert np.abs(H @ d).max() < 1e-10 * np.abs(H).max()


def test_assembly_is_the_sum_of_face_terms():
    m = inputs.cloth(6)
    prob = oracle.Problem(nv=m.nv, faces=m.faces, face_energy="arap", dm_inv=m.dm_inv,
                          area=m.area)
    rp, ci = oracle.pattern(prob)
    E, g, H = oracle.evaluate(prob, rp, ci, m.x)
    Es, gs = 0.0, np.zeros((m.nv, 3))
    Hd = np.zeros((3 * m.nv, 3 * m.nv))
    for f, t in enumerate(m.faces):
        e, gl, Hl = oracle.arap_local(m.x[t[0]], m.x[t[1]], m.x[t[2]], m.dm_inv[f], m.area[f])
        Es += e
        for i, a in enumerate(t):
            gs[a] += gl[3 * i:3 * i + 3]
            for j, b in enumerate(t):
                Hd[3 * a:3 * a + 3, 3 * b:3 * b + 3] += Hl[3 * i:3 * i + 3, 3 * j:3 * j + 3]
    assert E == pytest.approx(Es, rel=1e-12) and Es > 0.0
    np.testing.assert_allclose(g, gs, rtol=0, atol=1e-12 * np.abs(gs).max())
    dense = np.zeros_like(Hd)
    for a in range(m.nv):
        for k in range(rp[a], rp[a + 1]):
            b = ci[k]
            dense[3 * a:3 * a + 3, 3 * b:3 * b + 3] = H[k]
    np.testing.assert_allclose(dense, Hd, rtol=0, atol=1e-12 * np.abs(Hd).max())
