"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
identical seeded inputs.  Patterns must match bit for bit; values within the
relative Frobenius tolerances in gpu_util.TOL."""
import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from gpu_util import TOL, dev, host_input, log_case, rel

pytestmark = pytest.mark.gpu


def run_eval(lad, mesh, dtype, det=False, lds=0, springs=True, inertia=True, faces=False,
             path="auto"):
    import torch
    L = lad.Lad(mesh.nv, dtype=dtype, deterministic=det, patch_lds_bytes=lds, path=path,
                **lad.mesh_terms(mesh, springs=springs, inertia=inertia, faces=faces))
    prob = oracle.problem_from_mesh(mesh, springs=springs, inertia=inertia, faces=faces,
                                    f32=(dtype == "f32"))
    x_h = host_input(mesh.x, dtype)
    E, g, H = L.eval(dev(x_h, dtype))
    rp, ci = L.pattern()
    torch.cuda.synchronize()
    return L, prob, x_h, (E.cpu().numpy()[0], g.cpu().numpy(), H.cpu().numpy(),
                          rp.cpu().numpy(), ci.cpu().numpy())


def check_against_oracle(prob, x_h, res, dtype):
    E, g, H, rp, ci = res
    orp, oci = oracle.pattern(prob)
    assert np.array_equal(rp, orp), "row_ptr differs"
    assert np.array_equal(ci, oci), "col_idx differs"
    Eo, go, Ho = oracle.evaluate(prob, orp, oci, x_h)
    tol = TOL[dtype]
    assert rel([E], [Eo]) <= tol, (E, Eo)
    assert rel(g, go) <= tol, rel(g, go)
    assert rel(H[: oci.size], Ho) <= tol, rel(H[: oci.size], Ho)
    return orp, oci


@pytest.mark.parametrize("n,dtype,det,lds", [
    (10, "f64", False, 0), (10, "f64", True, 0), (10, "f32", False, 0),
    (37, "f32", False, 6144), (37, "f64", True, 6144), (37, "f32", True, 6144),
    (100, "f32", False, 0), (100, "f64", False, 0), (100, "f32", True, 0),
])
def test_cloth_eval_patch(lad, n, dtype, det, lds):
    """The patch path: colour phases (det, also the default assembly) and,
    without det, the LDS-atomic assembly."""
    log_case(test="cloth_eval_patch", n=n, dtype=dtype, det=det, lds=lds)
    m = inputs.cloth(n)
    path = "patch" if det else "patch_lds_atomic"
    L, prob, x_h, res = run_eval(lad, m, dtype, det, lds, path=path)
    info = L.get_info()
    assert info["eval_path"] == (lad.LAD_PATH_PATCH if det else lad.LAD_PATH_PATCH_LDS_ATOMIC)
    if lds:
        assert info["npatches"] > 4  # several patches and ribbons
    check_against_oracle(prob, x_h, res, dtype)
    L.close()


@pytest.mark.parametrize("n,dtype", [(2, "f64"), (3, "f64"), (10, "f64"), (10, "f32"),
                                     (37, "f32"), (37, "f64"), (100, "f32"), (100, "f64"),
                                     (129, "f32")])
def test_cloth_eval_rows(lad, n, dtype):
    """Row-owner path (the default for cloth).  Sizes span one partial chunk
    (n = 2, 3), several chunks with a ragged tail, and chunks that straddle
    grid rows."""
    log_case(test="cloth_eval_rows", n=n, dtype=dtype)
    m = inputs.cloth(n)
    L, prob, x_h, res = run_eval(lad, m, dtype)
    info = L.get_info()
    assert info["eval_path"] == lad.LAD_PATH_ROWS
    assert 0.0 < info["pattern_ms"] < 1e4  # the pattern build was timed on the GPU
    check_against_oracle(prob, x_h, res, dtype)
    L.close()


def test_rows_bitwise_reproducible(lad):
    """The row path writes every value once in a fixed order: repeated
    evaluations are bitwise identical."""
    import torch
    log_case(test="rows_reproducible")
    m = inputs.cloth(64)
    L = lad.Lad(m.nv, dtype="f32", **lad.mesh_terms(m))
    x = dev(host_input(m.x, "f32"), "f32")
    E0, g0, H0 = L.eval(x)
    for _ in range(5):
        E, g, H = L.eval(x)
        torch.cuda.synchronize()
        assert torch.equal(E, E0) and torch.equal(g, g0) and torch.equal(H, H0)
    L.close()


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_rows_energy_over_changing_inputs(lad, dtype):
    """Consecutive calls on different positions, with a call that skips the
    energy in between, each give the oracle's energy (no partial energy of
    an earlier call is summed), and no device error is latched."""
    import torch
    log_case(test="rows_energy_changing", dtype=dtype)
    m = inputs.cloth(70)
    L = lad.Lad(m.nv, dtype=dtype, **lad.mesh_terms(m))
    prob = oracle.problem_from_mesh(m, f32=(dtype == "f32"))
    orp, oci = oracle.pattern(prob)
    out = L.alloc_outputs()
    for k in range(4):
        x_h = host_input(m.x + 0.01 * k * m.h * np.sin(np.arange(3 * m.nv)).reshape(m.nv, 3), dtype)
        x = dev(x_h, dtype)
        if k == 2:
            L.eval(x, out=out, energy=False)
        E, g, H = L.eval(x, out=out)
        torch.cuda.synchronize()
        Eo, go, Ho = oracle.evaluate(prob, orp, oci, x_h)
        assert rel([E.item()], [Eo]) <= TOL[dtype], (k, E.item(), Eo)
    assert L.device_status() == 0
    L.close()


def test_springs_only_and_inertia_only_rows(lad):
    log_case(test="rows_single_terms")
    m = inputs.cloth(20)
    for springs, inertia in ((True, False), (False, True)):
        L, prob, x_h, res = run_eval(lad, m, "f64", springs=springs, inertia=inertia)
        assert L.get_info()["eval_path"] == lad.LAD_PATH_ROWS
        check_against_oracle(prob, x_h, res, "f64")
        L.close()


@pytest.mark.parametrize("n,dtype,det,lds,path", [
    (12, "f64", False, 0, "patch_lds_atomic"), (33, "f32", False, 8192, "patch"),
    (33, "f64", True, 8192, "patch"), (64, "f32", True, 0, "patch"),
    (64, "f32", False, 0, "patch_lds_atomic"),
    (2, "f64", False, 0, "rows"), (12, "f64", False, 0, "rows"), (33, "f32", False, 0, "rows"),
    (64, "f32", False, 0, "rows"), (64, "f64", False, 0, "rows"), (129, "f32", False, 0, "rows"),
])
def test_face_eval(lad, n, dtype, det, lds, path):
    log_case(test="face_eval", n=n, dtype=dtype, det=det, lds=lds, path=path)
    m = inputs.face_grid(n)
    L, prob, x_h, res = run_eval(lad, m, dtype, det, lds, springs=False, inertia=False,
                                 faces=True, path=path)
    assert L.get_info()["eval_path"] == {"rows": lad.LAD_PATH_ROWS, "patch": lad.LAD_PATH_PATCH,
                                         "patch_lds_atomic": lad.LAD_PATH_PATCH_LDS_ATOMIC}[path]
    check_against_oracle(prob, x_h, res, dtype)
    L.close()


@pytest.mark.parametrize("dtype,det,path", [("f64", False, "patch_lds_atomic"),
                                            ("f32", False, "patch"), ("f32", True, "patch"),
                                            ("f64", False, "rows"), ("f32", False, "rows")])
def test_all_terms_eval(lad, dtype, det, path):
    log_case(test="all_terms", dtype=dtype, det=det, path=path)
    m = inputs.cloth(29)
    L, prob, x_h, res = run_eval(lad, m, dtype, det, 7000, springs=True, inertia=True,
                                 faces=True, path=path)
    check_against_oracle(prob, x_h, res, dtype)
    L.close()


@pytest.mark.parametrize("n,dtype,det,faces,lds,path", [
    (20, "f64", False, True, 0, "patch_lds_atomic"), (45, "f32", False, True, 8192, "patch"),
    (45, "f32", False, False, 8192, "patch_lds_atomic"),
    (45, "f64", True, False, 8192, "patch"), (64, "f32", True, True, 0, "patch"),
    (45, "f64", False, False, 0, "rows"), (100, "f32", False, False, 0, "rows"),
    (20, "f64", False, True, 0, "rows"), (45, "f32", False, True, 0, "rows"),
    (64, "f64", False, True, 0, "rows"),
])
def test_hvp(lad, n, dtype, det, faces, lds, path):
    import torch
    log_case(test="hvp", n=n, dtype=dtype, det=det, faces=faces, lds=lds, path=path)
    m = inputs.cloth(n)
    L = lad.Lad(m.nv, dtype=dtype, deterministic=det, patch_lds_bytes=lds, path=path,
                **lad.mesh_terms(m, faces=faces))
    prob = oracle.problem_from_mesh(m, faces=faces, f32=(dtype == "f32"))
    x_h = host_input(m.x, dtype)
    v_h = host_input(inputs.hvp_direction(m.nv), dtype)
    y = L.hvp(dev(x_h, dtype), dev(v_h, dtype))
    torch.cuda.synchronize()
    orp, oci = oracle.pattern(prob)
    yo = oracle.hvp(prob, orp, oci, x_h, v_h)
    assert rel(y.cpu().numpy(), yo) <= TOL[dtype]
    L.close()


@pytest.mark.parametrize("path", ["auto", "patch", "patch_lds_atomic", "patch_atomic"])
def test_single_vertex_and_isolated(lad, path):
    """Degenerate meshes, on every decomposition: one vertex with inertia
    only; a mesh with isolated vertices (rows holding only the diagonal)."""
    import torch
    log_case(test="degenerate", path=path)
    X = np.array([[0.1, 0.2, 0.3]])
    L = lad.Lad(1, dtype="f64", x_tilde=np.zeros((1, 3)), c=4.0, path=path)
    E, g, H = L.eval(dev(X, "f64"))
    torch.cuda.synchronize()
    assert abs(E.item() - 0.5 * 4.0 * 0.14) < 1e-15
    assert np.allclose(g.cpu().numpy(), 4.0 * X)
    assert np.allclose(H.cpu().numpy()[0], 4.0 * np.eye(3))
    L.close()
    faces = np.array([[0, 1, 2]], dtype=np.int32)
    x = np.random.default_rng(3).normal(size=(6, 3))
    springs = np.array([[0, 1], [1, 2], [0, 2], [4, 5]], dtype=np.int32)
    rest = np.array([1.0, 1.1, 0.9, 0.5])
    L = lad.Lad(6, dtype="f64", faces=faces, springs=springs, rest_len=rest, k=3.0,
                x_tilde=np.zeros((6, 3)), c=2.0, path=path)
    E, g, H = L.eval(dev(x, "f64"))
    rp, ci = L.pattern()
    torch.cuda.synchronize()
    prob = oracle.Problem(nv=6, faces=faces, springs=springs, rest_len=rest, k=3.0,
                          x_tilde=np.zeros((6, 3)), c=2.0)
    check_against_oracle(prob, x, (E.item(), g.cpu().numpy(), H.cpu().numpy(),
                                   rp.cpu().numpy(), ci.cpu().numpy()), "f64")
    assert np.diff(rp.cpu().numpy())[3] == 1  # vertex 3 is isolated
    L.close()


def test_outputs_fully_overwritten(lad):
    """Every call overwrites its outputs: stale buffer contents never leak."""
    import torch
    log_case(test="overwrite")
    m = inputs.cloth(23)
    L = lad.Lad(m.nv, dtype="f32", patch_lds_bytes=6144, **lad.mesh_terms(m))
    x = dev(host_input(m.x, "f32"), "f32")
    E1, g1, H1 = L.eval(x)
    E2, g2, H2 = L.alloc_outputs()
    E2.fill_(1e30)
    g2.fill_(float("nan"))
    H2.fill_(float("nan"))
    L.eval(x, out=(E2, g2, H2))
    torch.cuda.synchronize()
    n = L.get_info()["nnzb_active"]
    assert torch.equal(E1, E2) or abs(E1.item() - E2.item()) <= 1e-6 * abs(E1.item())
    assert torch.isfinite(g2).all() and torch.isfinite(H2[:n]).all()
    L.close()


@pytest.mark.parametrize("path", ["rows", "patch"])
def test_eval_without_energy(lad, path):
    """d_energy = NULL skips the energy sum; gradient and Hessian are the
    same as with it, and the energy buffer is left untouched.  (The patch
    path runs in its deterministic mode so that two calls compare bitwise;
    its default mode sums with LDS atomics in a varying order.)"""
    import torch
    log_case(test="no_energy", path=path)
    m = inputs.cloth(33)
    L = lad.Lad(m.nv, dtype="f64", path=path, deterministic=(path == "patch"),
                **lad.mesh_terms(m))
    x = dev(m.x, "f64")
    E1, g1, H1 = L.eval(x)
    E2, g2, H2 = L.alloc_outputs()
    E2.fill_(-7.0)
    L.eval(x, out=(E2, g2, H2), energy=False)
    torch.cuda.synchronize()
    n = L.get_info()["nnzb_active"]
    assert E2.item() == -7.0
    assert torch.equal(g1, g2) and torch.equal(H1[:n], H2[:n])
    L.close()


@pytest.mark.parametrize("path,faces,det", [("patch", False, True), ("patch", True, True),
                                            ("rows", True, False), ("rows", False, False)])
def test_bitwise_reproducible(lad, path, faces, det):
    """The deterministic patch mode (colour phases) and the row path sum in a
    fixed order: ten evaluations and HVPs are bitwise identical."""
    import torch
    log_case(test="reproducible", path=path, faces=faces, det=det)
    m = inputs.cloth(41)
    L = lad.Lad(m.nv, dtype="f32", path=path, deterministic=det, patch_lds_bytes=6144,
                **lad.mesh_terms(m, faces=faces))
    x = dev(host_input(m.x, "f32"), "f32")
    v = dev(host_input(inputs.hvp_direction(m.nv), "f32"), "f32")
    E0, g0, H0 = L.eval(x)
    y0 = L.hvp(x, v)
    torch.cuda.synchronize()
    E0, g0, H0, y0 = E0.clone(), g0.clone(), H0.clone(), y0.clone()
    for _ in range(10):
        E, g, H = L.eval(x)
        y = L.hvp(x, v)
        torch.cuda.synchronize()
        assert torch.equal(E, E0) and torch.equal(g, g0) and torch.equal(H, H0)
        assert torch.equal(y, y0)
    L.close()


@pytest.mark.parametrize("path", ["rows", "patch"])
def test_no_host_sync_in_step_calls(lad, path):
    """Evaluation, HVP and pair insertion never synchronise with the host: the
    library's own count of host synchronisations grows only by the one that
    the second lad_get_info makes."""
    import torch
    log_case(test="no_host_sync", path=path)
    m = inputs.cloth(30)
    P = 18
    L = lad.Lad(m.nv, dtype="f32", path=path,
                **lad.mesh_terms(m, pair_capacity=P, kappa=inputs.BARRIER_KAPPA, dhat=0.5 * m.h))
    x = dev(host_input(m.x, "f32"), "f32")
    v = dev(host_input(inputs.hvp_direction(m.nv), "f32"), "f32")
    pairs, _ = inputs.contact_pairs(m, m.x, step=0)
    pd = torch.tensor(pairs, dtype=torch.int32, device="cuda")
    out = L.alloc_outputs()
    s0 = L.get_info()["host_syncs"]
    for _ in range(3):
        L.eval(x, out=out)
        L.eval(x, out=out, energy=False)
        L.hvp(x, v)
        L.insert_pairs(pd)
        L.eval(x, out=out)
        L.hvp(x, v)
        L.insert_pairs(None)
    s1 = L.get_info()["host_syncs"]
    assert s1 - s0 == 1
    torch.cuda.synchronize()
    L.close()


def _spin_seconds(torch, cycles):
    torch.cuda.synchronize()
    import time
    t0 = time.perf_counter()
    torch.cuda._sleep(cycles)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


@pytest.mark.parametrize("path", ["rows", "patch"])
def test_step_calls_return_while_stream_busy(lad, path):
    """The same check as test_no_host_sync_in_step_calls, independent of
    the library's own count: a spin kernel of at least a tenth of a second
    is queued first on the stream, and the step calls (evaluation, HVP,
    insertion, restore) must all return to the host well before it ends,
    which they could not if any of them waited for the stream."""
    import time
    import torch
    log_case(test="stream_busy", path=path)
    m = inputs.cloth(30)
    P = 18
    L = lad.Lad(m.nv, dtype="f32", path=path,
                **lad.mesh_terms(m, pair_capacity=P, kappa=inputs.BARRIER_KAPPA, dhat=0.5 * m.h))
    x = dev(host_input(m.x, "f32"), "f32")
    v = dev(host_input(inputs.hvp_direction(m.nv), "f32"), "f32")
    pairs, _ = inputs.contact_pairs(m, m.x, step=0)
    pd = torch.tensor(pairs, dtype=torch.int32, device="cuda")
    out = L.alloc_outputs()
    y = torch.empty_like(v)
    L.eval(x, out=out)  # first calls (lazy set-up) outside the timed part
    L.hvp(x, v, out=y)
    cycles = 20_000_000
    spin = _spin_seconds(torch, cycles)
    while spin < 0.1:
        cycles *= 2
        spin = _spin_seconds(torch, cycles)
    torch.cuda._sleep(cycles)
    t0 = time.perf_counter()
    for _ in range(3):
        L.eval(x, out=out)
        L.hvp(x, v, out=y)
        L.insert_pairs(pd)
        L.eval(x, out=out, energy=False)
        L.insert_pairs(None)
    host = time.perf_counter() - t0
    torch.cuda.synchronize()
    assert host < 0.5 * spin, (host, spin)
    L.close()


def test_debug_mode_reports_nonfinite_outputs(lad):
    """lad_set_debug(LAD_DEBUG_NONFINITE): an evaluation or product whose
    output holds a NaN or an inf latches LAD_ERR_NONFINITE for
    lad_device_status; finite outputs leave it clear; with the mode off no
    check runs."""
    import torch
    log_case(test="debug_nonfinite")
    m = inputs.cloth(20)
    L = lad.Lad(m.nv, dtype="f32", **lad.mesh_terms(m))
    x = dev(host_input(m.x, "f32"), "f32")
    v = dev(host_input(inputs.hvp_direction(m.nv), "f32"), "f32")
    out = L.alloc_outputs()
    L.set_debug(lad.LAD_DEBUG_NONFINITE)
    L.eval(x, out=out)
    L.hvp(x, v)
    assert L.device_status() == lad.LAD_OK
    xbad = x.clone()
    xbad[7, 1] = float("nan")
    L.eval(xbad, out=out)
    assert L.device_status() == lad.LAD_ERR_NONFINITE
    assert L.device_status() == lad.LAD_OK  # read and cleared
    vbad = v.clone()
    vbad[3, 0] = float("inf")
    L.hvp(x, vbad)
    assert L.device_status() == lad.LAD_ERR_NONFINITE
    L.set_debug(0)
    L.eval(xbad, out=out)
    assert L.device_status() == lad.LAD_OK
    with pytest.raises(lad.LadError):
        L.set_debug(2)
    torch.cuda.synchronize()
    L.close()
