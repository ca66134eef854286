"""The patch path with element-once patches and global atomics for the rows
of other patches (LAD_PATH_PATCH_ATOMIC, the page's own assembly) against
the fp64 CPU oracle: pattern bit for bit, E, g, H and H v within the
tolerances of gpu_util.TOL.  Small LDS budgets force many patches, so most
rows receive foreign atomics; outputs are pre-filled with NaN to show that
every entry is written (boundary slots zeroed, the rest stored)."""
import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from gpu_util import TOL, dev, host_input, log_case, rel

pytestmark = pytest.mark.gpu


def make(lad, mesh, dtype, lds, springs=True, inertia=True, faces=False):
    L = lad.Lad(mesh.nv, dtype=dtype, patch_lds_bytes=lds, path="patch_atomic",
                **lad.mesh_terms(mesh, springs=springs, inertia=inertia, faces=faces))
    info = L.get_info()
    assert info["eval_path"] == lad.LAD_PATH_PATCH_ATOMIC
    prob = oracle.problem_from_mesh(mesh, springs=springs, inertia=inertia, faces=faces,
                                    f32=(dtype == "f32"))
    return L, prob, info


def eval_nan_filled(L, x):
    import torch
    E, g, H = L.alloc_outputs()
    E.fill_(float("nan"))
    g.fill_(float("nan"))
    H.fill_(float("nan"))
    L.eval(x, out=(E, g, H))
    rp, ci = L.pattern()
    torch.cuda.synchronize()
    return (E.cpu().numpy()[0], g.cpu().numpy(), H.cpu().numpy(), rp.cpu().numpy(),
            ci.cpu().numpy())


def check_eval(prob, x_h, res, dtype):
    E, g, H, rp, ci = res
    orp, oci = oracle.pattern(prob)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    Hn = H[: oci.size]
    assert np.isfinite(g).all() and np.isfinite(Hn).all(), "an output entry was not written"
    Eo, go, Ho = oracle.evaluate(prob, orp, oci, x_h)
    tol = TOL[dtype]
    assert rel([E], [Eo]) <= tol, (E, Eo)
    assert rel(g, go) <= tol, rel(g, go)
    assert rel(Hn, Ho) <= tol, rel(Hn, Ho)


@pytest.mark.parametrize("n,dtype,lds,faces", [
    (10, "f64", 0, False), (10, "f32", 0, False), (37, "f32", 6144, False),
    (37, "f64", 6144, False), (100, "f32", 0, False), (29, "f64", 7000, True),
    (29, "f32", 7000, True), (64, "f32", 8192, True),
])
def test_cloth_eval_patch_atomic(lad, n, dtype, lds, faces):
    log_case(test="patch_atomic_eval", n=n, dtype=dtype, lds=lds, faces=faces)
    m = inputs.cloth(n)
    L, prob, info = make(lad, m, dtype, lds, faces=faces)
    if lds:
        assert info["npatches"] > 4
    x_h = host_input(m.x, dtype)
    check_eval(prob, x_h, eval_nan_filled(L, dev(x_h, dtype)), dtype)
    L.close()


@pytest.mark.parametrize("n,dtype,lds", [(33, "f32", 8192), (33, "f64", 8192), (64, "f32", 0)])
def test_face_eval_patch_atomic(lad, n, dtype, lds):
    log_case(test="patch_atomic_faces", n=n, dtype=dtype, lds=lds)
    m = inputs.face_grid(n)
    L, prob, _ = make(lad, m, dtype, lds, springs=False, inertia=False, faces=True)
    x_h = host_input(m.x, dtype)
    check_eval(prob, x_h, eval_nan_filled(L, dev(x_h, dtype)), dtype)
    L.close()


@pytest.mark.parametrize("n,dtype,faces,lds", [
    (20, "f64", True, 0), (45, "f32", True, 8192), (45, "f64", False, 8192), (100, "f32", False, 0),
])
def test_hvp_patch_atomic(lad, n, dtype, faces, lds):
    import torch
    log_case(test="patch_atomic_hvp", n=n, dtype=dtype, faces=faces, lds=lds)
    m = inputs.cloth(n)
    L, prob, _ = make(lad, m, dtype, lds, faces=faces)
    x_h = host_input(m.x, dtype)
    v_h = host_input(inputs.hvp_direction(m.nv), dtype)
    y = torch.full((m.nv, 3), float("nan"), dtype=torch.float32 if dtype == "f32" else torch.float64,
                   device="cuda")
    L.hvp(dev(x_h, dtype), dev(v_h, dtype), out=y)
    torch.cuda.synchronize()
    orp, oci = oracle.pattern(prob)
    yo = oracle.hvp(prob, orp, oci, x_h, v_h)
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    assert rel(yh, yo) <= TOL[dtype]
    L.close()


def test_cloth_1000_patch_atomic(lad):
    """Full-size 1000 x 1000 fp32 cloth (the headline workload) in the launch
    configuration the bench times, against the oracle."""
    import torch
    log_case(test="patch_atomic_1000")
    m = inputs.cloth(1000)
    L, prob, info = make(lad, m, "f32", 0)
    x_h = host_input(m.x, "f32")
    x = dev(x_h, "f32")
    check_eval(prob, x_h, eval_nan_filled(L, x), "f32")
    v_h = host_input(inputs.hvp_direction(m.nv), "f32")
    y = L.hvp(x, dev(v_h, "f32"))
    torch.cuda.synchronize()
    orp, oci = oracle.pattern(prob)
    assert rel(y.cpu().numpy(), oracle.hvp(prob, orp, oci, x_h, v_h)) <= TOL["f32"]
    L.close()
