"""Parity at the full benchmark sizes, in the configuration bench.py times
(default library options; fp32): the 1000 x 1000 cloth, the 512 x 512
symmetric-Dirichlet face grid (eval and HVP), and one step of the 1000 x
1000 cloth with 20,000 contact pairs.  The oracle evaluates each whole
problem on the host (fp32-rounded inputs, fp64 arithmetic); patterns must
match bit for bit and values within the fp32 tolerance."""
import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from gpu_util import TOL, dev, host_input, log_case, rel

pytestmark = pytest.mark.gpu


def compare(L, prob, x_h, res):
    E, g, H, rp, ci = res
    orp, oci = oracle.pattern(prob)
    assert np.array_equal(rp, orp), "row_ptr differs"
    assert np.array_equal(ci, oci), "col_idx differs"
    Eo, go, Ho = oracle.evaluate(prob, orp, oci, x_h)
    tol = TOL["f32"]
    assert rel([E], [Eo]) <= tol, (E, Eo)
    assert rel(g, go) <= tol, rel(g, go)
    assert rel(H[: oci.size], Ho) <= tol, rel(H[: oci.size], Ho)
    return orp, oci


def run(L, x_h):
    import torch
    E, g, H = L.eval(dev(x_h, "f32"))
    rp, ci = L.pattern()
    torch.cuda.synchronize()
    return E.item(), g.cpu().numpy(), H.cpu().numpy(), rp.cpu().numpy(), ci.cpu().numpy()


def test_cloth_1000(lad):
    log_case(test="full_cloth1000")
    m = inputs.cloth(1000)
    L = lad.Lad(m.nv, dtype="f32", **lad.mesh_terms(m))
    assert L.get_info()["nnzb_base"] == 6992002
    x_h = host_input(m.x, "f32")
    prob = oracle.problem_from_mesh(m, f32=True)
    compare(L, prob, x_h, run(L, x_h))
    L.close()


def test_faces_512_eval_and_hvp(lad):
    import torch
    log_case(test="full_faces512")
    m = inputs.face_grid(512)
    L = lad.Lad(m.nv, dtype="f32",
                **lad.mesh_terms(m, springs=False, inertia=False, faces=True))
    assert L.get_info()["nnzb_base"] == 1830914
    x_h = host_input(m.x, "f32")
    prob = oracle.problem_from_mesh(m, springs=False, inertia=False, faces=True, f32=True)
    orp, oci = compare(L, prob, x_h, run(L, x_h))
    v_h = host_input(inputs.hvp_direction(m.nv), "f32")
    y = L.hvp(dev(x_h, "f32"), dev(v_h, "f32"))
    torch.cuda.synchronize()
    yo = oracle.hvp(prob, orp, oci, x_h, v_h)
    assert rel(y.cpu().numpy(), yo) <= TOL["f32"]
    L.close()


def test_cloth_1000_with_pairs(lad):
    import torch
    log_case(test="full_pairs1000")
    m = inputs.cloth(1000)
    P = int(round(0.02 * m.nv))
    dhat = 0.5 * m.h
    L = lad.Lad(m.nv, dtype="f32",
                **lad.mesh_terms(m, pair_capacity=P, kappa=inputs.BARRIER_KAPPA, dhat=dhat))
    pairs, x = inputs.contact_pairs(m, m.x, step=0)
    L.insert_pairs(torch.tensor(pairs, dtype=torch.int32, device="cuda"))
    x_h = host_input(x, "f32")
    res = run(L, x_h)
    assert L.device_status() == 0
    assert L.get_info()["nnzb_active"] == 7032002
    prob = oracle.problem_from_mesh(m, pairs=pairs, kappa=inputs.BARRIER_KAPPA, dhat=dhat,
                                    f32=True)
    compare(L, prob, x_h, res)
    L.close()
