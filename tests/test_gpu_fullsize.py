"""Parity at the full benchmark sizes, in the configuration bench.py times
(default library options; fp32): the 1000 x 1000 cloth (row path, and the
patch path's assemblies the bench also times), the 512 x 512
symmetric-Dirichlet face grid (eval and HVP), and the 1000 x 1000 cloth
with 20,000 fresh contact pairs per step over three steps and a final
insert of nothing.  The oracle evaluates each whole
problem on the host (fp32-rounded inputs, fp64 arithmetic); patterns must
match bit for bit and values within the fp32 tolerance."""
import numpy as np
import pytest

import oracle
from sparse_autodiff_mesh_amd import inputs

from gpu_util import TOL, dev, host_input, log_case, rel, row_blocks

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


@pytest.mark.parametrize("det", [False, True])
def test_cloth_1000_patch_path(lad, det):
    """The element-owner patch path at the full size the bench times it at
    (LDS atomics, and colour phases with det): E, g, H and H v against the
    oracle.  It is also the automatic fallback for meshes the row path does
    not take."""
    import torch
    log_case(test="full_cloth1000_patch", det=det)
    m = inputs.cloth(1000)
    L = lad.Lad(m.nv, dtype="f32", path="patch", deterministic=det, **lad.mesh_terms(m))
    assert L.get_info()["eval_path"] == lad.LAD_PATH_PATCH
    x_h = host_input(m.x, "f32")
    prob = oracle.problem_from_mesh(m, f32=True)
    orp, oci = compare(L, prob, x_h, run(L, x_h))
    v_h = host_input(inputs.hvp_direction(m.nv), "f32")
    y = L.hvp(dev(x_h, "f32"), dev(v_h, "f32"))
    torch.cuda.synchronize()
    assert rel(y.cpu().numpy(), oracle.hvp(prob, orp, oci, x_h, v_h)) <= TOL["f32"]
    L.close()


@pytest.mark.parametrize("path", ["patch", "patch_atomic"])
def test_faces_512_patch_paths(lad, path):
    """The 512 x 512 face grid on the patch path's LDS-atomic and
    global-atomic assemblies, at the size the bench times them."""
    log_case(test="full_faces512_patch", path=path)
    m = inputs.face_grid(512)
    L = lad.Lad(m.nv, dtype="f32", path=path,
                **lad.mesh_terms(m, springs=False, inertia=False, faces=True))
    x_h = host_input(m.x, "f32")
    prob = oracle.problem_from_mesh(m, springs=False, inertia=False, faces=True, f32=True)
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


def test_cloth_1000_pair_steps(lad):
    """Contact steps at full size: fresh pairs at steps 0, 1 and 2 (the two
    pattern buffers alternate: 1, 2, 1, so each is written over again and
    the previous step's pairs must be gone), then an insert of nothing,
    which restores the topology pattern.  Every step: the pattern bit for
    bit, E, g, H and H v within the fp32 tolerance over the whole arrays,
    and over the rows the pairs touch alone (their blocks, g and y), where
    an error confined to the contact code would otherwise hide among the
    seven million topology blocks."""
    import torch
    log_case(test="full_pairs1000_steps")
    m = inputs.cloth(1000)
    P = int(round(0.02 * m.nv))
    dhat = 0.5 * m.h
    kappa = inputs.BARRIER_KAPPA
    L = lad.Lad(m.nv, dtype="f32",
                **lad.mesh_terms(m, pair_capacity=P, kappa=kappa, dhat=dhat))
    assert L.get_info()["eval_path"] == lad.LAD_PATH_ROWS
    v_h = host_input(inputs.hvp_direction(m.nv), "f32")
    tol = TOL["f32"]
    for step in range(3):
        log_case(test="full_pairs1000_steps", step=step)
        pairs, x = inputs.contact_pairs(m, m.x, step=step)
        L.insert_pairs(torch.tensor(pairs, dtype=torch.int32, device="cuda"))
        x_h = host_input(x, "f32")
        E, g, H, rp, ci = run(L, x_h)
        y = L.hvp(dev(x_h, "f32"), dev(v_h, "f32"))
        torch.cuda.synchronize()
        assert L.device_status() == 0
        info = L.get_info()
        assert info["active_buffer"] == 1 + step % 2
        assert info["nnzb_active"] == 7032002 and info["npairs_active"] == P
        prob = oracle.problem_from_mesh(m, pairs=pairs, kappa=kappa, dhat=dhat, f32=True)
        orp, oci = oracle.pattern(prob)
        assert np.array_equal(rp, orp), "row_ptr differs"
        assert np.array_equal(ci, oci), "col_idx differs"
        Eo, go, Ho = oracle.evaluate(prob, orp, oci, x_h)
        yo = oracle.bsr_spmv(orp, oci, Ho, v_h)
        Hg, yg = H[: oci.size], y.cpu().numpy()
        assert rel([E], [Eo]) <= tol, (E, Eo)
        assert rel(g, go) <= tol
        assert rel(Hg, Ho) <= tol
        assert rel(yg, yo) <= tol
        rows = np.unique(pairs.reshape(-1))
        blk = row_blocks(orp, rows)
        assert rel(Hg[blk], Ho[blk]) <= tol, rel(Hg[blk], Ho[blk])
        assert rel(g[rows], go[rows]) <= tol, rel(g[rows], go[rows])
        assert rel(yg[rows], yo[rows]) <= tol, rel(yg[rows], yo[rows])
        del H, Hg, Ho
    L.insert_pairs(None)
    x_h = host_input(m.x, "f32")
    res = run(L, x_h)
    assert L.get_info()["active_buffer"] == 0
    assert res[3][-1] == 6992002
    compare(L, oracle.problem_from_mesh(m, f32=True), x_h, res)
    L.close()
