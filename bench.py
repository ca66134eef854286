#!/usr/bin/env python3
"""Throughput of per-element forward-mode AD with on-GPU sparse assembly.

One step is one call of lad_eval_energy_grad_hess on the mass-spring cloth
over a 1000 x 1000 vertex grid in fp32 (2,996,001 springs + 1,000,000 inertia
terms; gradient of 3e6 values and a 3x3-block CSR Hessian of 6,992,002
blocks).  This is the workload of the cloth timing table on the page
"Locality-Aware Automatic Differentiation on the GPU for Mesh-Based
Computations" (section "Results": gradient and Hessian per step, linear solve
excluded).  Inputs are seeded synthetic grids, resident in HBM before the
timed region starts; the pattern build (initialisation) is not timed.

Prints ONE JSON line.  Besides the contract fields it carries
  roofline      the eval kernel against the HBM peak: compulsory bytes per
                launch (one read of the mesh data, one write of g and H) over
                the kernel's mean duration from HIP events on its stream
                (calls made without the energy, so each call is that one
                launch; ms_per_step includes the energy sum), plus the
                kernel's mean with a read-only 512 MB sweep before every call
                (inputs evicted from the last-level cache), the rate of a
                plain 256 MiB device copy (read + write bytes per second) and
                of a plain 256 MiB fill (write-only), all measured with the
                secondary workloads, and the counter-based HBM traffic of a
                launch from the committed profile when the kernel sources
                match it;
  cpu_baseline  the fp64 CPU oracle, single-threaded, on the same workload;
  init          the GPU time of the pattern build and the wall-clock time
                of the whole context build (not timed above);
  secondary     the other workloads (face-energy grid eval and matrix-free
                HVP, Newton-CG, the vector objective, cloth plus contact-pair
                insertion, cloth plus vertex-face contact insertion, 100 x 100
                cloth, the term front end: ARAP faces, the generic cloth set,
                ARAP + cloth fused and unfused, and the patch path's three
                assemblies).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--n 1000]
                    [--no-cpu-baseline] [--no-secondary] [--flush-mall]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published peak
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_eval_cloth1000_f32.txt")
KERNEL_SOURCES = ["lad_rows.hip", "lad_eval.hip", "lad_device.h", "dual2.h", "energies.h",
                  "lad_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic byte counts (one read of the mesh data, one write of g and H)
# ---------------------------------------------------------------------------
def compulsory_bytes_eval(nv, ns, nf, nnzb, es, inertia=True, faces=False, npairs=0):
    b = 3 * nv * es                       # x
    if inertia:
        b += 3 * nv * es                  # x_tilde
    b += ns * (es + 8)                    # rest length + two int32 endpoints
    if faces:
        b += nf * (12 + 5 * es)           # three int32 vertex ids, Dm^-1 (4), area
    b += npairs * 8                       # pair endpoints
    b += 3 * nv * es                      # g
    b += 9 * nnzb * es                    # H values
    return b


def compulsory_bytes_pair_step(L, m, npairs):
    """One contact step (insert the step's pairs, then evaluate): the pair
    list read and the new row pointers written by the insertion, then the
    evaluation's compulsory bytes on the active pattern (its nnzb includes
    the pairs' new blocks)."""
    info = L.get_info()
    b = 8 * npairs + 4 * (m.nv + 1)
    b += compulsory_bytes_eval(m.nv, m.springs.shape[0], 0, info["nnzb_active"], 4,
                               npairs=npairs)
    return b


def compulsory_bytes_terms(nv, blocks, nnzb, es, hvp=False):
    """Term front end: every element's vertex ids and constants once, x (and
    v), g (or y), and for the explicit call the H blocks once."""
    b = sum(el.shape[0] * (4 * el.shape[1] + es * cs.shape[1]) for el, cs in blocks)
    b += nv * 3 * es * (3 if hvp else 2)
    if not hvp:
        b += nnzb * 9 * es
    return b


def compulsory_bytes_hvp(nv, ns, nf, es, faces=False):
    b = 3 * 3 * nv * es                   # x, v read; y written
    b += ns * (es + 8)
    if faces:
        b += nf * (12 + 5 * es)
    return b


def compulsory_bytes_residual_jacobian(nv, ns, es):
    """Residuals and Jacobian values of the spring + inertia vector objective:
    x and x_tilde read, per spring two int32 ids and a rest length; R
    (ns + 3 nv rows) and the Jacobian values (6 ns + 3 nv) written."""
    return 2 * 3 * nv * es + ns * (8 + es) + (ns + 3 * nv) * es + (6 * ns + 3 * nv) * es


def compulsory_bytes_cg_iter(nv, ns, es):
    """One Newton-CG iteration: forming the direction d = -r + beta d_prev
    (r and d_prev read, d written: two vectors more than a plain HVP, which
    reads d as its operand), the HVP, then p and r updated from d and y (four
    vectors read, two written); the scalar steps move a few KB.  The row
    path on large meshes forms d in a launch of its own, which reads d once
    more; that is charged to the implementation."""
    return compulsory_bytes_hvp(nv, ns, 0, es) + 8 * 3 * nv * es


FACES_FILE = os.path.join(PROFILES, "counters_faces512_f32.txt")


def read_valu_busy(path, kernel):
    """VALU-busy share of `kernel` from a committed rocprofv3 counter summary
    (SQ_INSTS_VALU x 4 cycles over 1024 SIMDs at 2.4 GHz, divided by the
    traced average duration), if it was taken on the current kernel sources;
    else None."""
    if not os.path.exists(path):
        return None
    sha, cur, val = None, None, {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("[") and line.endswith("]"):
                cur = line[1:-1]
            elif line.startswith("kernel_source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("valu_busy:") and cur:
                val[cur] = float(line.split(":", 1)[1])
    if sha != kernel_source_sha():
        return None
    return val.get(kernel)


def code_only(text):
    """C++ source text without its comments, whitespace runs collapsed: what
    the compiler sees, so that a comment edit keeps the fingerprint."""
    out, i, n, quote = [], 0, len(text), None
    while i < n:
        c = text[i]
        if quote:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(text[i + 1])
                i += 2
                continue
            if c == quote:
                quote = None
            i += 1
        elif c in "\"'":
            quote = c
            out.append(c)
            i += 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha():
    """Fingerprint of the kernel sources the committed counter summaries were
    taken on (their code, not their comments)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_autodiff_mesh_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_only(f.read()).encode() + b"\0")
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_sha():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
class Timer:
    """HIP events on torch's current stream, which is the stream every lad_*
    call is enqueued on (the binding passes it explicitly).

    Warm-up: at least `warmup` untimed calls, and (unless warmup is 0) calls
    until `min_warm_s` of wall time has passed, so that a GPU left idle
    during a context's host-side set-up is back at its running clocks when
    the timed calls start."""

    def __init__(self, torch, min_warm_s=0.05):
        self.torch = torch
        self.min_warm_s = min_warm_s

    def run(self, fn, steps, warmup, flush=None):
        t = self.torch
        t0 = time.perf_counter()
        for _ in range(warmup):
            fn()
        t.cuda.synchronize()
        while warmup > 0 and time.perf_counter() - t0 < self.min_warm_s:
            for _ in range(warmup):
                fn()
            t.cuda.synchronize()
        starts = [t.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [t.cuda.Event(enable_timing=True) for _ in range(steps)]
        total0 = t.cuda.Event(enable_timing=True)
        total1 = t.cuda.Event(enable_timing=True)
        # the K-step region: the calls back to back, events only at its ends
        # (without a flush; with one, the region includes it)
        t.cuda.synchronize()
        total0.record()
        for _ in range(steps):
            if flush is not None:
                flush()
            fn()
        total1.record()
        t.cuda.synchronize()
        # per-call durations, an event pair around each call
        for i in range(steps):
            if flush is not None:
                flush()
            starts[i].record()
            fn()
            ends[i].record()
        t.cuda.synchronize()
        per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
        return {
            "mean_ms": sum(per) / len(per),
            "median_ms": per[len(per) // 2],
            "min_ms": per[0],
            "region_ms": total0.elapsed_time(total1),
        }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def cloth_ctx(binding, mesh, dtype, pair_capacity=0, dhat=0.0, kappa=0.0):
    return binding.Lad(mesh.nv, dtype=dtype,
                       **binding.mesh_terms(mesh, pair_capacity=pair_capacity,
                                            kappa=kappa, dhat=dhat))


def to_dev(torch, a, dtype):
    import numpy as np
    t = torch.float64 if dtype == "f64" else torch.float32
    return torch.tensor(np.ascontiguousarray(a), dtype=t, device="cuda")


def bench_headline(torch, binding, inputs, args, timer):
    m = inputs.cloth(args.n)
    t0 = time.perf_counter()
    L = binding.Lad(m.nv, dtype="f32", patch_lds_bytes=args.patch_lds, path=args.path,
                    deterministic=args.deterministic, **binding.mesh_terms(m))
    torch.cuda.synchronize()
    init_s = time.perf_counter() - t0
    info = L.get_info()
    x = to_dev(torch, m.x, "f32")
    E, g, H = L.alloc_outputs()
    out = (E, g, H)
    fn = lambda: L.eval(x, out=out)  # noqa: E731
    fn_kernel = lambda: L.eval(x, out=out, energy=False)  # noqa: E731
    # A read-only sweep of 512 MB (twice the 256 MB last-level cache) before
    # a call evicts the call's inputs without leaving dirty lines to drain
    # during the call.
    flush = None
    if args.flush_mall:
        scratch = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        flush = lambda: scratch.sum()  # noqa: E731
    # the whole call (evaluation + energy sum): the step time
    r = timer.run(fn, args.steps, args.warmup, flush=flush)
    # the evaluation kernel alone (energy not requested: one launch per call)
    rk = timer.run(fn_kernel, args.steps, args.warmup, flush=flush)
    # With the secondary workloads: the kernel again with a read-only 512 MB
    # sweep before every call, which evicts its inputs from the last-level
    # cache (MALL), and a plain device copy, the achievable HBM rate of a
    # read + write stream.  (Left out of the profiled headline-only runs,
    # whose kernel statistics must match the warm timing above.)
    rkf, copy_gbps, fill_gbps = None, None, None
    if not args.no_secondary:
        if not args.flush_mall:
            scratch = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
            rkf = timer.run(fn_kernel, min(args.steps, 50), 2, flush=lambda: scratch.sum())
            del scratch
        nb = 256 * 1024 * 1024
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        rc = timer.run(lambda: dst.copy_(src), 20, 3)
        copy_gbps = 2 * nb / (rc["mean_ms"] * 1e-3) / 1e9
        # a plain write-only stream (torch's fill): the ceiling of a
        # write-dominated kernel such as this one (88 % of its bytes are H
        # and g writes)
        rf = timer.run(lambda: dst.fill_(1.0), 20, 3)
        fill_gbps = nb / (rf["mean_ms"] * 1e-3) / 1e9
        del src, dst
    nv, ns = m.nv, m.springs.shape[0]
    nnzb = info["nnzb_base"]
    terms = ns + nv
    bc = compulsory_bytes_eval(nv, ns, 0, nnzb, 4)
    torch.cuda.synchronize()
    energy = E.item()
    res = {
        "mesh": m, "info": info, "timing": r, "timing_kernel": rk, "timing_flushed": rkf,
        "copy_gbps": copy_gbps, "fill_gbps": fill_gbps, "terms": terms, "bytes": bc,
        "energy": energy, "nnzb": nnzb, "ns": ns, "nv": nv, "init_s": init_s,
    }
    L.close()
    return res


def bench_hvp_only(torch, binding, inputs, args, timer):
    """The matrix-free HVP of the cloth alone (for counter runs): one line of
    JSON with its event timing and compulsory bytes."""
    m = inputs.cloth(args.n)
    L = cloth_ctx(binding, m, "f32")
    x = to_dev(torch, m.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(m.nv), "f32")
    y = torch.empty_like(v)
    r = timer.run(lambda: L.hvp(x, v, out=y), args.steps, args.warmup)
    bc = compulsory_bytes_hvp(m.nv, m.springs.shape[0], 0, 4)
    L.close()
    return {"workload": f"matrix-free HVP, mass-spring cloth {args.n}x{args.n}, fp32",
            "kernel": "k_hvp_rows<float, false, false>", "steps": args.steps,
            "warmup": args.warmup, "ms_mean": round(r["mean_ms"], 5),
            "algorithmic_bytes": bc, "GBps": round(bc / (r["mean_ms"] * 1e-3) / 1e9, 1)}


def bench_faces_only(torch, binding, inputs, args, timer):
    """The 512 x 512 symmetric-Dirichlet face grid alone (for counter runs):
    the explicit evaluation kernel (no energy sum: one launch per call),
    then the matrix-free HVP, with their event timings and compulsory
    bytes."""
    f = inputs.face_grid(512)
    L = binding.Lad(f.nv, dtype="f32",
                    **binding.mesh_terms(f, springs=False, inertia=False, faces=True))
    info = L.get_info()
    x = to_dev(torch, f.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(f.nv), "f32")
    y = torch.empty_like(v)
    out = L.alloc_outputs()
    re = timer.run(lambda: L.eval(x, out=out, energy=False), args.steps, args.warmup)
    rh = timer.run(lambda: L.hvp(x, v, out=y), args.steps, args.warmup)
    nf = f.faces.shape[0]
    be = compulsory_bytes_eval(f.nv, 0, nf, info["nnzb_base"], 4, inertia=False, faces=True)
    bh = compulsory_bytes_hvp(f.nv, 0, nf, 4, faces=True)
    L.close()
    return {"workload": "symmetric-Dirichlet faces, 512x512 vertex grid, fp32",
            "kernels": ["k_eval_face_rows<float>", "k_hvp_rows<float, true, false>"],
            "faces": nf, "chunks": info["npatches"], "steps": args.steps, "warmup": args.warmup,
            "eval_ms_mean": round(re["mean_ms"], 5), "eval_algorithmic_bytes": be,
            "eval_GBps": round(be / (re["mean_ms"] * 1e-3) / 1e9, 1),
            "hvp_ms_mean": round(rh["mean_ms"], 5), "hvp_algorithmic_bytes": bh,
            "hvp_GBps": round(bh / (rh["mean_ms"] * 1e-3) / 1e9, 1)}


def bench_pairs_only(torch, binding, inputs, args, timer):
    """The 1000 x 1000 cloth with 2 % contact pairs per step alone (for
    kernel traces and counter runs): a step inserts the step's pairs, then
    evaluates; one line of JSON with the step, insertion and evaluation
    timings and the step's compulsory bytes."""
    m = inputs.cloth(args.n)
    dhat = 0.5 * m.h
    P = int(round(0.02 * m.nv))
    L = cloth_ctx(binding, m, "f32", pair_capacity=P, dhat=dhat, kappa=inputs.BARRIER_KAPPA)
    sets = []
    for step in range(3):
        pairs, xs = inputs.contact_pairs(m, m.x, step=step)
        sets.append((torch.tensor(pairs, dtype=torch.int32, device="cuda"),
                     to_dev(torch, xs, "f32")))
    out = L.alloc_outputs()
    state = {"i": 0}

    def step_fn():
        p, xx = sets[state["i"] % len(sets)]
        state["i"] += 1
        L.insert_pairs(p)
        L.eval(xx, out=out)

    r = timer.run(step_fn, args.steps, args.warmup)
    ri = timer.run(lambda: L.insert_pairs(sets[0][0]), args.steps, args.warmup)
    L.insert_pairs(sets[0][0])
    re = timer.run(lambda: L.eval(sets[0][1], out=out), args.steps, args.warmup)
    bstep = compulsory_bytes_pair_step(L, m, P)
    if L.device_status() != 0:
        raise RuntimeError("pair insertion reported a device-side error")
    L.close()
    return {"workload": f"mass-spring cloth {args.n}x{args.n} + {P} contact pairs per step, "
                        "fp32: insert, then gradient + block-CSR Hessian",
            "kernels": ["k_ins_count", "k_ins_tiles",
                        "k_eval_rows<float, false, true>", "k_eval_pair_rows<float, false>"],
            "steps": args.steps, "warmup": args.warmup,
            "step_ms_median": round(r["median_ms"], 5),
            "insert_ms_median": round(ri["median_ms"], 5),
            "eval_ms_median": round(re["median_ms"], 5),
            "step_bytes": bstep,
            "step_hbm_frac": round(bstep / (r["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def bench_terms_cloth_only(torch, inputs, args, timer):
    """The term front end's generic cloth set alone (for counter runs): its
    fused explicit evaluation, then its product, with their event timings."""
    from sparse_autodiff_mesh_amd import terms
    m = inputs.cloth(args.n)
    blocks = terms.mesh_blocks(m, "cloth")
    T = terms.Terms(m.nv, "cloth", blocks, dtype="f32")
    x = to_dev(torch, m.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(m.nv), "f32")
    y = torch.empty_like(v)
    out = T.alloc_outputs()
    re = timer.run(lambda: T.eval(x, out=out, energy=False), args.steps, args.warmup)
    rh = timer.run(lambda: T.hvp(x, v, out=y), args.steps, args.warmup)
    be = compulsory_bytes_terms(m.nv, blocks, T.nnzb, 4)
    bh = compulsory_bytes_terms(m.nv, blocks, T.nnzb, 4, hvp=True)
    T.close()
    return {"workload": f"term front end, cloth set (spring + inertia), {args.n}x{args.n}, fp32",
            "kernels": ["k_terms_eval<float, false, Spring, Inertia>",
                        "k_terms_hvp<float, false, Spring, Inertia>"],
            "steps": args.steps, "warmup": args.warmup,
            "eval_ms_mean": round(re["mean_ms"], 5), "eval_algorithmic_bytes": be,
            "hvp_ms_mean": round(rh["mean_ms"], 5), "hvp_algorithmic_bytes": bh}


def bench_secondary(torch, binding, inputs, args, timer):
    import numpy as np
    sec = {}
    steps = max(10, min(args.steps, 50))
    warm = 5
    # 100 x 100 cloth, fp32 and fp64
    m = inputs.cloth(100)
    for dt in ("f32", "f64"):
        L = cloth_ctx(binding, m, dt)
        x = to_dev(torch, m.x, dt)
        out = L.alloc_outputs()
        r = timer.run(lambda: L.eval(x, out=out), steps, warm)
        sec[f"cloth100_{dt}_eval_ms"] = round(r["median_ms"], 5)
        L.close()
    # 1000 x 1000 cloth, fp32: matrix-free HVP
    mc = inputs.cloth(args.n)
    L = cloth_ctx(binding, mc, "f32")
    xc = to_dev(torch, mc.x, "f32")
    vc = to_dev(torch, inputs.hvp_direction(mc.nv), "f32")
    yc = torch.empty_like(vc)
    r = timer.run(lambda: L.hvp(xc, vc, out=yc), steps, warm)
    bh = compulsory_bytes_hvp(mc.nv, mc.springs.shape[0], 0, 4)
    sec["cloth1000_hvp_ms"] = round(r["median_ms"], 5)
    sec["cloth1000_hvp_GBps"] = round(bh / (r["median_ms"] * 1e-3) / 1e9, 1)
    # same context, cloth displaced 0.002 h from rest (H positive definite):
    # Newton-CG direction, a fixed number of iterations per call
    zc = inputs.gaussian_block(11, mc.X.size).reshape(mc.X.shape)
    xs = to_dev(torch, mc.X + 0.002 * mc.h * zc, "f32")
    _, gs, _ = L.eval(xs)
    ps = torch.empty_like(gs)
    its = 32
    stats = {}

    def cg_fn():
        stats.update(L.newton_cg(xs, gs, out=ps, max_iters=its, eta=1e-12)[1])

    r = timer.run(cg_fn, max(5, steps // 5), 2)
    if stats["iterations"] != its:
        raise RuntimeError(f"Newton-CG stopped early: {stats}")
    bcg = compulsory_bytes_cg_iter(mc.nv, mc.springs.shape[0], 4)
    sec["cloth1000_newton_cg_iters"] = its
    sec["cloth1000_newton_cg_ms_per_iter"] = round(r["median_ms"] / its, 5)
    sec["cloth1000_newton_cg_GBps"] = round(bcg * its / (r["median_ms"] * 1e-3) / 1e9, 1)
    sec["cloth1000_newton_cg_rel_residual"] = float(f"{stats['rel_residual']:.3e}")
    # the same solve on the 100 x 100 cloth, where every kernel is short and
    # the launches per iteration dominate
    m100 = inputs.cloth(100)
    L100 = cloth_ctx(binding, m100, "f32")
    z100 = inputs.gaussian_block(11, m100.X.size).reshape(m100.X.shape)
    xs100 = to_dev(torch, m100.X + 0.002 * m100.h * z100, "f32")
    _, gs100, _ = L100.eval(xs100)
    ps100 = torch.empty_like(gs100)
    st100 = {}

    def cg100():
        st100.update(L100.newton_cg(xs100, gs100, out=ps100, max_iters=its, eta=1e-12)[1])

    r = timer.run(cg100, max(5, steps // 5), 2)
    if st100["iterations"] != its:
        raise RuntimeError(f"Newton-CG stopped early: {st100}")
    sec["cloth100_newton_cg_ms_per_iter"] = round(r["median_ms"] / its, 5)
    L100.close()
    # vector objective on the 1000 x 1000 context: residuals + explicit
    # sparse Jacobian, and the matrix-free Gauss-Newton product
    R, Jv = L.residual_jacobian(xc)
    r = timer.run(lambda: L.residual_jacobian(xc, out=(R, Jv)), steps, warm)
    bj = compulsory_bytes_residual_jacobian(mc.nv, mc.springs.shape[0], 4)
    sec["cloth1000_residual_jacobian_ms"] = round(r["median_ms"], 5)
    sec["cloth1000_residual_jacobian_GBps"] = round(bj / (r["median_ms"] * 1e-3) / 1e9, 1)
    r = timer.run(lambda: L.gauss_newton(xc, vc, out=yc), steps, warm)
    sec["cloth1000_gauss_newton_ms"] = round(r["median_ms"], 5)
    sec["cloth1000_gauss_newton_GBps"] = round(bh / (r["median_ms"] * 1e-3) / 1e9, 1)
    L.close()
    # 512 x 512 symmetric-Dirichlet face grid, fp32: the explicit eval kernel
    # (no energy sum: one launch per call, as the headline's kernel timing)
    # and the HVP
    f = inputs.face_grid(512)
    L = binding.Lad(f.nv, dtype="f32",
                    **binding.mesh_terms(f, springs=False, inertia=False, faces=True))
    info = L.get_info()
    x = to_dev(torch, f.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(f.nv), "f32")
    out = L.alloc_outputs()
    r = timer.run(lambda: L.eval(x, out=out, energy=False), steps, warm)
    nf = f.faces.shape[0]
    bc = compulsory_bytes_eval(f.nv, 0, nf, info["nnzb_base"], 4, inertia=False, faces=True)
    sec["faces512_eval_ms"] = round(r["median_ms"], 5)
    sec["faces512_eval_Mfaces_per_s"] = round(nf / (r["median_ms"] * 1e-3) / 1e6, 2)
    sec["faces512_eval_GBps"] = round(bc / (r["median_ms"] * 1e-3) / 1e9, 1)
    y = torch.empty_like(v)
    r = timer.run(lambda: L.hvp(x, v, out=y), steps, warm)
    bh = compulsory_bytes_hvp(f.nv, 0, nf, 4, faces=True)
    sec["faces512_hvp_ms"] = round(r["median_ms"], 5)
    sec["faces512_hvp_GBps"] = round(bh / (r["median_ms"] * 1e-3) / 1e9, 1)
    sec["faces512_eval_hbm_frac"] = round(sec["faces512_eval_GBps"] / HBM_PEAK_GBPS, 4)
    sec["faces512_hvp_hbm_frac"] = round(sec["faces512_hvp_GBps"] / HBM_PEAK_GBPS, 4)
    # VALU-busy of the same kernels from the committed counter summary
    # (null when the kernel sources changed since it was taken)
    sec["faces512_eval_valu_busy"] = read_valu_busy(FACES_FILE, "k_eval_face_rows<float>")
    sec["faces512_hvp_valu_busy"] = read_valu_busy(FACES_FILE, "k_hvp_rows<float, true, false>")
    L.close()
    # 1000 x 1000 cloth + 2 % contact pairs per step, fp32: insert + eval
    m = inputs.cloth(args.n)
    dhat = 0.5 * m.h
    P = int(round(0.02 * m.nv))
    L = cloth_ctx(binding, m, "f32", pair_capacity=P, dhat=dhat, kappa=inputs.BARRIER_KAPPA)
    sets = []
    for step in range(3):
        pairs, xs = inputs.contact_pairs(m, m.x, step=step)
        sets.append((torch.tensor(pairs, dtype=torch.int32, device="cuda"),
                     to_dev(torch, xs, "f32")))
    out = L.alloc_outputs()
    vdir = to_dev(torch, inputs.hvp_direction(m.nv), "f32")
    yv = torch.empty_like(vdir)
    state = {"i": 0}

    def step_fn():
        p, xx = sets[state["i"] % len(sets)]
        state["i"] += 1
        L.insert_pairs(p)
        L.eval(xx, out=out)

    r = timer.run(step_fn, steps, warm)
    sec["cloth1000_pairs_insert_eval_ms"] = round(r["median_ms"], 5)
    bstep = compulsory_bytes_pair_step(L, m, P)
    sec["cloth1000_pairs_step_bytes"] = bstep
    sec["cloth1000_pairs_step_hbm_frac"] = round(
        bstep / (r["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    rh = timer.run(lambda: L.hvp(sets[0][1], vdir, out=yv), steps, warm)
    sec["cloth1000_pairs_hvp_ms"] = round(rh["median_ms"], 5)
    ri = timer.run(lambda: L.insert_pairs(sets[0][0]), steps, warm)
    sec["cloth1000_pairs_insert_ms"] = round(ri["median_ms"], 5)
    if L.device_status() != 0:
        raise RuntimeError("pair insertion reported a device-side error")
    L.close()
    sec["pairs_per_step"] = P
    # the same cloth + 2 % vertex-face contacts per step, fp32
    L = binding.Lad(m.nv, dtype="f32",
                    **binding.mesh_terms(m, vf_capacity=P, dhat=dhat, kappa=inputs.BARRIER_KAPPA))
    sets = []
    for step in range(3):
        vf, xs = inputs.vf_contacts(m, m.x, step, dhat=dhat)
        sets.append((torch.tensor(vf, dtype=torch.int32, device="cuda"), to_dev(torch, xs, "f32")))
    out = L.alloc_outputs()
    state = {"i": 0}

    def vf_step():
        c, xx = sets[state["i"] % len(sets)]
        state["i"] += 1
        L.insert_contacts(vf=c)
        L.eval(xx, out=out)

    r = timer.run(vf_step, steps, warm)
    sec["cloth1000_vf_insert_eval_ms"] = round(r["median_ms"], 5)
    rh = timer.run(lambda: L.hvp(sets[0][1], vdir, out=yv), steps, warm)
    sec["cloth1000_vf_hvp_ms"] = round(rh["median_ms"], 5)
    ri = timer.run(lambda: L.insert_contacts(vf=sets[0][0]), steps, warm)
    sec["cloth1000_vf_insert_ms"] = round(ri["median_ms"], 5)
    if L.device_status() != 0:
        raise RuntimeError("contact insertion reported a device-side error")
    L.close()
    sec["vf_contacts_per_step"] = P
    sec.update(bench_terms(torch, inputs, args, timer, steps, warm))
    sec.update(bench_patch_path(torch, binding, inputs, args, timer, steps, warm))
    return sec


def bench_patch_path(torch, binding, inputs, args, timer, steps, warm):
    """The element-owner patch path on the headline cloth and the face grid,
    for comparison with the row path: LDS patches with ghost vertices, the
    owned rows accumulated in LDS in colour phases (cloth1000_patch, the
    default assembly), with LDS atomics (_patch_lds_atomic), or with each
    element evaluated once and its blocks in other patches' rows added by
    global float atomics into slots zeroed by a small launch first
    (_patch_atomic: the pages' own assembly).  Times are whole calls (the
    zeroing launch included)."""
    sec = {}
    m = inputs.cloth(args.n)
    x = to_dev(torch, m.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(m.nv), "f32")
    y = torch.empty_like(v)
    for path, tag in (("patch", "cloth1000_patch"),
                      ("patch_lds_atomic", "cloth1000_patch_lds_atomic"),
                      ("patch_atomic", "cloth1000_patch_atomic")):
        L = binding.Lad(m.nv, dtype="f32", path=path, **binding.mesh_terms(m))
        out = L.alloc_outputs()
        r = timer.run(lambda: L.eval(x, out=out, energy=False), steps, warm)
        info = L.get_info()
        nnzb = info["nnzb_base"]
        sec[tag + "_eval_ms"] = round(r["median_ms"], 5)
        sec[tag + "_eval_GBps"] = round(
            compulsory_bytes_eval(m.nv, m.springs.shape[0], 0, nnzb, 4) /
            (r["median_ms"] * 1e-3) / 1e9, 1)
        sec[tag + "_spring_records"] = info["spring_records"]
        rh = timer.run(lambda: L.hvp(x, v, out=y), steps, warm)
        sec[tag + "_hvp_ms"] = round(rh["median_ms"], 5)
        L.close()
    f = inputs.face_grid(512)
    xf = to_dev(torch, f.x, "f32")
    for path, tag in (("patch", "faces512_patch"), ("patch_lds_atomic", "faces512_patch_lds_atomic"),
                      ("patch_atomic", "faces512_patch_atomic")):
        L = binding.Lad(f.nv, dtype="f32", path=path,
                        **binding.mesh_terms(f, springs=False, inertia=False, faces=True))
        out = L.alloc_outputs()
        r = timer.run(lambda: L.eval(xf, out=out, energy=False), steps, warm)
        sec[tag + "_eval_ms"] = round(r["median_ms"], 5)
        sec[tag + "_face_records"] = L.get_info()["face_records"]
        L.close()
    return sec


def bench_terms(torch, inputs, args, timer, steps, warm):
    """The term front end: ARAP faces on the 512 x 512 grid, the generic
    cloth set at 1000 x 1000 (the same energy as the headline kernel), and
    ARAP + cloth fused into one launch against one launch per term."""
    from sparse_autodiff_mesh_amd import terms
    sec = {}
    f = inputs.face_grid(512)
    blocks = terms.mesh_blocks(f, "arap")
    T = terms.Terms(f.nv, "arap", blocks, dtype="f32")
    x = to_dev(torch, f.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(f.nv), "f32")
    out = T.alloc_outputs()
    r = timer.run(lambda: T.eval(x, out=out, energy=False), steps, warm)
    b = compulsory_bytes_terms(f.nv, blocks, T.nnzb, 4)
    sec["terms_arap512_eval_ms"] = round(r["median_ms"], 5)
    sec["terms_arap512_eval_GBps"] = round(b / (r["median_ms"] * 1e-3) / 1e9, 1)
    y = torch.empty_like(v)
    r = timer.run(lambda: T.hvp(x, v, out=y), steps, warm)
    sec["terms_arap512_hvp_ms"] = round(r["median_ms"], 5)
    sec["terms_arap512_hvp_GBps"] = round(
        compulsory_bytes_terms(f.nv, blocks, T.nnzb, 4, hvp=True) / (r["median_ms"] * 1e-3) / 1e9, 1)
    T.close()
    m = inputs.cloth(args.n)
    x = to_dev(torch, m.x, "f32")
    v = to_dev(torch, inputs.hvp_direction(m.nv), "f32")
    y = torch.empty_like(v)
    for set_id in ("cloth", "arap_cloth"):
        blocks = terms.mesh_blocks(m, set_id)
        for fused in (True, False):
            if set_id == "cloth" and not fused:
                continue
            T = terms.Terms(m.nv, set_id, blocks, dtype="f32", fused=fused)
            out = T.alloc_outputs()
            r = timer.run(lambda: T.eval(x, out=out, energy=False), steps, warm)
            tag = f"terms_{set_id}1000_{'fused' if fused else 'unfused'}"
            sec[tag + "_eval_ms"] = round(r["median_ms"], 5)
            sec[tag + "_eval_GBps"] = round(
                compulsory_bytes_terms(m.nv, blocks, T.nnzb, 4) / (r["median_ms"] * 1e-3) / 1e9, 1)
            r = timer.run(lambda: T.hvp(x, v, out=y), steps, warm)
            sec[tag + "_hvp_ms"] = round(r["median_ms"], 5)
            T.close()
    return sec


CPU_SAMPLE_SECONDS = 10.0   # CPU work the baseline leg spends (bounded)


def cpu_baseline(inputs, res):
    """The fp64 oracle, single-threaded, on the same 1000 x 1000 cloth (inputs
    rounded to fp32 as the GPU sees them): full evaluations repeated until
    about CPU_SAMPLE_SECONDS of work (at most 100), the median one reported;
    the pattern is built beforehand and not timed."""
    import statistics
    import oracle
    m = res["mesh"]
    prob = oracle.problem_from_mesh(m, f32=True)
    t0 = time.perf_counter()
    rp, ci = oracle.pattern(prob)
    t_pat = time.perf_counter() - t0
    x = inputs.round_f32(m.x)
    times = []
    E = None
    while sum(times) < CPU_SAMPLE_SECONDS and len(times) < 100:
        t0 = time.perf_counter()
        E, _, _ = oracle.evaluate(prob, rp, ci, x)
        times.append(time.perf_counter() - t0)
    t_eval = statistics.median(times)
    rel_e = abs(E - res["energy"]) / abs(E)
    return {
        "value": round(res["terms"] / t_eval / 1e6, 4),
        "unit": "Melem/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(times)} full evaluations of the {m.n}x{m.n} cloth "
                   f"({res['terms']} terms) in {sum(times):.1f} s, fp64, single thread, "
                   f"median reported; pattern build {t_pat:.2f} s untimed"),
        "ms_per_eval": round(t_eval * 1e3, 1),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "energy_rel_diff_vs_gpu": float(f"{rel_e:.3e}"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--n", type=int, default=1000, help="cloth grid side (vertices)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--flush-mall", action="store_true",
                    help="write a 512 MB scratch buffer before every timed call")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "rows", "patch", "patch_atomic", "patch_lds_atomic"],
                    help="decomposition of the headline evaluation (auto picks rows)")
    ap.add_argument("--deterministic", action="store_true",
                    help="ask the library for bitwise reproducible results (the atomic "
                         "patch assemblies reject it)")
    ap.add_argument("--patch-lds", type=int, default=0,
                    help="LDS bytes per patch (0 = library default)")
    ap.add_argument("--hvp-only", action="store_true",
                    help="only time the cloth HVP (prints its own JSON line; for counter runs)")
    ap.add_argument("--faces-only", action="store_true",
                    help="only time the 512x512 face grid, eval kernel then HVP (prints its "
                         "own JSON line; for counter runs)")
    ap.add_argument("--pairs-only", action="store_true",
                    help="time only the cloth step with contact pairs (for traces and counters)")
    ap.add_argument("--terms-cloth-only", action="store_true",
                    help="only time the term front end's cloth set, eval then HVP (prints "
                         "its own JSON line; for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a device-to-device copy of 256 MiB five times "
                         "(reference kernel for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not "
              "supported (sharding over several GPUs is designed, not implemented)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        nbytes = 256 * 1024 * 1024
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": nbytes,
                          "calibrate_copy_bytes_written": nbytes, "launches": 5}))
        return 0
    from sparse_autodiff_mesh_amd import binding, inputs
    binding.lib()  # fails loudly if liblad.so is missing

    timer = Timer(torch)
    if args.hvp_only:
        print(json.dumps(bench_hvp_only(torch, binding, inputs, args, timer)))
        return 0
    if args.faces_only:
        print(json.dumps(bench_faces_only(torch, binding, inputs, args, timer)))
        return 0
    if args.terms_cloth_only:
        print(json.dumps(bench_terms_cloth_only(torch, inputs, args, timer)))
        return 0
    if args.pairs_only:
        print(json.dumps(bench_pairs_only(torch, binding, inputs, args, timer)))
        return 0
    log(f"bench: cloth {args.n}x{args.n} fp32, steps={args.steps} warmup={args.warmup}")
    res = bench_headline(torch, binding, inputs, args, timer)
    t = res["timing"]
    tk = res["timing_kernel"]
    ms = t["region_ms"] / args.steps
    kern_ms = tk["mean_ms"]
    melem = res["terms"] / (ms * 1e-3) / 1e6
    achieved = res["bytes"] / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic() if res["info"]["eval_path"] == 2 else None
    line = {
        "metric": "grad+Hessian ms/eval & Melem/s on 1000² cloth (1 GPU); "
                  "achieved HBM GB/s vs peak",
        "value": round(melem, 3),
        "unit": "Melem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"mass-spring cloth {args.n}x{args.n} vertices, fp32, "
                        "springs k=1e3 + inertia m/dt^2=100, gradient + block-CSR Hessian",
            "vertices": res["nv"], "springs": res["ns"], "terms": res["terms"],
            "nnzb": res["nnzb"], "chunks_or_patches": res["info"]["npatches"],
            "eval_path": {1: "patch", 2: "rows", 3: "patch_atomic",
                          4: "patch_lds_atomic"}.get(res["info"]["eval_path"], "?"),
            "workgroups": res["info"]["grid_eval"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": {2: "k_eval_rows<float>",
                       3: "k_zero_boundary<float> + k_eval_patch<float, 2>",
                       4: "k_eval_patch<float, 0>"}.get(res["info"]["eval_path"],
                                                        "k_eval_patch<float, 1>"),
            "kernel_ms_mean": round(kern_ms, 5),
            "kernel_ms_median": round(tk["median_ms"], 5),
            "call_ms_mean_with_energy": round(t["mean_ms"], 5),
            "algorithmic_bytes": res["bytes"],
            "flush_mall": bool(args.flush_mall),
            "kernel_ms_mean_mall_flushed": (round(res["timing_flushed"]["mean_ms"], 5)
                                            if res["timing_flushed"] else None),
            # the same kernel with its inputs evicted from the last-level
            # cache first (a read-only 512 MB sweep before every call)
            "frac_mall_flushed": (round(res["bytes"] / (res["timing_flushed"]["mean_ms"] * 1e-3)
                                        / 1e9 / HBM_PEAK_GBPS, 4)
                                  if res["timing_flushed"] else None),
            "copy_GBps_measured": (round(res["copy_gbps"], 1) if res["copy_gbps"] else None),
            "fill_GBps_measured": (round(res["fill_gbps"], 1) if res["fill_gbps"] else None),
        },
        # initialisation (untimed above): the GPU pattern build (HIP events
        # around its launches) and the whole context build (host patching,
        # uploads and the pattern, wall clock)
        "init": {"pattern_gpu_ms": round(res["info"]["pattern_ms"], 3),
                 "context_build_ms": round(res["init_s"] * 1e3, 1)},
        "springs_per_s_M": round(res["ns"] / (ms * 1e-3) / 1e6, 2),
        "energy": res["energy"],
    }
    if not args.no_secondary:
        log("bench: secondary workloads")
        line["secondary"] = bench_secondary(torch, binding, inputs, args, timer)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(inputs, res)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
