"""The oracle's element routines against the hand-derived worked values in
tests/golden/element_values.txt (closed forms evaluated by hand; each case
carries its derivation in the file)."""
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def cases():
    out = []
    with open(os.path.join(HERE, "golden", "element_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, args, e, g = [t.strip() for t in line.split("|")]
            out.append((kind, args, float(e), np.array([float(v) for v in g.split()])))
    return out


def parse_args(args):
    vecs, params = [], {}
    for part in args.split(";"):
        toks = part.split()
        if toks[0].isalpha() or toks[0] in ("dminv",):
            params[toks[0]] = [float(t) for t in toks[1:]]
        else:
            vecs.append(np.array([float(t) for t in toks]))
    return vecs, params


@pytest.mark.parametrize("kind,args,e,g", cases())
def test_golden_element(kind, args, e, g):
    vecs, p = parse_args(args)
    if kind == "spring":
        E, gg, _ = oracle.spring_local(vecs[0], vecs[1], p["rest"][0], p["k"][0])
    elif kind == "inertia":
        E, gg, _ = oracle.inertia_local(vecs[0], vecs[1], p["c"][0])
    elif kind == "barrier":
        E, gg, _ = oracle.barrier_local(vecs[0], vecs[1], p["kappa"][0], p["dhat"][0])
    elif kind == "face":
        E, gg, _ = oracle.face_local(vecs[0], vecs[1], vecs[2], p["dminv"], p["area"][0])
    else:
        raise AssertionError(kind)
    assert E == pytest.approx(e, rel=1e-13, abs=1e-13)
    assert np.allclose(gg, g, rtol=1e-12, atol=1e-12)


def test_golden_file_has_every_kind():
    kinds = {c[0] for c in cases()}
    assert kinds == {"spring", "inertia", "barrier", "face"}
