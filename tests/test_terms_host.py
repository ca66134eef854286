"""The term front end's C ABI without a GPU: every entry point that
include/lad_terms.h declares is exported, the compiled sets describe
themselves, and bad descriptors are rejected on the host before any GPU
work (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_autodiff_mesh_amd import binding, inputs, terms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lad_terms.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("liblad.so not built")
    return terms.lib()


def test_exports_match_header(L):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(lad_terms_[a-z_]+)\s*\(", text)))
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"{n} declared in lad_terms.h but not exported"
    assert set(names) == set(terms.TERMS_EXPORTS)


def test_sets_describe_their_terms(L):
    assert terms.describe("cloth") == [("spring", 2, 2), ("inertia", 1, 4)]
    assert terms.describe("arap") == [("arap_face", 3, 5)]
    assert terms.describe("symdir") == [("symmetric_dirichlet_face", 3, 5)]
    assert terms.describe("arap_cloth") == [("arap_face", 3, 5), ("spring", 2, 2),
                                            ("inertia", 1, 4)]
    assert terms.describe("cloth_quad") == [("spring", 2, 2), ("inertia", 1, 4),
                                            ("quad_planarity", 4, 1)]
    with pytest.raises(binding.LadError):
        terms.describe(99)
    n, ar = ctypes.c_int32(), ctypes.c_int32()
    assert L.lad_terms_describe(2, 1, ctypes.byref(n), ctypes.byref(ar), None, None) == \
        binding.LAD_ERR_ARG


def build_status(desc):
    out = ctypes.c_void_p()
    st = terms.lib().lad_terms_build(ctypes.byref(desc) if desc is not None else None, None,
                                     ctypes.byref(out))
    return st, terms.lib().lad_terms_last_error(None).decode(), out


def mesh_desc(set_id="arap_cloth", **kw):
    m = inputs.cloth(4)
    blocks = [list(b) for b in terms.mesh_blocks(m, set_id)]
    return m, blocks


@pytest.mark.parametrize("mutate,msg", [
    (lambda m, b, d: setattr(d, "nv", 0), "nv must be"),
    (lambda m, b, d: setattr(d, "dtype", 7), "dtype"),
    (lambda m, b, d: setattr(d, "set", 42), "unknown term set"),
    (lambda m, b, d: setattr(d, "fused", 2), "fused"),
    (lambda m, b, d: setattr(d, "nblocks", 2), "nblocks must be 3"),
])
def test_bad_descriptor_fields(L, mutate, msg):
    m, blocks = mesh_desc()
    d, keep = terms.make_desc(m.nv, "arap_cloth", blocks)
    mutate(m, blocks, d)
    st, err, out = build_status(d)
    assert st == binding.LAD_ERR_ARG and msg in err and not out.value


@pytest.mark.parametrize("which,fix,msg", [
    (0, lambda el, cs: el.__setitem__((3, 1), 10_000), "vertex id out of range"),
    (0, lambda el, cs: el.__setitem__((2, 2), el[2, 0]), "repeats a vertex"),
    (1, lambda el, cs: el.__setitem__((0, 0), -1), "vertex id out of range"),
    (1, lambda el, cs: cs.__setitem__((4, 0), np.nan), "non-finite constant"),
    (2, lambda el, cs: cs.__setitem__((1, 3), np.inf), "non-finite constant"),
])
def test_bad_elements(L, which, fix, msg):
    m, blocks = mesh_desc()
    el, cs = (np.array(a, copy=True) for a in blocks[which])
    fix(el, cs)
    blocks[which] = (el, cs)
    d, keep = terms.make_desc(m.nv, "arap_cloth", blocks)
    st, err, out = build_status(d)
    assert st == binding.LAD_ERR_ARG and msg in err and not out.value


def test_null_arguments(L):
    st, err, _ = build_status(None)
    assert st == binding.LAD_ERR_ARG and "NULL" in err
    m, blocks = mesh_desc("arap")
    d, keep = terms.make_desc(m.nv, "arap", blocks)
    d.blocks = None
    st, err, _ = build_status(d)
    assert st == binding.LAD_ERR_ARG and "blocks is NULL" in err
    blk = terms.lad_term_block()
    blk.count = 3
    d.blocks = ctypes.pointer(blk)
    st, err, _ = build_status(d)
    assert st == binding.LAD_ERR_ARG and "elems is NULL" in err
    assert L.lad_terms_eval(None, None, None, None, None, 0, None) == binding.LAD_ERR_ARG
    assert L.lad_terms_hvp(None, None, None, None, None) == binding.LAD_ERR_ARG
    assert L.lad_terms_get_pattern(None, None, None, None) == binding.LAD_ERR_ARG
    L.lad_terms_destroy(None)
