"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/pctree.h declares, and rejects bad arguments on the host before
anything is enqueued (no GPU is touched)."""
import ctypes as C
import os
import re

import pytest

import draft_tree_construction_markov_amd as pct

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "include", "pctree.h")


def declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pct_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pct.lib()
    names = declared()
    assert "pct_build_tree" in names and "pct_verify_accept" in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(pct.exported_symbols()) == names


def test_status_strings():
    lib = pct.lib()
    for s in range(5):
        assert lib.pct_status_string(s)


def _shape(**kw):
    d = dict(batch=1, B=4, V=1000, r=16, k=4, beam_w=4, N=16, uw_dtype=0)
    d.update(kw)
    return pct.TreeShape(**d)


@pytest.mark.parametrize("bad", [dict(k=0), dict(k=2000), dict(V=1 << 18),
                                 dict(B=0), dict(B=65), dict(N=0),
                                 dict(batch=0), dict(k=65), dict(uw_dtype=7)])
def test_build_tree_rejects_bad_shapes(bad):
    lib = pct.lib()
    sh = _shape(**bad)
    assert lib.pct_build_tree_workspace(C.byref(sh)) == 0
    dummy = C.c_void_p(16)
    rc = lib.pct_build_tree(C.byref(sh), dummy, None, None, dummy, dummy,
                            dummy, dummy, dummy, dummy, None, dummy, 1 << 30,
                            None)
    assert rc in (1, 2)
    assert lib.pct_last_error()


def test_build_tree_rejects_null_and_small_workspace():
    lib = pct.lib()
    sh = _shape()
    need = lib.pct_build_tree_workspace(C.byref(sh))
    assert need > 0
    d = C.c_void_p(16)
    assert lib.pct_build_tree(C.byref(sh), None, None, None, d, d, d, d, d,
                              d, None, d, need, None) == 1
    # only one of the two factors
    assert lib.pct_build_tree(C.byref(sh), d, d, None, d, d, d, d, d, d,
                              None, d, need, None) == 1
    assert lib.pct_build_tree(C.byref(sh), d, d, d, d, d, d, d, d, d,
                              None, d, need - 1, None) == 3


def test_pool_too_large_is_unsupported():
    lib = pct.lib()
    sh = _shape(B=40, k=64, beam_w=64, V=5000)
    assert lib.pct_build_tree_workspace(C.byref(sh)) == 0
    d = C.c_void_p(16)
    assert lib.pct_build_tree(C.byref(sh), d, None, None, d, d, d, d, d, d,
                              None, d, 1 << 40, None) == 2


def test_adaptive_rejects_bad_arguments():
    lib = pct.lib()
    d = C.c_void_p(16)
    assert lib.pct_build_tree_adaptive_workspace(1, 2, 100, 2000) == 0
    assert lib.pct_build_tree_adaptive_workspace(1, 2, 100, 64) > 0
    bad = pct.CostModel(1.0, 2.0, 0.004, -1e-6, 1e-5)
    rc = lib.pct_build_tree_adaptive(1, 2, 100, 64, d, d, C.byref(bad), d, d,
                                     d, d, d, d, d, None, d, 1 << 30, None)
    assert rc == 1
    zero = pct.CostModel(0.0, 0.0, 0.0, 0.0, 0.0)
    rc = lib.pct_build_tree_adaptive(1, 2, 100, 64, d, d, C.byref(zero), d, d,
                                     d, d, d, d, d, None, d, 1 << 30, None)
    assert rc == 1


def test_verify_and_mask_reject_bad_arguments():
    lib = pct.lib()
    d = C.c_void_p(16)
    assert lib.pct_verify_accept(0, 4, 2, d, d, d, d, None, d, d, d, d,
                                 None) == 1
    assert lib.pct_verify_accept(1, 9000, 2, d, d, d, d, d, d, d, d, d,
                                 None) == 1
    # the mask is optional; the target is not
    assert lib.pct_verify_accept(1, 4, 2, d, d, d, d, d, None, d, d, d,
                                 None) == 1
    assert lib.pct_tree_mask(1, 0, d, d, d, None) == 1
    assert lib.pct_tree_mask(1, 4, None, d, d, None) == 1


def test_markov_logits_rejects_bad_arguments():
    lib = pct.lib()
    d = C.c_void_p(16)
    # k > V
    assert lib.pct_markov_logits(d, 100, 1, d, d, 1, 100, 32, d, d, 4, 101, d,
                                 d, d, None, d, 1 << 30, None) == 1
    # L stride below V
    assert lib.pct_markov_logits(d, 50, 1, d, d, 1, 100, 32, d, d, 4, 8, d,
                                 d, d, None, d, 1 << 30, None) == 1
    # workspace too small
    assert lib.pct_markov_logits(d, 100, 1, d, d, 1, 100, 32, d, d, 4, 8, d,
                                 d, d, None, d, 16, None) == 3


def test_build_tree_rejects_unaligned_factors():
    # a factor view at an element offset would feed misaligned 16-byte
    # loads to the kernels: rejected on the host, nothing enqueued
    lib = pct.lib()
    sh = _shape(r=32, uw_dtype=1)
    need = lib.pct_build_tree_workspace(C.byref(sh))
    d = C.c_void_p(256)
    odd = C.c_void_p(256 + 2)
    for U, W in ((odd, d), (d, odd)):
        rc = lib.pct_build_tree(C.byref(sh), d, U, W, d, d, d, d, d, d, None,
                                d, need, None)
        assert rc == 1
        assert b"aligned" in lib.pct_last_error()


def test_adaptive_pc_and_curve_reject_bad_arguments():
    lib = pct.lib()
    d = C.c_void_p(256)
    sh = _shape(r=32, uw_dtype=1, N=16)
    need = lib.pct_build_tree_adaptive_pc_workspace(C.byref(sh))
    assert need == lib.pct_build_tree_workspace(C.byref(sh)) > 0
    bad = pct.CostModel(1.0, 2.0, -0.004, 0.0, 1e-5)
    rc = lib.pct_build_tree_adaptive_pc(C.byref(sh), d, d, d, d, d,
                                        C.byref(bad), d, d, d, d, d, d, d,
                                        None, d, need, None)
    assert rc == 1
    good = pct.CostModel(1.0, 2.0, 0.004, 0.0, 1e-5)
    # ctx_len is required with a cost model
    rc = lib.pct_build_tree_adaptive_pc(C.byref(sh), d, d, d, d, None,
                                        C.byref(good), d, d, d, d, d, d, d,
                                        None, d, need, None)
    assert rc == 1
    assert lib.pct_throughput_curve(0, 4, d, d, d, None, d, None) == 1
    assert lib.pct_throughput_curve(1, 4, d, None, d, None, d, None) == 1
    assert lib.pct_throughput_curve(1, 4, d, d, d, C.byref(bad), d,
                                    None) == 1


def test_verify_sample_rejects_bad_arguments():
    lib = pct.lib()
    d = C.c_void_p(256)
    args = [d] * 4
    assert lib.pct_verify_sample(1, 4, 2, 100, *args, None, d, 0.0, 1, d, d,
                                 d, d, None, 0, None) == 1
    assert lib.pct_verify_sample(1, 4, 2, 100, *args, None, d, float("inf"),
                                 1, d, d, d, d, None, 0, None) == 1
    assert lib.pct_verify_sample(1, 4, 2, 0, *args, None, d, 1.0, 1, d, d, d,
                                 d, None, 0, None) == 1
    assert lib.pct_verify_sample(1, 4, 2, 100, *args, None, None, 1.0, 1, d,
                                 d, d, d, None, 0, None) == 1
    assert lib.pct_verify_sample(70000, 4, 2, 100, *args, None, d, 1.0, 1, d,
                                 d, d, d, None, 0, None) == 2


def test_verify_sample_workspace():
    lib = pct.lib()
    # few rows of a large vocabulary: rows are cut into slices whose
    # partial results need a workspace; a missing one is an error
    need = lib.pct_verify_sample_workspace(1, 64, 151936)
    assert need > 0
    d = C.c_void_p(256)
    args = [d] * 4
    assert lib.pct_verify_sample(1, 64, 7, 151936, *args, None, d, 1.0, 1, d,
                                 d, d, d, None, 0, None) == 3
    assert lib.pct_verify_sample(1, 64, 7, 151936, *args, None, d, 1.0, 1, d,
                                 d, d, d, d, need - 1, None) == 3
    # many rows, or a short vocabulary: one workgroup per row, no workspace
    assert lib.pct_verify_sample_workspace(32, 256, 151936) == 0
    assert lib.pct_verify_sample_workspace(1, 64, 1000) == 0
    assert lib.pct_verify_sample_workspace(0, 64, 1000) == 0
