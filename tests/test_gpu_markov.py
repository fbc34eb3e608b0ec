"""GPU parity of the fused Markov-logit kernel (pct_markov_logits) against
the CPU oracle: exact small-integer contractions, random bf16 factors within
the 2e-2 relative bound, and per-parent lse / top-k."""
import math

import numpy as np
import pytest
import torch

import draft_tree_construction_markov_amd as pct
import oracle
import synth
from gpu_util import announce, dev_f32, dev_factors, dev_i32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,r,P", [(300, 32, 5), (1000, 256, 40),
                                   (4160, 128, 300), (777, 64, 33)])
def test_integer_factors_are_exact(V, r, P):
    # Small integers: every product and partial sum is an exact fp32 integer,
    # so the MFMA contraction must equal the exact integer dot product.
    announce("markov integer", V, r, P)
    rng = np.random.default_rng(V + r)
    Ui = rng.integers(-3, 4, size=(V, r))
    Wi = rng.integers(-3, 4, size=(V, r))
    U = synth.bf16_bits(Ui.astype(np.float32))
    W = synth.bf16_bits(Wi.astype(np.float32))
    toks = rng.integers(0, V, size=P).astype(np.int32)
    dU, dW = dev_factors(U, W)
    lse, tt, tl, z = pct.markov_logits(None, dU, dW, dev_i32(toks), None, 4,
                                       want_z=True)
    z = z.cpu().numpy()
    want = (Ui[toks].astype(np.int64) @ Wi.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(z, want)


@pytest.mark.parametrize("bf16", [True, False])
def test_random_factors_within_bound(bf16):
    V, r, P = 5000, 256 if bf16 else 48, 70
    announce("markov random", bf16)
    U, W = synth.markov_factors(17, V, r, bf16)
    rng = np.random.default_rng(3)
    toks = rng.integers(0, V, size=P).astype(np.int32)
    dU, dW = dev_factors(U, W)
    _, _, _, z = pct.markov_logits(None, dU, dW, dev_i32(toks), None, 8,
                                   want_z=True)
    z = z.cpu().numpy()
    worst = 0.0
    for p in range(P):
        ref = oracle.markov_row(U, W, int(toks[p]))
        err = np.abs(z[p] - ref).max() / np.abs(ref).max()
        worst = max(worst, err)
        assert err <= 2e-2
    print(f"max relative error {worst:.3e}")
    assert worst < 1e-5  # fp32 accumulation of exact products


@pytest.mark.parametrize("V,r,k", [(151936, 256, 8), (3000, 256, 16),
                                   (1000, 16, 4)])
def test_lse_and_topk_match_oracle(V, r, k):
    announce("markov stats", V, r, k)
    bf16 = r % 16 == 0 and r >= 32
    U, W = synth.markov_factors(23, V, r, bf16)
    rows = 3
    L = synth.drafter_logits(23, 1, rows, V, 3.0, (0.5, 2.0))[0]
    rng = np.random.default_rng(5)
    P = 24
    toks = rng.integers(0, V, size=P).astype(np.int32)
    lrow = rng.integers(0, rows, size=P).astype(np.int32)
    dU, dW = dev_factors(U, W)
    lse, tt, tl, _ = pct.markov_logits(dev_f32(L), dU, dW, dev_i32(toks),
                                       dev_i32(lrow), k)
    lse, tt, tl = lse.cpu().numpy(), tt.cpu().numpy(), tl.cpu().numpy()
    exact = near = 0
    for p in range(P):
        M = oracle.markov_row(U, W, int(toks[p]))
        ol, ot, oz, gap = oracle.row_stats(L[lrow[p]], M, k)
        assert abs(lse[p] - ol) <= 1e-5 * max(1.0, abs(ol))
        olp = (oz - np.float32(ol)).astype(np.float32)
        if np.array_equal(tt[p], ot):
            exact += 1
            assert np.abs(tl[p] - olp).max() <= 1e-4
        else:
            assert gap < 1e-5, (p, tt[p], ot)
            near += 1
    print(f"exact {exact} near-tie {near}")


@pytest.mark.parametrize("r,k,P", [(32, 24, 512), (256, 24, 512),
                                   (256, 20, 640), (64, 40, 300),
                                   (128, 64, 70)])
def test_long_lists_across_ranks_and_parent_counts(r, k, P):
    # long per-parent lists change the kernel's shape (parents per wave,
    # waves per workgroup, vocabulary slices), and the shape depends on r
    # through the LDS it needs; the workspace query must cover each of them
    announce("markov long lists", r, k, P)
    V = 20000
    U, W = synth.markov_factors(31 + r, V, r, True)
    rows = 5
    L = synth.drafter_logits(31, 1, rows, V, 3.0, (0.5, 2.0))[0]
    rng = np.random.default_rng(k + P)
    toks = rng.integers(0, V, size=P).astype(np.int32)
    lrow = rng.integers(0, rows, size=P).astype(np.int32)
    dU, dW = dev_factors(U, W)
    lse, tt, tl, _ = pct.markov_logits(dev_f32(L), dU, dW, dev_i32(toks),
                                       dev_i32(lrow), k)
    lse, tt, tl = lse.cpu().numpy(), tt.cpu().numpy(), tl.cpu().numpy()
    near = 0
    for p in range(0, P, 7):
        M = oracle.markov_row(U, W, int(toks[p]))
        ol, ot, oz, gap = oracle.row_stats(L[lrow[p]], M, k)
        assert abs(lse[p] - ol) <= 1e-5 * max(1.0, abs(ol))
        if np.array_equal(tt[p], ot):
            olp = (oz - np.float32(ol)).astype(np.float32)
            assert np.abs(tl[p] - olp).max() <= 1e-4
        else:
            assert gap < 1e-5, (p, tt[p], ot)
            near += 1
    assert near <= 2


@pytest.mark.parametrize("V,r,P,k", [(2003, 128, 17, 12), (3000, 256, 32, 30),
                                     (640, 32, 1, 4)])
def test_thin_form_small_frontiers(V, r, P, k):
    # at most 32 parents take the thin form (every wave its own 32-row
    # pieces): a ragged last piece with V % 4 != 0 (scalar L reads), a full
    # block of 32 parents with long lists, a single parent; the logits it
    # writes, the log-normalisers and the top-k against the oracle
    announce("markov thin", V, r, P, k)
    U, W = synth.markov_factors(41 + r, V, r, True)
    rows = 4
    L = synth.drafter_logits(41, 1, rows, V, 3.0, (0.5, 2.0))[0]
    rng = np.random.default_rng(V + P)
    toks = rng.integers(0, V, size=P).astype(np.int32)
    lrow = rng.integers(0, rows, size=P).astype(np.int32)
    dU, dW = dev_factors(U, W)
    lse, tt, tl, z = pct.markov_logits(dev_f32(L), dU, dW, dev_i32(toks),
                                       dev_i32(lrow), k, want_z=True)
    lse, tt, tl, z = (x.cpu().numpy() for x in (lse, tt, tl, z))
    near = 0
    for p in range(P):
        M = oracle.markov_row(U, W, int(toks[p]))
        ref = L[lrow[p]].astype(np.float64) + M
        assert np.abs(z[p] - ref).max() <= 1e-5 * np.abs(ref).max()
        ol, ot, oz, gap = oracle.row_stats(L[lrow[p]], M, k)
        assert abs(lse[p] - ol) <= 1e-5 * max(1.0, abs(ol))
        if np.array_equal(tt[p], ot):
            olp = (oz - np.float32(ol)).astype(np.float32)
            assert np.abs(tl[p] - olp).max() <= 1e-4
        else:
            assert gap < 1e-5, (p, tt[p], ot)
            near += 1
    assert near <= 1


def test_invalid_arguments_rejected():
    announce("markov invalid args")
    t = dev_i32(np.zeros(4, np.int32))
    U = torch.zeros(10, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pct.PCTError):
        pct.markov_logits(None, U, U, t, None, 11)  # k > V
    with pytest.raises(ValueError):
        pct.markov_logits(None, U, None, t, None, 2)
