"""GPU parity of the parent-conditioned tree build (pct_build_tree), the
ancestry mask and the acceptance walk against the CPU oracle.

Bins per request (comparison protocol): EXACT when tok/parent/depth/n_nodes
match bit for bit and scores within 1e-4; NEAR-TIE when they differ but the
oracle saw an fp32 gap below 1e-5 at a selection boundary or between two
adjacent nodes, in which case the GPU tree must still be a valid tree whose
scores are the oracle's path scores; FAIL otherwise."""
import math
import os

import numpy as np
import pytest
import torch

import draft_tree_construction_markov_amd as pct
import oracle
import synth
from gpu_util import announce, dev_f32, dev_factors, dev_i32
from parity import RequestContext, classify
from treecheck import check_structure, naive_accept

pytestmark = pytest.mark.gpu


def _golden(name):
    """The oracle's trees for every request of a full-size workload
    (written by tests/golden/make_golden.py from the oracle alone)."""
    path = os.path.join(os.path.dirname(__file__), "golden",
                        f"{name}_trees.npz")
    z = np.load(path)
    w = synth.TREE_WORKLOADS[name]
    assert list(z["shape"]) == [w.seed, w.batch, w.B, w.V, w.k, w.beam_w,
                                w.N, w.r], "golden file is for another shape"
    return {k: z[k] for k in z.files if k != "shape"}


def compare_all(g, o, L, U, W, A, k, beam_w, N, reqs, mask=True):
    """Bin every request of reqs (rows j of o correspond to requests
    reqs[j]); FAIL raises."""
    bins = {"exact": 0, "near": 0}
    worst = 0.0
    for j, q in enumerate(reqs):
        gq = {k2: g[k2][[q]] for k2 in ("tok", "parent", "depth", "score",
                                         "n_nodes")}
        oq = {k2: o[k2][[j]] for k2 in ("tok", "parent", "depth", "score",
                                         "n_nodes")}
        ctx = RequestContext(L[q], U, W, A[q], k, beam_w, N)
        res, det = classify(gq, oq, 0, ctx)
        bins[res] += 1
        if res == "exact":
            worst = max(worst, det)
        else:
            print(f"request {q}: near-tie ({det})")
        if mask:
            want = oracle.mask(g["parent"][q], int(g["n_nodes"][q]), N)
            assert np.array_equal(g["mask"][q], want), q
    print(f"bins {bins}, max |dscore| {worst:.2e}")
    return bins


def run_and_compare(L, U, W, A, k, beam_w, N, reqs=None, mask=True):
    batch, B, V = L.shape
    dU, dW = dev_factors(U, W)
    announce("build", dict(batch=batch, B=B, V=V, k=k, beam=beam_w, N=N,
                           r=None if U is None else U.shape[1]))
    out = pct.build_tree(dev_f32(L), dU, dW, dev_i32(A), k, beam_w, N,
                         mask=mask)
    torch.cuda.synchronize()
    g = out.numpy()
    reqs = list(range(batch)) if reqs is None else reqs
    o = oracle.build_tree(L[reqs], U, W, A[reqs], k, beam_w, N)
    bins = compare_all(g, o, L, U, W, A, k, beam_w, N, reqs, mask)
    return g, o, bins


def _random(seed, batch, B, V, r, bf16=True, T=1.0):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(batch, B, V)) * 1.7 / T).astype(np.float32)
    A = rng.integers(0, V, size=batch).astype(np.int32)
    if r == 0:
        return L, None, None, A
    U, W = synth.markov_factors(seed, V, r, bf16)
    return L, U, W, A


def test_tiny_workload():
    w = synth.TREE_WORKLOADS["tiny"]
    L, U, W, A = synth.tree_inputs(w)
    g, o, bins = run_and_compare(L, U, W, A, w.k, w.beam_w, w.N)
    assert bins["exact"] == 1


@pytest.mark.parametrize("batch,B,V,k,beam,N,r", [
    (4, 5, 3000, 8, 16, 64, 256),     # ragged last vocab tile
    (3, 6, 4096, 4, 6, 40, 128),
    (2, 3, 640, 16, 32, 100, 64),
    (20, 4, 2048, 8, 16, 128, 32),     # many parents: several waves
])
def test_markov_tree_parity(batch, B, V, k, beam, N, r):
    L, U, W, A = _random(batch * 100 + V, batch, B, V, r)
    run_and_compare(L, U, W, A, k, beam, N)


@pytest.mark.parametrize("batch,B,V,k,beam,N,r", [
    (3, 3, 40, 4, 6, 30, 64),    # the whole vocabulary in one ragged tile
    (2, 4, 20, 8, 12, 50, 32),   # fewer tokens than the 32 seed slots
    (2, 2, 5, 5, 10, 30, 32),    # k = V: every token of every parent
])
def test_vocab_smaller_than_a_tile(batch, B, V, k, beam, N, r):
    L, U, W, A = _random(batch * 17 + V, batch, B, V, r)
    run_and_compare(L, U, W, A, k, beam, N)


@pytest.mark.parametrize("batch,B,V,k,beam,N,r,reqs", [
    # frontiers above 256 parents take the 8-wave fused kernel (512
    # parents per workgroup): 576-640 parents make two parent tiles, the
    # second partly empty; ragged last vocabulary tile
    (40, 3, 3000, 8, 16, 64, 256, None),
    (36, 4, 5000, 8, 16, 96, 128, None),          # rank 128
    (33, 3, 2002, 8, 16, 64, 256, None),          # V % 4 != 0: other kernel
    (24, 3, 151936, 8, 16, 64, 256, [0, 11, 23]),  # full vocabulary
])
def test_large_frontier_parity(batch, B, V, k, beam, N, r, reqs):
    L, U, W, A = _random(batch * 7 + V, batch, B, V, r)
    run_and_compare(L, U, W, A, k, beam, N, reqs=reqs)


@pytest.mark.parametrize("batch,B,V,k,beam,N,r", [
    # frontiers of 64 parents or more take the two-kernel expand (one wave
    # per parent, up to four parents per workgroup, the seeds of up to 32
    # children per MFMA block): four parents of k = 4 (16 children) and a
    # last workgroup of two; two parents of k = 16; one parent of k = 32;
    # a split already at depth 1 (70 anchors, k = 3)
    (24, 4, 3000, 4, 6, 40, 128),
    (12, 3, 2500, 16, 8, 60, 64),
    (10, 3, 2000, 32, 7, 50, 256),
    (70, 2, 1500, 3, 5, 20, 32),
])
def test_two_kernel_expand_shapes(batch, B, V, k, beam, N, r):
    L, U, W, A = _random(batch * 11 + V + k, batch, B, V, r)
    g, o, bins = run_and_compare(L, U, W, A, k, beam, N)
    assert bins["near"] <= max(1, batch // 16), bins


@pytest.mark.parametrize("N", [12, 200, 248])
def test_rows_with_few_finite_logits(N):
    # three finite logits per row, k = 8: most children score -inf, so their
    # keys share the score bits and differ in parent and token only; the
    # top-N cut falls among them (N = 200 of a 248-child pool) or keeps the
    # whole pool
    L, U, W, A = _random(5, 3, 4, 600, 32)
    rng = np.random.default_rng(1)
    for q in range(3):
        for d in range(4):
            keep = rng.choice(600, 3, replace=False)
            row = np.full(600, -np.inf, np.float32)
            row[keep] = L[q, d, keep]
            L[q, d] = row
    g, o, bins = run_and_compare(L, U, W, A, 8, 10, N)
    assert bins["exact"] == 3, bins
    if N == 200:
        assert np.isneginf(g["score"][0]).sum() > 100


@pytest.mark.parametrize("batch,B,V,k,beam,N,r", [
    # the global top-N selects the N smallest keys of a pool by radix
    # select, then sorts them (runs of 64 by counting, merged level by
    # level): 6 + 36 + 216 + 4 * 1200 = 5058 children, N = 700 (11 runs,
    # four merge levels).  When the pool and the kept keys do not fit one
    # workgroup's LDS, every key is ranked by counting over several
    # workgroups: 32 + 4 * 1920 = 7712 children, N = 4200
    (2, 7, 4000, 6, 200, 700, 64),
    (2, 5, 4000, 32, 60, 4200, 64),
])
def test_top_n_sorted_and_counted(batch, B, V, k, beam, N, r):
    L, U, W, A = _random(batch * 13 + k, batch, B, V, r)
    g, o, bins = run_and_compare(L, U, W, A, k, beam, N)
    # thousands of kept nodes: an fp32 score tie between two of them is
    # binned as a near-tie
    assert bins["near"] <= 1, bins


@pytest.mark.parametrize("batch,B,V,k,beam,N,r", [
    (8, 4, 8192, 8, 16, 64, 256),     # frontiers of 128 parents, groups of 16
    (32, 3, 4096, 8, 16, 64, 256),    # 512 parents: two blocks per wave
])
def test_flat_rows_many_candidates(batch, B, V, k, beam, N, r):
    # flat logits put many elements of every row near the seed threshold, so
    # the fused kernel's per-lane lists take many inserts; the groups are
    # whole quads of lanes, which share their L values
    L, U, W, A = _random(batch * 3 + V, batch, B, V, r, T=8.0)
    run_and_compare(L, U, W, A, k, beam, N)


def test_marginal_tree_parity():
    L, U, W, A = _random(7, 5, 6, 5000, 0)
    run_and_compare(L, U, W, A, 8, 16, 128)


def test_chain_and_uniform_ties():
    # k = 1: the greedy chain
    L, U, W, A = _random(11, 3, 7, 2000, 256)
    g, o, _ = run_and_compare(L, U, W, A, 1, 4, 7)
    for q in range(3):
        assert list(g["tok"][q]) == list(oracle.greedy_chain(L[q], U, W,
                                                             int(A[q])))
    # all-equal logits, no Markov term: massive exact ties resolved by key
    Lu = np.zeros((2, 3, 640), np.float32)
    A = np.array([3, 5], np.int32)
    g, o, bins = run_and_compare(Lu, None, None, A, 3, 2, 10)
    assert bins["exact"] == 2


def test_long_lists_small_staged_form_without_quads():
    # k = 20 leaves LDS for 16 staged L row slots only; beam 18 makes groups
    # of 18 parents (not whole quads of lanes), so the staged form reads each
    # lane's L values itself; 360 parents per depth, ragged last tile
    L, U, W, A = _random(71, 20, 3, 5000, 256)
    g, o, bins = run_and_compare(L, U, W, A, 20, 18, 100)
    assert bins["near"] <= 1, bins


def test_integer_ties_in_queued_tile_order():
    # Integer factors and logits: every z = L + U.W is an exact integer, so
    # children of one parent tie exactly, also at the top-k boundary.  Depth
    # 3 has 320 parents over V = 40000 (625 vocabulary tiles): the fused
    # kernel hands the tiles past the first 512 out from its queue, so a
    # lane meets its tiles out of vocabulary order.  The oracle keeps the
    # smaller token of a tie; the GPU tree must match it exactly (a tie the
    # kernel broke the other way would show as a near-tie bin).
    rng = np.random.default_rng(29)
    batch, B, V, r = 20, 3, 40000, 256
    U = synth.bf16_bits(rng.integers(-1, 2, size=(V, r)).astype(np.float32))
    W = synth.bf16_bits(rng.integers(-1, 2, size=(V, r)).astype(np.float32))
    L = rng.integers(-4, 5, size=(batch, B, V)).astype(np.float32)
    A = rng.integers(0, V, size=batch).astype(np.int32)
    g, o, bins = run_and_compare(L, U, W, A, 8, 16, 64)
    assert bins["near"] == 0, bins


@pytest.mark.parametrize("batch,beam", [(32, 16), (12, 16)])
def test_spiked_rows_move_the_exponent_shift(batch, beam):
    # Some L rows hold one logit 60 or 120 above the rest (natural units):
    # the fused kernel's exponent sum starts from a shift just below the
    # seed threshold, and a group that lies more than 64 (log2 units) above
    # it, up to past the fp32 range of 2^(z*log2e - shift), must move the
    # shift.  32 requests give 512-parent launches (queued tiles), 12 give
    # 192 (contiguous slices).
    L, U, W, A = _random(41 + batch, batch, 4, 6000, 256)
    rng = np.random.default_rng(43)
    for q in range(batch):
        for d in range(4):
            if (q + d) % 3 == 0:
                L[q, d, rng.integers(0, 6000)] += 60.0 if (q + d) % 2 else 120.0
    g, o, bins = run_and_compare(L, U, W, A, 8, beam, 64)
    assert bins["near"] <= 1, bins


def test_tile_queue_cleared_for_large_frontiers():
    # 17600 parents at depth 3 make 35 parent tiles, so the fused kernel's
    # tile queue has 70 counters; the build clears them itself, so a
    # workspace full of stale bytes must give the same trees as a cleared one
    batch, B, V, r = 1100, 3, 2000, 32
    L, U, W, A = _random(53, batch, B, V, r)
    dU, dW = dev_factors(U, W)
    dL, dA = dev_f32(L), dev_i32(A)
    announce("tile queue", dict(batch=batch, B=B, V=V))
    tb = pct.TreeBuilder(batch, B, V, 8, 16, 16, r=r, mask=False)
    tb.ws.fill_(0x41)
    a = {k: v.clone() for k, v in vars(tb.run(dL, dU, dW, dA)).items()
         if v is not None}
    tb.ws.zero_()
    b = tb.run(dL, dU, dW, dA)
    for key in ("tok", "parent", "depth", "score", "n_nodes"):
        assert torch.equal(a[key], getattr(b, key)), key
    # and a few requests against the oracle
    g = b.numpy()
    reqs = [0, 549, 1099]
    o = oracle.build_tree(L[reqs], U, W, A[reqs], 8, 16, 16)
    bins = compare_all(g, o, L, U, W, A, 8, 16, 16, reqs, mask=False)
    assert bins["exact"] == len(reqs), bins


def test_deterministic_and_stream_safe():
    L, U, W, A = _random(13, 6, 5, 3000, 256)
    dU, dW = dev_factors(U, W)
    dL, dA = dev_f32(L), dev_i32(A)
    announce("determinism")
    tb = pct.TreeBuilder(6, 5, 3000, 8, 16, 64, r=256, mask=True)
    a = {k: v.clone() for k, v in vars(tb.run(dL, dU, dW, dA)).items()}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = tb.run(dL, dU, dW, dA)
    s.synchronize()
    for key in ("tok", "parent", "depth", "score", "n_nodes", "mask"):
        assert torch.equal(a[key], getattr(b, key)), key


def test_b7_workload_full():
    w = synth.TREE_WORKLOADS["b7"]
    L, U, W, A = synth.tree_inputs(w)
    run_and_compare(L, U, W, A, w.k, w.beam_w, w.N)


def test_b16_workload_full():
    # the benchmark's workload at full size, every request against the
    # oracle's trees (golden file), the masks against their definition
    w = synth.TREE_WORKLOADS["b16"]
    o = _golden("b16")
    L, U, W, A = synth.tree_inputs(w)
    dU, dW = dev_factors(U, W)
    announce("build b16", dict(batch=w.batch, N=w.N))
    tb = pct.TreeBuilder(w.batch, w.B, w.V, w.k, w.beam_w, w.N, r=w.r,
                         bf16=True, mask=True)
    g = tb.run(dev_f32(L), dU, dW, dev_i32(A)).numpy()
    torch.cuda.synchronize()
    bins = compare_all(g, o, L, U, W, A, w.k, w.beam_w, w.N,
                       list(range(w.batch)))
    assert bins["exact"] + bins["near"] == w.batch
    assert bins["near"] <= w.batch // 16, bins


def test_round_workload_full():
    # the full round at its own size (batch 128, N = 512, 512x512 masks,
    # acceptance walk): every tree against the oracle's (golden file), every
    # mask against its definition, every walk against the oracle's walk
    w = synth.TREE_WORKLOADS["round"]
    o = _golden("round")
    print("generating the round inputs (1.2 GB of logits)", flush=True)
    L, U, W, A = synth.tree_inputs(w)
    dU, dW = dev_factors(U, W)
    announce("build round", dict(batch=w.batch, N=w.N))
    tb = pct.TreeBuilder(w.batch, w.B, w.V, w.k, w.beam_w, w.N, r=w.r,
                         bf16=True, mask=True)
    g = tb.run(dev_f32(L), dU, dW, dev_i32(A)).numpy()
    torch.cuda.synchronize()
    bins = compare_all(g, o, L, U, W, A, w.k, w.beam_w, w.N,
                       list(range(w.batch)))
    assert bins["exact"] + bins["near"] == w.batch
    assert bins["near"] <= w.batch // 16, bins
    tgt = synth.targets_from_tree(w.seed, g["tok"], g["parent"], g["depth"],
                                  g["n_nodes"], A, w.V, w.B,
                                  synth.round_agreement(w.B))
    announce("round verify", dict(batch=w.batch, N=w.N))
    args = (dev_i32(g["tok"]), dev_i32(g["parent"]), dev_i32(g["depth"]),
            dev_i32(g["n_nodes"]), dev_i32(tgt), w.B)
    walks = [pct.verify_accept(*args),
             pct.verify_accept(*args, mask=tb.out.mask)]
    for tau, an, at in walks:
        tau, an, at = tau.cpu().numpy(), an.cpu().numpy(), at.cpu().numpy()
        for q in range(w.batch):
            t2, an2, at2 = oracle.accept(g["tok"][q], g["parent"][q],
                                         int(g["n_nodes"][q]), w.B, tgt[q])
            assert tau[q] == t2 and list(an[q]) == list(an2) and \
                list(at[q]) == list(at2), q
    print(f"round: mean tau {tau.mean():.3f}")


@pytest.mark.parametrize("case", ["pool_below_N", "k48_seedless",
                                  "fp32_factors", "bf16_rank48"])
def test_other_build_paths(case):
    # paths of pct_build_tree outside the MFMA fast path: a pool smaller
    # than the budget (padded outputs), k above the 32 seed tokens (no seed
    # thresholds), fp32 factors and a bf16 rank that is not a multiple of
    # 32 (the plain VALU kernel)
    if case == "pool_below_N":
        L, U, W, A = _random(31, 3, 3, 3000, 256)
        k, beam, N = 4, 2, 40   # pool 4 + 8 + 8 = 20 < 40
    elif case == "k48_seedless":
        L, U, W, A = _random(32, 4, 3, 6000, 128)
        k, beam, N = 48, 8, 150
    elif case == "fp32_factors":
        L, U, W, A = _random(33, 3, 4, 2500, 48, bf16=False)
        k, beam, N = 8, 12, 60
    else:
        L, U, W, A = _random(34, 3, 4, 2500, 48)
        k, beam, N = 8, 12, 60
    g, o, bins = run_and_compare(L, U, W, A, k, beam, N)
    if case == "pool_below_N":
        for q in range(L.shape[0]):
            n = int(g["n_nodes"][q])
            assert n == 20
            assert np.all(g["tok"][q][n:] == -1)
            assert np.all(g["parent"][q][n:] == -1)
            assert np.all(g["depth"][q][n:] == 0)
            assert np.all(np.isneginf(g["score"][q][n:]))


def _near_one_hot(seed, batch, B, V):
    """Rows of log-probabilities with a top-1 probability above 1 - 1e-7:
    the row maximum is within 1e-7 of 0 and every other entry is tiny."""
    rng = np.random.default_rng(seed)
    rest = rng.normal(size=(batch, B, V)) - 24.0
    top = rng.integers(0, V, size=(batch, B))
    for q in range(batch):
        for d in range(B):
            rest[q, d, top[q, d]] = 0.0
    m = rest.max(axis=2, keepdims=True)
    lse = m + np.log(np.exp(rest - m).sum(axis=2, keepdims=True))
    return (rest - lse).astype(np.float32)


def test_near_one_hot_rows_keep_children_below_parents():
    # z - lse is never positive, so a child never outscores its parent and
    # parents always precede children in the output
    L = _near_one_hot(41, 4, 5, 3000)
    A = np.arange(4, dtype=np.int32)
    g, o, bins = run_and_compare(L, None, None, A, 4, 8, 60)
    for q in range(4):
        n = int(g["n_nodes"][q])
        assert np.all(g["score"][q][:n] <= 0.0)
        for i in range(n):
            p = int(g["parent"][q][i])
            assert p < i
    U, W = synth.markov_factors(41, 3000, 32, True)
    g, o, bins = run_and_compare(L, U, W, A, 4, 8, 60)


def test_verify_standalone_matches_oracle():
    # the walk on identical inputs (oracle trees and synthetic targets)
    # must match bit for bit
    rng = np.random.default_rng(21)
    B, V, N, batch = 6, 50, 48, 40
    L, U, W, A = _random(21, batch, B, V, 16, bf16=False)
    o = oracle.build_tree(L, U, W, A, 4, 8, N)
    tgt = synth.targets_from_tree(21, o["tok"], o["parent"], o["depth"],
                                  o["n_nodes"], A, V, B, lambda d: 0.7)
    announce("verify standalone")
    masks = np.stack([oracle.mask(o["parent"][q], int(o["n_nodes"][q]), N)
                      for q in range(batch)])
    dmask = torch.from_numpy(masks.view(np.int64)).cuda()
    args = (dev_i32(o["tok"]), dev_i32(o["parent"]), dev_i32(o["depth"]),
            dev_i32(o["n_nodes"]), dev_i32(tgt), B)
    for mk in (None, dmask):
        tau, an, at = pct.verify_accept(*args, mask=mk)
        tau, an, at = tau.cpu().numpy(), an.cpu().numpy(), at.cpu().numpy()
        for q in range(batch):
            t2, an2, at2 = oracle.accept(o["tok"][q], o["parent"][q],
                                         int(o["n_nodes"][q]), B, tgt[q])
            assert tau[q] == t2 and list(an[q]) == list(an2) and \
                list(at[q]) == list(at2), q
            t3, an3, at3 = naive_accept(o["tok"][q], o["parent"][q],
                                        o["depth"][q], int(o["n_nodes"][q]),
                                        tgt[q], B)
            assert t3 == t2


def test_verify_worked_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "accept_worked_example.json")))
    tok = dev_i32(np.array([g["tok"]]))
    par = dev_i32(np.array([g["parent"]]))
    dep = dev_i32(np.array([list(range(1, len(g["tok"]) + 1))]))
    n = dev_i32(np.array([len(g["tok"])]))
    tgt = dev_i32(np.array([g["target"]]))
    announce("verify worked example")
    tau, an, at = pct.verify_accept(tok, par, dep, n, tgt, g["B"])
    assert int(tau[0]) == g["expected_tau"] == 5
    assert at[0].cpu().tolist() == g["expected_accept_tok"]


def _random_tree(rng, N, n, B):
    """Parents before children, depth <= B, siblings numbered 0, 1, ... as
    their tokens (so siblings never share a token)."""
    par = np.full(N, -1, np.int32)
    dep = np.zeros(N, np.int32)
    tok = np.zeros(N, np.int32)
    kids = {}
    for i in range(n):
        p = -1
        if i > 0 and rng.random() > 0.02:
            p = int(rng.integers(max(0, i - 64), i))
            if dep[p] >= B:
                p = -1
        par[i] = p
        dep[i] = 1 if p < 0 else dep[p] + 1
        tok[i] = kids.get(p, 0)
        kids[p] = tok[i] + 1
    return tok, par, dep


@pytest.mark.parametrize("N,ns", [(8192, (8192, 5000)), (700, (700, 321))])
def test_walk_on_large_trees(N, ns):
    # N = 8192, the largest the call takes (128 mask words per node, more
    # than 64 KB of LDS), and N = 700 (11 words): the acceptance test's
    # word-by-word path, with and without the mask
    rng = np.random.default_rng(N + 61)
    B = 12
    trees = [_random_tree(rng, N, n, B) for n in ns]
    tok = np.stack([x[0] for x in trees])
    par = np.stack([x[1] for x in trees])
    dep = np.stack([x[2] for x in trees])
    n = np.array(ns, np.int32)
    tgt = rng.integers(0, 3, size=(len(ns), N + 1)).astype(np.int32)
    announce("walk large", dict(N=N))
    args = (dev_i32(tok), dev_i32(par), dev_i32(dep), dev_i32(n), dev_i32(tgt),
            B)
    mk = pct.tree_mask(dev_i32(par), dev_i32(n))
    for m in (None, mk):
        tau, an, at = pct.verify_accept(*args, mask=m)
        tau, an, at = (x.cpu().numpy() for x in (tau, an, at))
        for q in range(len(ns)):
            t2, an2, at2 = oracle.accept(tok[q], par[q], int(n[q]), B, tgt[q])
            assert int(tau[q]) == t2, (q, m is None)
            assert list(an[q]) == list(an2), q
            assert list(at[q]) == list(at2), q


def test_mask_edge_cases():
    announce("mask edges")
    N = 130
    par = np.stack([np.arange(-1, N - 1), -np.ones(N, np.int64)]).astype(np.int32)
    n = np.array([N, 70], np.int32)
    m = pct.tree_mask(dev_i32(par), dev_i32(n)).cpu().numpy().view(np.uint64)
    for q in range(2):
        assert np.array_equal(m[q], oracle.mask(par[q], int(n[q]), N))
