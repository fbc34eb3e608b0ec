"""GPU parity of the adaptive best-first build (pct_build_tree_adaptive)
against the CPU oracle: the b16-sized adaptive workload (peaked and flat
rounds, context lengths, the convex cost model), fixed budgets that need the
full-length list pass, exhausted trees, exact ties and the closed form."""
import math

import numpy as np
import pytest
import torch

import draft_tree_construction_markov_amd as pct
import oracle
import synth
from gpu_util import announce, dev_f32, dev_i32
from treecheck import NEAR_TIE, SCORE_TOL, check_structure, path_tokens

pytestmark = pytest.mark.gpu

COST = {k: synth.ADAPTIVE[k] for k in ("C_d", "c0", "c1", "c2", "c_ell")}


def _true_scores(L, tok, parent, n):
    """Double-precision path log-probabilities of a best-first tree over
    marginal rows (each edge: z - lse of its depth's row)."""
    lse = [oracle.row_stats(L[d], None, 1)[0] for d in range(L.shape[0])]
    out = []
    for i in range(n):
        p = int(parent[i])
        d = 0 if p < 0 else len(path_tokens(tok, parent, p))
        s = (0.0 if p < 0 else out[p]) + float(L[d][int(tok[i])]) - lse[d]
        out.append(s)
    return out


def _near_ok(g, o, q, L, B):
    """A request whose GPU tree differs from the oracle's: the first
    difference must sit at an oracle near-tie (an ordering tie of the two
    nodes there, or a stop decision whose gain is within 1e-4 relative of
    zero), and the GPU tree must be valid: structure, scores equal to their
    recomputation within 1e-4, and Phi within n * 1e-5 * max P of the
    oracle's (the best-first tree maximises Phi for its size)."""
    ns, no = int(g["n_star"][q]), o["n_star"]
    check_structure(g["tok"][q], g["parent"][q], g["depth"][q], ns, B)
    ts = _true_scores(L[q], g["tok"][q], g["parent"][q], ns)
    for i in range(ns):
        assert abs(ts[i] - float(g["score"][q][i])) < SCORE_TOL, (q, i)
    if ns != no:
        assert o["gain_margin"] < 1e-4, (q, ns, no, o["gain_margin"])
    m = min(ns, no)
    diff = [i for i in range(m)
            if (g["tok"][q][i], g["parent"][q][i]) !=
            (o["tok"][i], o["parent"][i])]
    if diff:
        i = diff[0]
        assert abs(ts[i] - float(o["score"][i])) < NEAR_TIE, (q, i)
        phi_g = sum(math.exp(x) for x in ts[:m])
        phi_o = sum(math.exp(float(x)) for x in o["score"][:m])
        maxP = math.exp(max(float(o["score"][0]), ts[0]))
        assert phi_g >= phi_o - m * NEAR_TIE * maxP, (q, phi_g, phi_o)


def run_compare(L, ctx, n_max, cost, label):
    batch, B, V = L.shape
    announce("adaptive", label, dict(batch=batch, B=B, V=V, n_max=n_max,
                                     cost=cost is not None))
    ab = pct.build_tree_adaptive(dev_f32(L), dev_i32(ctx), n_max, cost,
                                 mask=True)
    torch.cuda.synchronize()
    g = ab.numpy()
    bins = {"exact": 0, "near": 0}
    for q in range(batch):
        o = oracle.adaptive(L[q], n_max, int(ctx[q]), cost)
        ns = int(g["n_star"][q])
        same = (ns == o["n_star"] and
                np.array_equal(g["tok"][q], o["tok"]) and
                np.array_equal(g["parent"][q], o["parent"]) and
                np.array_equal(g["depth"][q], o["depth"]))
        if same:
            d = np.abs(g["score"][q][:ns].astype(np.float64)
                       - o["score"][:ns].astype(np.float64))
            assert (d.max() if ns else 0.0) <= SCORE_TOL, q
            assert abs(g["phi"][q] - o["phi"]) <= 1e-4 * max(1.0, o["phi"])
            assert abs(g["throughput"][q] - o["throughput"]) <= \
                1e-4 * o["throughput"]
            bins["exact"] += 1
        else:
            _near_ok(g, o, q, L, B)
            print(f"{label}: request {q} near-tie (n* {ns} vs {o['n_star']})")
            bins["near"] += 1
        want = oracle.mask(g["parent"][q], max(ns, 0), n_max)
        assert np.array_equal(g["mask"][q], want), q
    print(f"{label}: bins {bins}, n* {[int(x) for x in g['n_star'][:16]]}")
    return g, bins


def test_adaptive_workload_full():
    # the adaptive workload at full size, every request against the oracle
    a = synth.ADAPTIVE
    L, peaked, ctx = synth.adaptive_round(a["seed"], a["batch"], a["B"],
                                          a["V"])
    g, bins = run_compare(L, ctx, a["n_max"], COST, "adaptive")
    assert bins["exact"] + bins["near"] == a["batch"]
    assert bins["near"] <= a["batch"] // 16, bins


def test_sibling_score_tie_takes_the_larger_logit():
    # two siblings whose fp32 scores tie exactly while their logits differ
    # (tokens 1 < 2 carry logits 0.0010000 < 0.0010001 next to a logit of
    # 20): the more probable one, token 2, is taken first
    row = np.full(6, -50.0, np.float32)
    row[3] = 20.0
    row[1] = np.float32(0.0010000)
    row[2] = np.float32(0.0010001)
    L = np.stack([row, row])[None]
    g, bins = run_compare(L, np.array([0], np.int32), 42, None, "sibling-tie")
    d1 = [int(t) for t, p in zip(g["tok"][0], g["parent"][0]) if p == -1]
    assert d1.index(2) < d1.index(1)


def test_near_one_hot_rows():
    # log-probability rows with a top-1 probability above 1 - 1e-7: every
    # log pi stays <= 0, so children never outscore their parents
    rng = np.random.default_rng(43)
    V = 4000
    rest = rng.normal(size=(3, 4, V)) - 24.0
    rest[:, :, 17] = 0.0
    m = rest.max(axis=2, keepdims=True)
    L = (rest - (m + np.log(np.exp(rest - m).sum(axis=2,
                                                  keepdims=True)))).astype(
        np.float32)
    g, bins = run_compare(L, np.full(3, 600, np.int32), 64, None, "one-hot")
    assert np.all(g["score"][:, :64] <= 0.0)
    g, bins = run_compare(L, np.full(3, 600, np.int32), 64, COST,
                          "one-hot-cost")


def test_fixed_budget_uses_full_lists():
    # no cost model: n* = n_max = 200 > the 64-entry first-pass lists, so the
    # requests go through the full-length pass
    rng = np.random.default_rng(4)
    L = (rng.normal(size=(6, 5, 3000)) * 2).astype(np.float32)
    ctx = np.full(6, 1000, np.int32)
    g, bins = run_compare(L, ctx, 200, None, "fixed-200")
    assert all(int(x) == 200 for x in g["n_star"])


def test_exhausted_tree_and_small_vocab():
    rng = np.random.default_rng(5)
    L = (rng.normal(size=(3, 3, 5)) * 1.5).astype(np.float32)
    ctx = np.full(3, 100, np.int32)
    g, bins = run_compare(L, ctx, 300, None, "exhausted")
    assert all(int(x) == 5 + 25 + 125 for x in g["n_star"])


@pytest.mark.parametrize("V,B", [(2, 5), (3, 3), (4, 2), (6, 2)])
def test_full_tree_over_tiny_vocab_in_the_batched_pass(V, B):
    # the budget is the whole tree (at most 64 nodes, so the batched pass
    # takes it) and exceeds the B*V single deviations, so the threshold is
    # -inf and every block end of the padded lists passes; every family has
    # at most 4 children, or 6 (written by the whole wave)
    rng = np.random.default_rng(11 + V)
    L = (rng.normal(size=(4, B, V)) * 2.0).astype(np.float32)
    ctx = np.array([100, 2000, 9000, 30000], np.int32)
    full = sum(V ** d for d in range(1, B + 1))
    g, bins = run_compare(L, ctx, full, None, f"full-V{V}")
    assert all(int(x) == full for x in g["n_star"])
    assert bins["near"] == 0
    _, bins = run_compare(L, ctx, full, COST, f"full-V{V}-cost")
    assert bins["near"] == 0


def test_row_lists_bound_overflow():
    # The single-read row statistics cut a row of V = 151936 into 4 pieces
    # of 9496 16-byte vectors, vector j of a piece going to thread j % 512.
    # Large logits only on threads 0..251 (63 groups of 4, fewer than the 64
    # list entries) make the first selection bound loose: over 2048
    # candidates pass it, so the bound is tightened and the piece re-read.
    V = 151936
    rng = np.random.default_rng(7)
    L = rng.normal(size=(2, 3, V)).astype(np.float32)
    vec = np.arange(V) // 4
    slot = (vec - (vec // 9496) * 9496) % 512
    L[:, :, slot < 252] += 10.0
    ctx = np.array([700, 9000], np.int32)
    g, bins = run_compare(L, ctx, 64, None, "bound-overflow")
    assert all(int(x) == 64 for x in g["n_star"])


def test_uniform_rows_ties():
    L = np.zeros((2, 4, 700), np.float32)
    ctx = np.array([512, 30000], np.int32)
    run_compare(L, ctx, 90, None, "uniform-fixed")
    run_compare(L, ctx, 500, COST, "uniform-cost")


def test_uniform_single_row_closed_form():
    for V, ell in ((50, 0), (200, 3000), (1000, 20000)):
        L = np.zeros((1, 1, V), np.float32)
        ab = pct.build_tree_adaptive(dev_f32(L), dev_i32(np.array([ell])),
                                     min(V, 1024), COST)
        torch.cuda.synchronize()
        c = COST

        def D(n):
            return c["C_d"] + c["c0"] + c["c1"] * n + c["c2"] * n * n + \
                c["c_ell"] * ell * n
        want = V
        for n in range(V):
            if D(n) / V <= (1 + n / V) * (D(n + 1) - D(n)):
                want = n
                break
        assert int(ab.n_star[0]) == want


def _tie_rows(B, n_dev, n_next, V=2000):
    """Rows with exact score ties across depths: one token of logit 0 (its
    log-probability rounds to a few 1e-12 below 0), n_dev tokens at -30 and
    n_next at -31 (their log-probabilities round to exactly -30 and -31),
    the rest at -200.  Every deviation from the greedy chain, and every
    greedy continuation after one, scores exactly -30 (or -31): the order
    inside those groups is decided by the parents' output order alone."""
    row = np.full(V, -200.0, np.float32)
    row[5] = 0.0
    row[10:10 + n_dev] = -30.0
    row[10 + n_dev:10 + n_dev + n_next] = -31.0
    return np.tile(row, (1, B, 1))


def test_exact_ties_across_depths_in_order():
    # 4 depths, 8 tokens at -30, 55 at -31: the first 64 nodes are the
    # chain and 60 nodes of the -30 group, whose order runs through the
    # deviations of each depth and then the greedy continuations after them
    L = _tie_rows(4, 8, 55)
    g, bins = run_compare(L, np.array([800], np.int32), 64, None, "ties-4")
    assert bins["exact"] == 1
    assert int(g["n_star"][0]) == 64
    assert np.all(g["score"][0][4:64] == -30.0)
    run_compare(L, np.array([800], np.int32), 64, COST, "ties-4-cost")


def test_tie_groups_too_large_for_the_batched_pass():
    # 16 depths with 20 tokens at -30: over 2048 prefixes reach the
    # threshold, so the request is rebuilt by the serial pass
    L = _tie_rows(16, 20, 43)
    g, bins = run_compare(L, np.array([800], np.int32), 64, None, "ties-16")
    assert bins["exact"] == 1
    # 16 depths with 8 tokens at -30: about 1100 tied prefixes, ranked in
    # the batched pass
    L = _tie_rows(16, 8, 55)
    g, bins = run_compare(L, np.array([800], np.int32), 64, None,
                          "ties-16-small")
    assert bins["exact"] == 1


@pytest.mark.parametrize("B", [64, 65])
def test_deepest_blocks(B):
    # 64 depths (the most the batched pass stages) and 65 (serial pass)
    rng = np.random.default_rng(B)
    L = (rng.normal(size=(3, B, 3000)) * 3).astype(np.float32)
    L[:, :, 7] += 12.0  # confident rows: long greedy chains
    ctx = np.array([600, 5000, 30000], np.int32)
    run_compare(L, ctx, 64, None, f"deep-{B}")
    run_compare(L, ctx, 64, COST, f"deep-{B}-cost")


def test_adaptive_rejects_bad_cost():
    L = torch.zeros(1, 2, 100, device="cuda")
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = dict(COST, c2=-1e-3)
    with pytest.raises(pct.PCTError):
        pct.build_tree_adaptive(L, ctx, 10, bad)
