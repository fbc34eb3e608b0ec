"""Pins of the oracle's greedy best-first tree and its adaptive stop (CPU
only): brute-force enumeration of every prefix and of every ancestor-closed
subset on tiny vocabularies, exhaustive throughput scans (unimodality under a
convex verification cost, with a concave negative control) and a closed form
for uniform rows."""
import math

import numpy as np
import pytest

import oracle
import synth
from treecheck import (check_structure, closed_subsets, enumerate_prefixes,
                       path_tokens, unimodal)


def _lp_fn(L, U, W, anchor):
    """Per-depth fp32 log-probs given a prefix, from the oracle's row
    statistics (the selection logic below is independent of the oracle)."""
    V = L.shape[1]

    def f(prefix, d):
        prev = anchor if not prefix else prefix[-1]
        M = None if U is None else oracle.markov_row(U, W, prev)
        lse, tt, tz, _ = oracle.row_stats(L[d - 1], M, V)
        lp = np.empty(V, np.float32)
        lp[tt] = (tz - np.float32(lse)).astype(np.float32)
        return lp
    return f


def _tiny(seed, B, V, r):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(B, V)) * 1.5).astype(np.float32)
    if r == 0:
        return L, None, None
    U = synth.bf16_bits((rng.normal(size=(V, r)) * 0.8).astype(np.float32))
    W = synth.bf16_bits((rng.normal(size=(V, r)) * 0.8).astype(np.float32))
    return L, U, W


@pytest.mark.parametrize("seed,B,V,r", [(1, 3, 5, 0), (2, 4, 4, 0),
                                        (3, 3, 5, 4), (4, 4, 3, 4)])
def test_bestfirst_is_top_n_of_all_prefixes(seed, B, V, r):
    L, U, W = _tiny(seed, B, V, r)
    anchor = 1
    pre = enumerate_prefixes(_lp_fn(L, U, W, anchor), B, V)
    scores = sorted((s for s, _ in pre), reverse=True)
    total = len(pre)
    bf = oracle.bestfirst(L, U, W, anchor, total)
    assert bf["n"] == total
    check_structure(bf["tok"], bf["parent"], bf["depth"], total, B)
    # the order is by probability: the first n nodes are the n best prefixes
    assert np.array_equal(bf["score"], np.array(scores, np.float32))
    got = {tuple(path_tokens(bf["tok"], bf["parent"], i)) for i in range(total)}
    assert got == {p for _, p in pre}
    for n in (1, 2, 5, 9, total // 2):
        best = {p for s, p in sorted(pre, key=lambda x: -x[0])[:n]}
        first = {tuple(path_tokens(bf["tok"], bf["parent"], i))
                 for i in range(n)}
        assert first == best


@pytest.mark.parametrize("r", [0, 3])
def test_bestfirst_maximises_phi_over_all_closed_trees(r):
    # V = 3, B = 3: every ancestor-closed set of n prefixes is enumerated;
    # none has a larger expected acceptance Phi than the best-first one.
    B, V = 3, 3
    L, U, W = _tiny(7 + r, B, V, r)
    pre = enumerate_prefixes(_lp_fn(L, U, W, 2), B, V)
    P = [math.exp(s) for s, _ in pre]
    bf = oracle.bestfirst(L, U, W, 2, len(pre))
    for n in range(1, 6):
        best = max(sum(P[i] for i in c) for c in closed_subsets(pre, n))
        phi_bf = sum(math.exp(float(s)) for s in bf["score"][:n])
        assert phi_bf >= best - 1e-12
        assert abs(phi_bf - best) < 1e-12


def test_restricted_children_do_not_change_the_prefix():
    # Children are restricted to the n_max best tokens of their row; the
    # first n nodes must not depend on n_max >= n.
    rng = np.random.default_rng(11)
    B, V = 5, 400
    L = (rng.normal(size=(B, V)) * 2).astype(np.float32)
    big = oracle.bestfirst(L, None, None, 0, 300)
    for n in (1, 7, 40, 150):
        small = oracle.bestfirst(L, None, None, 0, n)
        assert small["n"] == n
        assert list(small["tok"]) == list(big["tok"][:n])
        assert list(small["parent"]) == list(big["parent"][:n])


COST = dict(C_d=1.0, c0=2.0, c1=0.004, c2=2e-6, c_ell=1e-5)


def _f_curve(scores, n_avail, cost, ell):
    """Throughput (1 + Phi_n)/(C_d + C_v(n)) for n = 0..n_avail, typed from
    the objective's definition."""
    out = []
    phi = 0.0
    for n in range(n_avail + 1):
        if n > 0:
            phi += math.exp(float(scores[n - 1]))
        D = (cost["C_d"] + cost["c0"] + cost["c1"] * n + cost["c2"] * n * n
             + cost["c_ell"] * ell * n)
        out.append((1.0 + phi) / D)
    return np.array(out)


@pytest.mark.parametrize("req", range(6))
def test_stop_is_the_argmax_of_a_unimodal_curve(req):
    B, V, n_max = 6, 3000, 256
    L, peaked, ctx = synth.adaptive_round(77, 1, B, V, req0=req)
    bf = oracle.bestfirst(L[0], None, None, 0, n_max)
    f = _f_curve(bf["score"], bf["n"], COST, int(ctx[0]))
    assert unimodal(f)
    ad = oracle.adaptive(L[0], n_max, int(ctx[0]), COST)
    best = int(np.argmax(f))  # smallest maximiser
    assert ad["n_star"] == best
    assert abs(ad["throughput"] - f[best]) <= 1e-12 * f[best]
    assert list(ad["tok"][:best]) == list(bf["tok"][:best])
    assert all(t == -1 for t in ad["tok"][best:])


def test_concave_cost_is_caught_by_the_checker():
    # Negative control: with a concave verification cost the curve need not
    # be unimodal, the unimodality checker must say so, and the greedy stop
    # (first non-positive gain) is no longer the global maximiser.
    scores = np.log(np.array([0.5] + [0.3] * 2 + [0.25] * 40)).astype(np.float32)
    cost = dict(C_d=0.0, c0=1.0, c1=1.0, c2=-0.02, c_ell=0.0)
    n_avail = len(scores)
    f = _f_curve(scores, n_avail, cost, 0)
    assert not unimodal(f)
    # the oracle's stop rule on the same P sequence
    phi, first = 0.0, n_avail
    for n in range(n_avail):
        D = lambda m: cost["c0"] + cost["c1"] * m + cost["c2"] * m * m
        g = math.exp(float(scores[n])) * D(n) - (1 + phi) * (D(n + 1) - D(n))
        if g <= 0:
            first = n
            break
        phi += math.exp(float(scores[n]))
    assert first != int(np.argmax(f))


@pytest.mark.parametrize("V,ell", [(50, 0), (200, 3000), (1000, 20000)])
def test_uniform_row_closed_form(V, ell):
    # B = 1, uniform row: every node has P = 1/V; the stop is the first n
    # with D(n)/V <= (1 + n/V) * (D(n+1) - D(n)).
    L = np.zeros((1, V), np.float32)
    ad = oracle.adaptive(L, V, ell, COST)
    c = COST

    def D(n):
        return c["C_d"] + c["c0"] + c["c1"] * n + c["c2"] * n * n + \
            c["c_ell"] * ell * n
    want = V
    for n in range(V):
        if D(n) / V <= (1 + n / V) * (D(n + 1) - D(n)):
            want = n
            break
    # P is exp(fp32(-ln V)) rather than 1/V exactly; the boundary is not
    # within a rounding of a tie for these sizes
    assert ad["n_star"] == want


def test_fixed_budget_without_cost():
    B, V = 4, 100
    L, _, ctx = synth.adaptive_round(5, 1, B, V)
    ad = oracle.adaptive(L[0], 64, int(ctx[0]), None)
    assert ad["n_star"] == 64


def test_longer_context_never_grows_the_budget():
    B, V, n_max = 8, 4000, 512
    L, _, _ = synth.adaptive_round(9, 1, B, V, req0=3)
    prev = None
    for ell in (512, 2048, 8192, 32768):
        ns = oracle.adaptive(L[0], n_max, ell, COST)["n_star"]
        if prev is not None:
            assert ns <= prev
        prev = ns
