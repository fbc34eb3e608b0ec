"""Pins of the oracle's adaptive build over parent-conditioned rows (the
throughput stop of the CaDDTree summary, "Method", on the PCTree article's
Markov-conditioned tree) and of its throughput curve (CPU only):

- brute force: on tiny vocabularies every prefix is enumerated and sorted
  by probability; the stop chosen by the oracle is the smallest maximiser
  of f(n) = (1 + Phi_n) / D(n) over that order, and the kept nodes are the
  n* most probable prefixes;
- f is unimodal along the best-first order under a convex cost, and a
  concave cost can break that (negative control);
- the beam tree with k = beam = N >= n* (a derived lemma: every top-N
  prefix survives such a beam) stopped by the same rule keeps the same
  prefixes;
- the throughput curve matches its definition on closed-form rows.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from treecheck import enumerate_prefixes, path_tokens, unimodal

COST = dict(C_d=1.0, c0=2.0, c1=0.004, c2=2e-6, c_ell=1e-5)


def _lp_fn(L, U, W, anchor):
    V = L.shape[1]

    def f(prefix, d):
        prev = anchor if not prefix else prefix[-1]
        M = oracle.markov_row(U, W, prev)
        lse, tt, tz, _ = oracle.row_stats(L[d - 1], M, V)
        lp = np.empty(V, np.float32)
        lp[tt] = (tz - np.float32(lse)).astype(np.float32)
        return lp
    return f


def _tiny(seed, B, V, r, scale=1.5):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(B, V)) * scale).astype(np.float32)
    U = synth.bf16_bits((rng.normal(size=(V, r)) * 0.8).astype(np.float32))
    W = synth.bf16_bits((rng.normal(size=(V, r)) * 0.8).astype(np.float32))
    return L, U, W


def _D(c, n, ell):
    return c["C_d"] + c["c0"] + c["c1"] * n + c["c2"] * n * n + \
        c["c_ell"] * ell * n


@pytest.mark.parametrize("seed,B,V,ell,c1", [(1, 3, 5, 100, 0.004),
                                             (2, 4, 4, 3000, 0.02),
                                             (3, 3, 6, 20000, 0.001),
                                             (4, 4, 3, 600, 0.05)])
def test_stop_is_the_best_prefix_count_by_brute_force(seed, B, V, ell, c1):
    L, U, W = _tiny(seed, B, V, 4)
    anchor = 1
    cost = dict(COST, c1=c1)
    pre = enumerate_prefixes(_lp_fn(L, U, W, anchor), B, V)
    order = sorted(pre, key=lambda x: -x[0])
    P = [math.exp(s) for s, _ in order]
    f = []
    phi = 0.0
    for n in range(len(order) + 1):
        f.append((1.0 + phi) / _D(cost, n, ell))
        if n < len(order):
            phi += P[n]
    best = max(f)
    want = min(n for n in range(len(f)) if f[n] >= best * (1 - 1e-12))
    ad = oracle.adaptive(L, len(order), ell, cost, U=U, W=W, anchor=anchor)
    assert ad["n_star"] == want
    got = {tuple(path_tokens(ad["tok"], ad["parent"], i))
           for i in range(ad["n_star"])}
    assert got == {p for _, p in order[:want]}
    assert abs(ad["phi"] - sum(P[:want])) < 1e-12
    assert abs(ad["throughput"] - f[want]) < 1e-12 * f[want]
    assert unimodal(f, tol=1e-15)


def test_concave_cost_can_break_unimodality():
    # a cost that falls after rising is not convex: f can rise again, and
    # the first non-positive gain is then not the best prefix count
    L, U, W = _tiny(9, 3, 4, 4, scale=0.3)
    pre = enumerate_prefixes(_lp_fn(L, U, W, 0), 3, 4)
    s = sorted((x for x, _ in pre), reverse=True)
    f = []
    phi = 0.0
    for n in range(len(s) + 1):
        D = 1.0 + 2.0 * min(n, 3) - 0.5 * max(0, n - 3)
        f.append((1.0 + phi) / max(D, 1e-3))
        if n < len(s):
            phi += math.exp(s[n])
    assert not unimodal(f)


@pytest.mark.parametrize("seed,B,V,r,n_max", [(11, 4, 300, 16, 12),
                                              (12, 5, 500, 32, 16),
                                              (13, 3, 200, 8, 20)])
def test_beam_tree_with_k_beam_n_at_least_n_star(seed, B, V, r, n_max):
    # PCTree with k = beam = N = n_max keeps every one of the n_max most
    # probable prefixes (derived lemma), so its key-ordered output stopped
    # by the same rule keeps the same prefixes as the best-first build
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(1, B, V)) * 2.0).astype(np.float32)
    U, W = synth.markov_factors(seed, V, r, True)
    A = np.array([int(rng.integers(0, V))], np.int32)
    ell = 4000
    for cost in (COST, dict(COST, c1=0.02, c0=0.5)):
        ad = oracle.adaptive(L[0], n_max, ell, cost, U=U, W=W, anchor=A[0])
        t = oracle.build_tree(L, U, W, A, n_max, n_max, n_max)
        n = int(t["n_nodes"][0])
        st = oracle.stop(t["score"][0], n, ell, cost)
        assert st["n_star"] == ad["n_star"]
        a = {tuple(path_tokens(ad["tok"], ad["parent"], i))
             for i in range(ad["n_star"])}
        b = {tuple(path_tokens(t["tok"][0], t["parent"][0], i))
             for i in range(st["n_star"])}
        assert a == b
        assert abs(st["phi"] - ad["phi"]) <= 1e-12 * max(1.0, ad["phi"])


def test_no_cost_model_keeps_the_budget():
    L, U, W = _tiny(21, 3, 5, 4)
    ad = oracle.adaptive(L, 17, 100, None, U=U, W=W, anchor=2)
    assert ad["n_star"] == 17
    bf = oracle.bestfirst(L, U, W, 2, 17)
    assert np.array_equal(ad["tok"], bf["tok"])
    assert np.array_equal(ad["parent"], bf["parent"])


def test_throughput_curve_closed_form():
    # B = 1, uniform row of V tokens: P_i = 1/V (to fp32 rounding), so
    # f(n) = (1 + n/V) / D(n) up to that rounding
    V, ell = 300, 2500
    L = np.zeros((1, V), np.float32)
    bf = oracle.bestfirst(L, None, None, 0, V)
    f = oracle.throughput_curve(bf["score"], bf["n"], ell, COST)
    assert f.shape == (V + 1,)
    for n in (0, 1, 7, 150, V):
        want = (1.0 + n / V) / _D(COST, n, ell)
        assert abs(f[n] - want) < 1e-6 * want
    st = oracle.stop(bf["score"], bf["n"], ell, COST)
    best = max(f)
    assert st["n_star"] == min(n for n in range(V + 1) if f[n] == best)
    g = oracle.throughput_curve(bf["score"], bf["n"], ell, None)
    assert abs(g[V] - 2.0) < 1e-5 and g[0] == 1.0
