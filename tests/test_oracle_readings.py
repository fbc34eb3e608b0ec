"""Pins of the oracle's readings where the pages leave a detail open (CPU
only).  Each case is built so that a plausible alternative reading, or a
slip in the oracle, gives a different answer:

- sibling order at an exact fp32 score tie in the best-first tree: the
  sibling with the larger logit (the more probable prefix) comes first;
- the stop rule: a gain that is exactly zero stops the build (CaDDTree
  summary, "Method": nodes are added while the gain is positive);
- the log-normaliser is the exactly rounded double value, not an fp32 sum;
- the path score adds the edge log-probability log pi = z - lse to the
  parent's score (the sum of per-edge log-probabilities of the PCTree
  article, "straight draft"), which keeps it exact even when the logits
  themselves are huge.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from treecheck import path_tokens

pytestmark = pytest.mark.filterwarnings("ignore")


def _f32(x):
    return float(np.float32(x))


def _true_lse(row):
    """log sum exp of a float32 row, from an exactly rounded sum of the
    double exponentials (math.fsum), in double."""
    z = np.asarray(row, np.float64)
    m = float(z.max())
    return m + math.log(math.fsum(np.exp(z - m).tolist()))


def _tie_row(V=6, lo=1, hi=2, big=3):
    """A row where tokens lo < hi carry logits 0.0010000 < 0.0010001 and a
    token of logit 20 sets lse near 20: both log-probabilities round to the
    same fp32 value although the logits differ."""
    row = np.full(V, -50.0, np.float32)
    row[big] = 20.0
    row[lo] = np.float32(0.0010000)
    row[hi] = np.float32(0.0010001)
    return row


def _double_prefix_logprob(L, toks):
    """Prefix log-probability of a token path over marginal rows, in
    double (each edge: z - lse with lse from an exactly rounded sum)."""
    s = 0.0
    for d, v in enumerate(toks):
        s += float(L[d][v]) - _true_lse(L[d])
    return s


@pytest.mark.parametrize("B", [1, 2])
def test_sibling_tie_goes_to_the_larger_logit(B):
    L = np.stack([_tie_row() for _ in range(B)])
    lse, tt, tz, _ = oracle.row_stats(L[0], None, 6)
    # precondition: equal fp32 log-probabilities, different logits
    l_lo = np.float32(np.float32(L[0][1]) - np.float32(lse))
    l_hi = np.float32(np.float32(L[0][2]) - np.float32(lse))
    assert l_lo == l_hi and L[0][1] < L[0][2]
    n_all = sum(6 ** d for d in range(1, B + 1))
    bf = oracle.bestfirst(L, None, None, 0, n_all)
    n = bf["n"]
    assert n == n_all
    seen_tie = 0
    for i in range(n - 1):
        if bf["score"][i] != bf["score"][i + 1]:
            continue
        if bf["parent"][i] != bf["parent"][i + 1]:
            continue  # other parents: the parent's output index decides
        a = path_tokens(bf["tok"], bf["parent"], i)
        b = path_tokens(bf["tok"], bf["parent"], i + 1)
        pa = _double_prefix_logprob(L, a)
        pb = _double_prefix_logprob(L, b)
        # siblings at an exact fp32 tie: the truly more probable prefix goes
        # first (or the two are equally probable)
        assert pa >= pb, (i, a, b, pa, pb)
        seen_tie += pa > pb
    # the planted pair (and, at depth 2, the pairs under every parent)
    assert seen_tie >= 1
    # the planted depth-1 pair explicitly: token 2 before token 1
    d1 = [int(t) for t, p in zip(bf["tok"][:n], bf["parent"][:n]) if p == -1]
    assert d1.index(2) < d1.index(1)


def test_sibling_tie_in_the_adaptive_build():
    L = np.stack([_tie_row(), _tie_row()])
    ad = oracle.adaptive(L, 42, 0, None)
    d1 = [int(t) for t, p in zip(ad["tok"][:ad["n_star"]],
                                 ad["parent"][:ad["n_star"]]) if p == -1]
    assert d1.index(2) < d1.index(1)


@pytest.mark.parametrize("c1,want", [(1.0, 0), (1.0 - 2.0 ** -20, 4),
                                     (1.0 + 2.0 ** -20, 0)])
def test_zero_gain_stops(c1, want):
    # A one-token vocabulary: every prefix has probability exactly 1
    # (lse = z, log pi = 0), so Phi_n = n.  With D(n) = 1 + c1 n the gain
    # P_{n+1} D(n) - (1 + Phi_n)(D(n+1) - D(n)) = 1 - c1 is exactly zero
    # for c1 = 1: a non-positive gain stops at once (n* = 0); a slightly
    # cheaper node keeps every gain positive (all 4 nodes); a slightly
    # dearer one stops at once.
    L = np.array([[3.5], [-2.0], [0.25], [7.0]], np.float32)
    cost = dict(C_d=1.0, c0=0.0, c1=c1, c2=0.0, c_ell=0.0)
    ad = oracle.adaptive(L, 16, 100, cost)
    assert ad["n_star"] == want
    assert ad["phi"] == float(want)
    # f(n) = (1 + n) / (1 + c1 n): constant at c1 = 1, so the smallest
    # maximiser is n = 0
    f = [(1.0 + n) / (1.0 + c1 * n) for n in range(5)]
    best = max(f)
    assert min(n for n in range(5) if f[n] == best) == want


def test_lse_is_the_rounded_double_value():
    # rows of the b16 workload's shape and spread, one at each temperature
    # extreme: the oracle's fp32 log-normaliser is within one fp32 ulp of
    # the exactly summed double value (an fp32 running sum of 151936 terms
    # is off by tens of ulps)
    V = 151936
    L = synth.drafter_logits(911, 3, 2, V, 3.0, (0.5, 2.0))
    for q in range(3):
        for d in range(2):
            row = L[q, d]
            lse, _, _, _ = oracle.row_stats(row, None, 1)
            want = _true_lse(row)
            ulp = float(np.spacing(np.float32(abs(want))))
            assert abs(lse - want) <= ulp, (q, d, lse, want, ulp)
    # the same for z = L + M with a Markov row (one fp32 add per element)
    U, W = synth.markov_factors(911, V, 32, True)
    M = oracle.markov_row(U, W, 17)
    z = (L[0, 0] + M).astype(np.float32)
    lse, _, _, _ = oracle.row_stats(L[0, 0], M, 1)
    want = _true_lse(z)
    assert abs(lse - want) <= float(np.spacing(np.float32(abs(want))))


def _huge_rows():
    # depth 1: two equal logits, log pi = -ln 2; depth 2: logits near 2^24
    # whose lse is 2^24 exactly (the second term is e^-1024 = 0 in double)
    L = np.zeros((2, 2), np.float32)
    L[1] = [2.0 ** 24, 2.0 ** 24 - 1024.0]
    return L


def test_path_score_adds_the_edge_log_prob_tree():
    # PCTree without a Markov term: the child of a depth-1 node must score
    # -ln 2 + 0 (the edge log-prob z - lse is 0 exactly); adding the parent's
    # score to the logit first would lose the fraction at 2^24 and give -1
    L = _huge_rows()[None]
    o = oracle.build_tree(L, None, None, np.array([0], np.int32), 2, 2, 6)
    n = int(o["n_nodes"][0])
    for i in range(n):
        toks = path_tokens(o["tok"][0], o["parent"][0], i)
        want = _double_prefix_logprob(L[0], toks)
        assert abs(float(o["score"][0][i]) - want) < 1e-4, (i, toks)


def test_path_score_adds_the_edge_log_prob_bestfirst():
    L = _huge_rows()
    bf = oracle.bestfirst(L, None, None, 0, 6)
    for i in range(bf["n"]):
        toks = path_tokens(bf["tok"], bf["parent"], i)
        want = _double_prefix_logprob(L, toks)
        assert abs(float(bf["score"][i]) - want) < 1e-4, (i, toks)
