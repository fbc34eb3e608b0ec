"""CPU checks of the comparison protocol used by the GPU parity tests
(tests/parity.py): an unchanged oracle tree is EXACT, a tree with a planted
mistake FAILS, and a tree built from inputs nudged across a planted
near-tie is excused as NEAR only because the tie sits at the first
differing node."""
import numpy as np
import pytest

import oracle
import synth
from parity import RequestContext, classify

K, BEAM, N = 4, 6, 24


def _inputs(seed=5, B=3, V=400, r=32):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(1, B, V)) * 1.7).astype(np.float32)
    U, W = synth.markov_factors(seed, V, r, True)
    A = np.array([7], np.int32)
    return L, U, W, A


def _ctx(L, U, W, A):
    return RequestContext(L[0], U, W, A[0], K, BEAM, N)


def test_same_tree_is_exact():
    L, U, W, A = _inputs()
    o = oracle.build_tree(L, U, W, A, K, BEAM, N)
    g = {k: v.copy() for k, v in o.items()}
    assert classify(g, o, 0, _ctx(L, U, W, A))[0] == "exact"


@pytest.mark.parametrize("mistake", ["swap_far", "wrong_token", "score"])
def test_planted_mistakes_fail(mistake):
    L, U, W, A = _inputs()
    o = oracle.build_tree(L, U, W, A, K, BEAM, N)
    g = {k: v.copy() for k, v in o.items()}
    n = int(o["n_nodes"][0])
    if mistake == "swap_far":
        # two depth-1 siblings far apart in score swap places
        d1 = [i for i in range(n) if g["parent"][0][i] == -1]
        i, j = d1[0], d1[-1]
        assert o["score"][0][i] - o["score"][0][j] > 1e-3
        g["tok"][0][[i, j]] = g["tok"][0][[j, i]]
    elif mistake == "wrong_token":
        # a leaf replaced by a token outside its parent's top-k
        leaf = n - 1
        g["tok"][0][leaf] = (int(g["tok"][0][leaf]) + 123) % L.shape[2]
    else:
        g["score"][0][3] += 1e-3
    with pytest.raises(AssertionError):
        classify(g, o, 0, _ctx(L, U, W, A))


def test_nudged_tie_is_near_only_at_the_tie():
    L, U, W, A = _inputs(seed=9)
    o = oracle.build_tree(L, U, W, A, K, BEAM, N)
    # plant a near-tie at the root's top-k boundary: the (K+1)-th token gets
    # the K-th token's logit minus 2e-6, then a copy is nudged 4e-6 up so
    # that the two swap.  The oracle on the planted inputs is the reference,
    # the oracle on the nudged inputs plays the GPU.
    M = oracle.markov_row(U, W, int(A[0]))
    lse, tt, tz, _ = oracle.row_stats(L[0, 0], M, K + 1)
    kth, nxt = int(tt[K - 1]), int(tt[K])
    Lp = L.copy()
    Lp[0, 0, nxt] = np.float32(tz[K - 1] - M[nxt] - np.float32(2e-6))
    Ln = Lp.copy()
    Ln[0, 0, nxt] = np.float32(Lp[0, 0, nxt] + np.float32(4e-6))
    o = oracle.build_tree(Lp, U, W, A, K, BEAM, N)
    g = oracle.build_tree(Ln, U, W, A, K, BEAM, N)
    ctx = _ctx(Lp, U, W, A)
    res, why = classify(g, o, 0, ctx)
    assert res == "near", why
    # the same difference without the tie in the reference is a failure
    o2 = oracle.build_tree(L, U, W, A, K, BEAM, N)
    if not np.array_equal(o2["tok"][0], g["tok"][0]):
        with pytest.raises(AssertionError):
            classify(g, o2, 0, _ctx(L, U, W, A))
