"""Pins of the oracle's parent-conditioned tree (CPU only): the greedy chain
special case, the best-first exact case, brute-force enumeration without
pruning, the beam rule, closed-form ties and structural invariants."""
import math

import numpy as np
import pytest

import oracle
import synth
from treecheck import (check_structure, enumerate_prefixes, key_sort_pool,
                       path_tokens)


def _inputs(seed, batch, B, V, r, bf16=True, scale_m=1.0):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(batch, B, V)) * 1.7).astype(np.float32)
    if r == 0:
        return L, None, None, rng.integers(0, V, size=batch).astype(np.int32)
    U = (rng.normal(size=(V, r)) / math.sqrt(r) * scale_m).astype(np.float32)
    W = (rng.normal(size=(V, r)) / math.sqrt(r) * scale_m).astype(np.float32)
    if bf16:
        U, W = synth.bf16_bits(U), synth.bf16_bits(W)
    A = rng.integers(0, V, size=batch).astype(np.int32)
    return L, U, W, A


@pytest.mark.parametrize("r", [0, 8])
def test_k1_is_the_greedy_chain(r):
    # k = 1, N = B: the tree is the chain of the Markov-head drafter.
    batch, B, V = 3, 6, 300
    L, U, W, A = _inputs(10 + r, batch, B, V, r, scale_m=3.0)
    t = oracle.build_tree(L, U, W, A, k=1, beam_w=4, N=B)
    for q in range(batch):
        chain = oracle.greedy_chain(L[q], U, W, int(A[q]))
        assert list(t["tok"][q]) == list(chain)
        assert list(t["parent"][q]) == list(range(-1, B - 1))
        assert list(t["depth"][q]) == list(range(1, B + 1))
        assert t["n_nodes"][q] == B


@pytest.mark.parametrize("r,N", [(0, 10), (8, 10), (8, 25)])
def test_wide_beam_equals_bestfirst(r, N):
    # k >= N and beam >= N: every prefix among the N best survives each
    # stage, so PCTree's top-N equals the best-first tree of N nodes.
    batch, B, V = 2, 4, 60
    L, U, W, A = _inputs(20 + N + r, batch, B, V, r, scale_m=2.0)
    t = oracle.build_tree(L, U, W, A, k=N, beam_w=N, N=N)
    for q in range(batch):
        bf = oracle.bestfirst(L[q], U, W, int(A[q]), N)
        assert bf["n"] == N
        assert list(t["tok"][q]) == list(bf["tok"])
        assert list(t["parent"][q]) == list(bf["parent"])
        assert np.array_equal(t["score"][q], bf["score"])


def test_no_pruning_equals_enumeration():
    # Beam wide enough to keep every child: the pool is the full k-ary tree
    # of per-parent top-k children, and the output is its top-N by key.
    B, V, k, r = 3, 12, 3, 6
    L, U, W, A = _inputs(31, 1, B, V, r)
    N = 20
    t = oracle.build_tree(L, U, W, A, k=k, beam_w=k ** B, N=N)
    nodes = []  # (score, parent pool id, token, token path)
    level = [((), np.float32(0.0), -1, int(A[0]))]  # path, s, pool id, token
    base = 0
    for d in range(1, B + 1):
        nxt = []
        for j, (path, s, par_id, ptok) in enumerate(level):
            M = oracle.markov_row(U, W, ptok)
            lse, tt, tz, _ = oracle.row_stats(L[0, d - 1], M, k)
            for i in range(k):
                sc = np.float32(s + np.float32(tz[i] - np.float32(lse)))
                sc = np.float32(sc + np.float32(0.0))
                nodes.append((float(sc), par_id, int(tt[i]),
                              path + (int(tt[i]),)))
                nxt.append((path + (int(tt[i]),), sc, base + j * k + i,
                            int(tt[i])))
        base += len(level) * k
        level = nxt
    order = sorted(nodes, key=lambda x: (-x[0], x[1], x[2]))[:N]
    got = [tuple(path_tokens(t["tok"][0], t["parent"][0], i))
           for i in range(N)]
    assert got == [x[3] for x in order]
    assert np.array_equal(t["score"][0], np.array([x[0] for x in order],
                                                  np.float32))


def test_beam_rule_and_pool():
    # Every stage's beam is the top-W of the children of the previous beam,
    # by (score desc, parent id asc, token asc); the output is the top-N of
    # the whole pool.
    batch, B, V, k, Wb, N, r = 2, 5, 200, 3, 4, 14, 8
    L, U, W, A = _inputs(41, batch, B, V, r, scale_m=2.0)
    t = oracle.build_tree(L, U, W, A, k=k, beam_w=Wb, N=N, diagnostics=True)
    pool = oracle.pool_size(batch, B, V, r, k, Wb, N)
    assert t["pool_tok"].shape[1] == pool
    for q in range(batch):
        ps, pp, pt = t["pool_score"][q], t["pool_ppid"][q], t["pool_tok"][q]
        base, front = 0, [-1]
        for d in range(1, B + 1):
            nc = len(front) * k
            ids = list(range(base, base + nc))
            # children ids are grouped by parent in frontier order
            for j, par in enumerate(front):
                for i in range(k):
                    assert pp[base + j * k + i] == par
            srt = sorted(ids, key=lambda i: (-float(ps[i]), int(pp[i]),
                                             int(pt[i])))
            want = srt[:Wb]
            got = [int(x) for x in t["beam_pid"][q, d - 1] if x >= -1]
            assert got == want
            front = want
            base += nc
        top = key_sort_pool(ps, pp, pt)[:N]
        assert list(t["tok"][q]) == [int(pt[i]) for i in top]
        assert np.array_equal(t["score"][q], ps[top])


def test_structure_and_path_scores():
    batch, B, V, k, Wb, N, r = 3, 7, 500, 4, 6, 40, 16
    L, U, W, A = _inputs(51, batch, B, V, r, scale_m=2.0)
    t = oracle.build_tree(L, U, W, A, k=k, beam_w=Wb, N=N)
    for q in range(batch):
        n = int(t["n_nodes"][q])
        assert n == N
        check_structure(t["tok"][q], t["parent"][q], t["depth"][q], n, B)
        sc = t["score"][q]
        assert all(sc[i] >= sc[i + 1] for i in range(n - 1))
        # recompute every path's log-probability in double
        for i in range(n):
            toks = path_tokens(t["tok"][q], t["parent"][q], i)
            prev, s = int(A[q]), 0.0
            for d, v in enumerate(toks, start=1):
                M = oracle.markov_row(U, W, prev).astype(np.float64)
                z = L[q, d - 1].astype(np.float64) + M
                m = z.max()
                s += z[v] - (m + math.log(np.exp(z - m).sum()))
                prev = v
            assert abs(s - float(sc[i])) < 1e-4


def test_uniform_rows_closed_form():
    # All logits equal and no Markov term: every child has log-prob -ln V,
    # ties are broken by parent id then token, so the beam expands the
    # first W parents (by pool id) and children are tokens 0..k-1.
    batch, B, V, k, Wb, N = 1, 3, 50, 3, 2, 10
    L = np.zeros((batch, B, V), np.float32)
    t = oracle.build_tree(L, None, None, np.array([7], np.int32), k=k,
                          beam_w=Wb, N=N)
    lp = np.float32(np.float32(0.0) - np.float32(math.log(V)))
    # depth 1: tokens 0..2 (ids 0,1,2); beam = ids 0,1
    # depth 2: children of id 0 (ids 3,4,5), of id 1 (ids 6,7,8); beam 3,4
    # depth 3: children of 3 (ids 9..11), of 4 (ids 12..14)
    want_tok = [0, 1, 2, 0, 1, 2, 0, 1, 2, 0]
    want_par = [-1, -1, -1, 0, 0, 0, 1, 1, 1, 3]
    want_dep = [1, 1, 1, 2, 2, 2, 2, 2, 2, 3]
    assert list(t["tok"][0]) == want_tok
    assert list(t["parent"][0]) == want_par
    assert list(t["depth"][0]) == want_dep
    s1 = lp
    s2 = np.float32(s1 + lp)
    assert t["score"][0][0] == s1 and t["score"][0][3] == s2


def test_small_pool_pads():
    # pool (k * ...) smaller than N: all candidates are kept, rest padded
    batch, B, V, k, Wb, N = 1, 2, 30, 2, 1, 10
    L, _, _, A = _inputs(61, batch, B, V, 0)
    t = oracle.build_tree(L, None, None, A, k=k, beam_w=Wb, N=N)
    assert t["n_nodes"][0] == 4
    assert list(t["tok"][0][4:]) == [-1] * 6
    assert list(t["parent"][0][4:]) == [-1] * 6
    assert np.all(np.isneginf(t["score"][0][4:]))
