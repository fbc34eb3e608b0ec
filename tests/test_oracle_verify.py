"""Pins of the oracle's ancestry mask and acceptance walk (CPU only): the
pages' worked example, a naive per-node path check on random trees, and mask
invariants."""
import json
import os

import numpy as np
import pytest

import oracle
from treecheck import naive_accept

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_four_accepted_plus_one_correction():
    g = json.load(open(os.path.join(GOLD, "accept_worked_example.json")))
    tok = np.array(g["tok"], np.int32)
    par = np.array(g["parent"], np.int32)
    tau, an, at = oracle.accept(tok, par, len(tok), g["B"],
                                np.array(g["target"], np.int32))
    assert tau == g["expected_tau"] == 5
    assert list(an) == g["expected_accept_node"]
    assert list(at) == g["expected_accept_tok"]


def random_tree(rng, n, B, V):
    """Random topologically ordered tree with distinct sibling tokens (at most
    V children per node, depth at most B)."""
    tok = np.empty(n, np.int32)
    par = np.empty(n, np.int32)
    dep = np.empty(n, np.int32)
    used = {}
    nkids = {}
    for i in range(n):
        # parents that can still take a child: the root (-1) or earlier nodes
        ok = [p for p in range(-1, i)
              if nkids.get(p, 0) < V and (p < 0 or dep[p] < B)]
        if not ok:  # tree is full: return the nodes built so far
            return tok[:i].copy(), par[:i].copy(), dep[:i].copy()
        p = int(ok[int(rng.integers(0, len(ok)))])
        d = 1 if p < 0 else int(dep[p]) + 1
        free = [t for t in range(V) if (p, t) not in used]
        t = int(free[int(rng.integers(0, len(free)))])
        used[(p, t)] = i
        nkids[p] = nkids.get(p, 0) + 1
        tok[i], par[i], dep[i] = t, p, d
    return tok, par, dep


def test_walk_equals_naive_check_on_random_trees():
    rng = np.random.default_rng(0)
    for trial in range(3000):
        B = int(rng.integers(1, 7))
        n = int(rng.integers(0, 30))
        V = int(rng.integers(2, 6))  # small V: many matches
        tok, par, dep = random_tree(rng, n, B, V)
        n = len(tok)
        N = n + int(rng.integers(0, 3))
        tokp = np.concatenate([tok, -np.ones(N - n, np.int32)])
        parp = np.concatenate([par, -np.ones(N - n, np.int32)])
        depp = np.concatenate([dep, np.zeros(N - n, np.int32)])
        target = rng.integers(0, V, size=N + 1).astype(np.int32)
        tau, an, at = oracle.accept(tokp, parp, n, B, target)
        t2, an2, at2 = naive_accept(tokp, parp, depp, n, target, B)
        assert (tau, list(an), list(at)) == (t2, an2, at2), trial


def test_all_match_and_none_match():
    B = 6
    tok = np.array([3, 4, 5, 6, 7, 8], np.int32)
    par = np.array([-1, 0, 1, 2, 3, 4], np.int32)
    tgt = np.array([3, 4, 5, 6, 7, 8, 42], np.int32)
    tau, an, at = oracle.accept(tok, par, 6, B, tgt)
    assert tau == B + 1 and list(at) == [3, 4, 5, 6, 7, 8, 42]
    tgt0 = np.array([9, 4, 5, 6, 7, 8, 42], np.int32)
    tau, an, at = oracle.accept(tok, par, 6, B, tgt0)
    assert tau == 1 and list(at) == [9] + [-1] * B and list(an) == [-1] * B


def _bits(mask_row, N):
    return [(int(mask_row[j // 64]) >> (j % 64)) & 1 for j in range(N)]


def test_mask_chain_star_and_invariants():
    N = 130  # three words per row, ragged last word
    # chain: lower-triangular ones
    par = np.arange(-1, N - 1, dtype=np.int32)
    m = oracle.mask(par, N, N)
    for i in range(N):
        assert _bits(m[i], N) == [1] * (i + 1) + [0] * (N - i - 1)
    # star: identity
    par = -np.ones(N, np.int32)
    m = oracle.mask(par, N, N)
    for i in range(N):
        assert _bits(m[i], N) == [int(j == i) for j in range(N)]
    # random: popcount = depth, row(i) contains row(parent(i)), pads zero
    rng = np.random.default_rng(3)
    tok, par, dep = random_tree(rng, 100, 12, 50)
    parp = np.concatenate([par, -np.ones(N - 100, np.int32)])
    m = oracle.mask(parp, 100, N)
    for i in range(100):
        assert sum(_bits(m[i], N)) == dep[i]
        if par[i] >= 0:
            assert np.all((m[i] & m[par[i]]) == m[par[i]])
    assert not m[100:].any()
