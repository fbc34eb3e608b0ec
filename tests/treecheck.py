"""Independent checkers used by the oracle pins and the GPU parity tests.

Nothing here computes what the library computes; these are structural
checks, brute-force enumerations on tiny inputs and the comparison protocol
(exact / near-tie / fail bins)."""
from __future__ import annotations

import itertools
import math

import numpy as np

NEAR_TIE = 1e-5
SCORE_TOL = 1e-4


def key_sort_pool(scores, ppids, toks):
    """Indices sorted by (score desc, parent pool id asc, token asc)."""
    return sorted(range(len(scores)),
                  key=lambda i: (-float(scores[i]), int(ppids[i]), int(toks[i])))


def check_structure(tok, parent, depth, n, B=None):
    """Ancestor-closed, topological, depth = parent depth + 1, distinct
    sibling tokens; pads after n."""
    kids = {}
    for i in range(n):
        p = int(parent[i])
        assert -1 <= p < i, f"node {i}: parent {p} not before it"
        want = 1 if p < 0 else int(depth[p]) + 1
        assert int(depth[i]) == want, f"node {i}: depth {depth[i]} != {want}"
        if B is not None:
            assert 1 <= int(depth[i]) <= B
        key = (p, int(tok[i]))
        assert key not in kids, f"node {i}: duplicate sibling token {tok[i]}"
        kids[key] = i
    for i in range(n, len(tok)):
        assert int(tok[i]) == -1, f"pad {i} has token {tok[i]}"


def path_tokens(tok, parent, i):
    out = []
    while i >= 0:
        out.append(int(tok[i]))
        i = int(parent[i])
    return out[::-1]


def naive_accept(tok, parent, depth, n, target, B):
    """Per-node check: a node is accepted when every node on its root path
    matches the target's token after that node's parent; the answer is the
    deepest accepted node."""
    best, best_d = -1, 0
    for i in range(n):
        ok = True
        j = i
        while j >= 0:
            p = int(parent[j])
            if int(tok[j]) != int(target[p + 1]):
                ok = False
                break
            j = p
        if ok and int(depth[i]) > best_d:
            best, best_d = i, int(depth[i])
    nodes = []
    j = best
    while j >= 0:
        nodes.append(j)
        j = int(parent[j])
    nodes = nodes[::-1]
    toks = [int(tok[j]) for j in nodes] + [int(target[best + 1])]
    an = nodes + [-1] * (B - len(nodes))
    at = toks + [-1] * (B + 1 - len(toks))
    return len(nodes) + 1, an, at


def unimodal(f, tol=0.0):
    """True if f rises (weakly) to a peak and never rises after it."""
    i = int(np.argmax(f))
    rising = all(f[j + 1] >= f[j] - tol for j in range(i))
    falling = all(f[j + 1] <= f[j] + tol for j in range(i, len(f) - 1))
    return rising and falling


def enumerate_prefixes(child_lp, B, V):
    """All token prefixes of length 1..B with fp32 path scores, where
    child_lp(prefix_tokens, depth) returns the fp32 log-probs of the V tokens
    at that depth given the prefix.  Returns list of (score, tokens)."""
    out = []
    frontier = [((), np.float32(0.0))]
    for d in range(1, B + 1):
        nxt = []
        for pre, s in frontier:
            lp = child_lp(pre, d)
            for v in range(V):
                sc = np.float32(s + np.float32(lp[v])) + np.float32(0.0)
                nxt.append((pre + (v,), sc))
        out.extend((float(sc), pre) for pre, sc in nxt)
        frontier = nxt
    return out


def closed_subsets(prefixes, n):
    """All ancestor-closed sets of n prefixes (tiny inputs only)."""
    pset = [p for _, p in prefixes]
    for combo in itertools.combinations(range(len(pset)), n):
        chosen = {pset[i] for i in combo}
        if all(len(p) == 1 or p[:-1] in chosen for p in chosen):
            yield combo
