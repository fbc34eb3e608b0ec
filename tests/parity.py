"""Comparison protocol of the GPU parity tests: every request lands in one
of three bins.

EXACT  tok, parent, depth and n_nodes equal bit for bit, scores within 1e-4.
NEAR   the trees differ, and the difference is explained by a near-tie of
       the oracle (a gap below 1e-5) AT THE FIRST DIFFERING NODE:
        - the GPU's node there is in the oracle's pool and its oracle score
          is within 1e-5 of the oracle's node there (an ordering tie); or
        - the oracle's node there is missing from the GPU tree and sits at a
          selection boundary of the oracle (its parent's top-k, or the beam
          that expanded its parent) within 1e-5; or
        - the GPU's node there is not in the oracle's pool: its first
          ancestor-or-self c outside the pool sits at the oracle's top-k
          boundary of c's parent, or c's parent lost the oracle's beam at a
          boundary gap below 1e-5.
       A near-tie request must also be a valid tree: structure; every score
       equal to the oracle's recomputation along its path within 1e-4;
       every child in its parent's oracle top-k with 1e-5 slack; and, when
       the difference is an ordering tie among nodes of the oracle's pool,
       the GPU tree's Phi at least the oracle's minus N * 1e-5 * max P.  (A
       tie at a top-k or beam boundary hands the beam a different subtree,
       whose mass is unrelated to the size of the gap, so no Phi bound
       follows from it.)
FAIL   anything else.

The oracle supplies pools, rows and gaps on demand (only for requests that
are not exact); the checks themselves are written here.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from treecheck import NEAR_TIE, SCORE_TOL, check_structure, path_tokens


def _same_tree(g, o, q):
    n_o, n_g = int(o["n_nodes"][q]), int(g["n_nodes"][q])
    return (n_o == n_g and np.array_equal(g["tok"][q], o["tok"][q]) and
            np.array_equal(g["parent"][q], o["parent"][q]) and
            np.array_equal(g["depth"][q], o["depth"][q]))


def first_diff(g, o, q):
    """Index of the first output node where the two trees differ."""
    n = max(int(o["n_nodes"][q]), int(g["n_nodes"][q]))
    N = g["tok"].shape[1]
    for i in range(min(max(n, 1), N)):
        if (g["tok"][q][i] != o["tok"][q][i] or
                g["parent"][q][i] != o["parent"][q][i] or
                g["depth"][q][i] != o["depth"][q][i]):
            return i
    return None


class RequestContext:
    """One request's inputs and lazily computed oracle diagnostics."""

    def __init__(self, L, U, W, anchor, k, beam_w, N):
        self.L, self.U, self.W = L, U, W
        self.anchor = int(anchor)
        self.k, self.beam_w, self.N = k, beam_w, N
        self.B = L.shape[0]
        self._diag = None
        self._rows = {}

    def diag(self):
        """The oracle's pool (path -> (score, depth, pool id)), its beams
        and boundary gaps for this request."""
        if self._diag is None:
            d = oracle.build_tree(self.L[None], self.U, self.W,
                                  np.array([self.anchor], np.int32), self.k,
                                  self.beam_w, self.N, diagnostics=True)
            pt, pp, ps = d["pool_tok"][0], d["pool_ppid"][0], d["pool_score"][0]
            paths = {}
            depth_of = {}
            path_of = {}
            for i in range(len(pt)):
                p = int(pp[i])
                pre = () if p < 0 else path_of[p]
                path_of[i] = pre + (int(pt[i]),)
                depth_of[i] = len(path_of[i])
                paths[path_of[i]] = (float(ps[i]), depth_of[i], i)
            beams = set()
            for dd in range(self.B):
                for pid in d["beam_pid"][0][dd]:
                    if pid >= 0:
                        beams.add(path_of[int(pid)])
            self._diag = dict(paths=paths, beams=beams,
                              depth_gap=d["depth_gap"][0])
        return self._diag

    def row(self, prefix):
        """(lse, z row) of the parent whose token path is `prefix` (the
        root for ()), at depth len(prefix) + 1."""
        key = tuple(prefix)
        if key not in self._rows:
            d = len(key) + 1
            prev = self.anchor if not key else key[-1]
            Lr = self.L[d - 1]
            M = None if self.U is None else oracle.markov_row(self.U, self.W,
                                                              prev)
            z = Lr if M is None else (Lr + M).astype(np.float32)
            lse, _, _, _ = oracle.row_stats(Lr, M, 1)
            self._rows[key] = (float(lse), z)
        return self._rows[key]

    def kth_z(self, prefix, i):
        """The i-th largest z (1-based) of a parent's row."""
        _, z = self.row(prefix)
        return float(np.partition(z, len(z) - i)[len(z) - i])


def _topk_boundary_near(ctx, prefix, tok):
    """Does token `tok` sit at the oracle's top-k boundary of the parent
    with path `prefix` (within 1e-5 of the k-th or (k+1)-th logit)?"""
    _, z = ctx.row(prefix)
    zk = ctx.kth_z(prefix, ctx.k)
    zk1 = ctx.kth_z(prefix, ctx.k + 1) if ctx.k < len(z) else -math.inf
    zt = float(z[tok])
    return abs(zt - zk) < NEAR_TIE or abs(zt - zk1) < NEAR_TIE or \
        abs(zk - zk1) < NEAR_TIE


def _beam_boundary_near(ctx, prefix):
    """Did the parent with path `prefix` (depth len(prefix)) fall at the
    oracle's beam boundary of its depth?"""
    dg = ctx.diag()["depth_gap"]
    return float(dg[len(prefix) - 1]) < NEAR_TIE


def _explained_missing(ctx, path):
    """A node of the oracle's tree that the GPU tree lacks: explained by a
    boundary near-tie where it (or an ancestor) was selected."""
    beams = ctx.diag()["beams"]
    for d in range(1, len(path) + 1):
        pre = path[:d - 1]
        if d > 1 and pre not in beams:
            return False  # inconsistent oracle diagnostics
        if _topk_boundary_near(ctx, pre, path[d - 1]):
            return True
        if d > 1 and _beam_boundary_near(ctx, pre):
            return True
    # an ordering tie at the global top-N boundary
    return float(ctx.diag()["depth_gap"][-1]) < NEAR_TIE


def explain_first_diff(g, o, q, ctx):
    """(True, why) if the first differing node is explained by an oracle
    near-tie there, else (False, why)."""
    i = first_diff(g, o, q)
    if i is None:
        return True, "order: scores only"
    n_o, n_g = int(o["n_nodes"][q]), int(g["n_nodes"][q])
    if n_o != n_g:
        return False, f"n_nodes {n_g} != {n_o}"
    paths = ctx.diag()["paths"]
    a = tuple(path_tokens(o["tok"][q], o["parent"][q], i))
    b = tuple(path_tokens(g["tok"][q], g["parent"][q], i))
    g_paths = {tuple(path_tokens(g["tok"][q], g["parent"][q], j))
               for j in range(n_g)}
    if b in paths:
        sb = paths[b][0]
        sa = paths[a][0]
        if abs(sb - sa) < NEAR_TIE:
            return True, f"order: tie at {i}: {sa} vs {sb}"
        if a not in g_paths and _explained_missing(ctx, a):
            return True, f"boundary: oracle node {i} lost at a tie"
        return False, f"node {i}: oracle {a} ({sa}) vs GPU {b} ({sb})"
    # b is not in the oracle's pool: find its first ancestor-or-self c
    # outside the pool
    for d in range(1, len(b) + 1):
        c = b[:d]
        if c in paths:
            continue
        pre = c[:-1]
        if d > 1 and pre not in ctx.diag()["beams"]:
            if _beam_boundary_near(ctx, pre):
                return True, f"boundary: beam tie above {c}"
            return False, f"{c}: parent not expanded by the oracle, no tie"
        if _topk_boundary_near(ctx, pre, c[-1]):
            return True, f"boundary: top-k tie at {c}"
        return False, f"{c}: outside the parent's top-k, no tie"
    return False, "unreachable"


def valid_tree(g, o, q, ctx, check_phi=True):
    """Validity of a near-tie GPU tree (raises AssertionError)."""
    n = int(g["n_nodes"][q])
    tok, par, dep, sc = g["tok"][q], g["parent"][q], g["depth"][q], \
        g["score"][q]
    check_structure(tok, par, dep, n, ctx.B)
    true_s = {}
    maxP = 0.0
    for i in range(n):
        path = tuple(path_tokens(tok, par, i))
        pre = path[:-1]
        lse, z = ctx.row(pre)
        ps = 0.0 if not pre else true_s[pre]
        s = ps + (float(z[path[-1]]) - lse)
        true_s[path] = s
        assert abs(s - float(sc[i])) < SCORE_TOL, (i, s, float(sc[i]))
        zk = ctx.kth_z(pre, ctx.k)
        assert float(z[path[-1]]) >= zk - NEAR_TIE, (i, path)
        maxP = max(maxP, math.exp(s))
    phi_g = sum(math.exp(s) for s in true_s.values())
    n_o = int(o["n_nodes"][q])
    phi_o = sum(math.exp(float(s)) for s in o["score"][q][:n_o])
    maxP = max(maxP, max((math.exp(float(s)) for s in o["score"][q][:n_o]),
                         default=0.0))
    if check_phi:
        assert phi_g >= phi_o - ctx.N * NEAR_TIE * maxP, (phi_g, phi_o)


def classify(g, o, q, ctx):
    """('exact' | 'near', detail); raises AssertionError for FAIL."""
    if _same_tree(g, o, q):
        n = int(o["n_nodes"][q])
        gs = g["score"][q][:n].astype(np.float64)
        os_ = o["score"][q][:n].astype(np.float64)
        # equal scores (-inf included: children of rows with fewer finite
        # logits than k) differ by nothing
        with np.errstate(invalid="ignore"):
            d = np.where(gs == os_, 0.0, np.abs(gs - os_))
        md = float(d.max()) if n else 0.0
        assert md <= SCORE_TOL, (q, f"score diff {md}")
        return "exact", md
    ok, why = explain_first_diff(g, o, q, ctx)
    assert ok, (q, why)
    valid_tree(g, o, q, ctx, check_phi=why.startswith("order"))
    return "near", why
