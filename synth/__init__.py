"""Seeded synthetic inputs shaped like the pages' workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it only draws
numbers.  Every value is a pure function of (seed, tag, index) through a
counter-based generator, so any slice can be regenerated independently.

Generator (SplitMix64, Steele/Lea/Flood 2014, "Fast splittable pseudorandom
number generators"):
    h(seed, tag, i) = sm(sm(sm(seed) ^ tag) ^ i)
    u(seed, tag, i) = ((h >> 11) + 0.5) * 2**-53          in (0, 1)
    n(seed, tag, i) = sqrt(-2 ln u(2i)) * cos(2 pi u(2i+1))  (Box-Muller)

Workloads (vocabulary of the Qwen3 family, the pages' block lengths 7 and
16, budgets up to ~1k nodes); the recipe is restated in the design notes:
  tiny      batch 1,   V=1000,   B=4,  k=4, beam 4,  N=16,  r=16,  fp32 U/W
  b7        batch 1,   V=151936, B=7,  k=8, beam 8,  N=64,  r=256, bf16 U/W
  b16       batch 32,  V=151936, B=16, k=8, beam 16, N=256, r=256, bf16 U/W
  adaptive  batch 64,  V=151936, B=16, n_max=1024, marginals only
  round     batch 128, V=151936, B=16, k=8, beam 16, N=512, r=256, bf16 U/W
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GOLD = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)

TAG_NOISE, TAG_PERM, TAG_TEMP, TAG_U, TAG_W, TAG_ANCHOR, TAG_TARGET, \
    TAG_REGIME, TAG_CTX = 1, 2, 3, 4, 5, 6, 7, 8, 9

ZIPF_S = 1.1


def _sm(x):
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GOLD
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
    return z ^ (z >> np.uint64(31))


def _sm_int(x: int) -> int:
    return int(_sm(np.array([x & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0])


def stream_key(seed: int, tag: int) -> int:
    return _sm_int(_sm_int(seed) ^ tag)


def hash_at(seed: int, tag: int, idx) -> np.ndarray:
    key = np.uint64(stream_key(seed, tag))
    return _sm(np.asarray(idx, dtype=np.uint64) ^ key)


def uniform(seed: int, tag: int, idx) -> np.ndarray:
    h = hash_at(seed, tag, idx)
    return ((h >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal_chunk(seed: int, tag: int, idx: np.ndarray) -> np.ndarray:
    u1 = uniform(seed, tag, idx * np.uint64(2))
    u2 = uniform(seed, tag, idx * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


_CHUNK = 1 << 20


def normal(seed: int, tag: int, idx) -> np.ndarray:
    """Standard normals at the given counters (float64).  Large requests are
    cut into chunks and drawn on a few threads; the values do not depend on
    the chunking."""
    idx = np.asarray(idx, dtype=np.uint64)
    flat = idx.reshape(-1)
    if flat.size <= _CHUNK:
        return _normal_chunk(seed, tag, flat).reshape(idx.shape)
    out = np.empty(flat.size, dtype=np.float64)
    starts = range(0, flat.size, _CHUNK)

    def work(s):
        out[s:s + _CHUNK] = _normal_chunk(seed, tag, flat[s:s + _CHUNK])

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(work, starts))
    return out.reshape(idx.shape)


def _threads() -> int:
    return max(1, min(8, os.cpu_count() or 1))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rnd) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# drafter logits

def zipf_bias(seed: int, req: int, V: int) -> np.ndarray:
    """Bias -s*ln(rank+1) over one seeded token permutation per request
    (softmax of the bias alone is exactly Zipf(s))."""
    keys = uniform(seed, TAG_PERM, np.arange(V, dtype=np.uint64)
                   + np.uint64(req) * np.uint64(V))
    perm = np.argsort(keys, kind="stable")
    b = np.empty(V, dtype=np.float64)
    b[perm] = -ZIPF_S * np.log(np.arange(1, V + 1, dtype=np.float64))
    return b


def base_rows(seed: int, req: int, B: int, V: int, var: float) -> np.ndarray:
    """[B][V] float64: N(0, var) noise + the request's Zipf bias."""
    idx = (np.arange(B * V, dtype=np.uint64)
           + np.uint64(req) * np.uint64(B) * np.uint64(V))
    noise = normal(seed, TAG_NOISE, idx).reshape(B, V) * math.sqrt(var)
    return noise + zipf_bias(seed, req, V)[None, :]


def request_temperature(seed: int, req: int, lo: float, hi: float) -> float:
    return float(lo + (hi - lo) * uniform(seed, TAG_TEMP, np.array([req]))[0])


def drafter_logits(seed: int, batch: int, B: int, V: int, var: float,
                   temp_range=None, req0: int = 0) -> np.ndarray:
    """[batch][B][V] fp32 block logits.  With temp_range=(lo, hi) each
    request's rows are divided by its own temperature T ~ U[lo, hi]."""
    out = np.empty((batch, B, V), dtype=np.float32)
    for q in range(batch):
        rq = req0 + q
        rows = base_rows(seed, rq, B, V, var)
        if temp_range is not None:
            rows = rows / request_temperature(seed, rq, *temp_range)
        out[q] = rows.astype(np.float32)
    return out


def markov_factors(seed: int, V: int, r: int, bf16: bool):
    """U, W as [V][r] arrays ~ N(0, 1/r).  bf16=True returns uint16 bits."""
    sd = 1.0 / math.sqrt(r)
    idx = np.arange(V * r, dtype=np.uint64)
    U = (normal(seed, TAG_U, idx) * sd).astype(np.float32).reshape(V, r)
    W = (normal(seed, TAG_W, idx) * sd).astype(np.float32).reshape(V, r)
    if bf16:
        return bf16_bits(U), bf16_bits(W)
    return U, W


def anchors(seed: int, batch: int, V: int, req0: int = 0) -> np.ndarray:
    u = uniform(seed, TAG_ANCHOR, np.arange(req0, req0 + batch,
                                            dtype=np.uint64))
    return np.minimum((u * V).astype(np.int64), V - 1).astype(np.int32)


# --------------------------------------------------------------------------
# adaptive (marginal) rounds

def _entropy_rows(z: np.ndarray, beta: np.ndarray):
    a = z * beta[:, None]
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    s = e.sum(axis=1)
    p = e / s[:, None]
    mean_a = (p * a).sum(axis=1)
    H = np.log(s) - mean_a
    var = (p * a * a).sum(axis=1) - mean_a * mean_a
    return H, var


def flatten_to_entropy(rows: np.ndarray, target: float) -> np.ndarray:
    """Per row, the temperature T with H(softmax(rows/T)) = target nats
    (safeguarded Newton on log beta, beta = 1/T, with a bisection bracket)."""
    n = rows.shape[0]
    lo = np.full(n, -12.0)  # log beta bracket
    hi = np.full(n, 6.0)
    lb = np.zeros(n)
    for _ in range(60):
        beta = np.exp(lb)
        H, var_a = _entropy_rows(rows, beta)
        err = H - target
        # H decreases as beta grows
        hi = np.where(err < 0, lb, hi)
        lo = np.where(err >= 0, lb, lo)
        if np.all(np.abs(err) < 1e-10):
            break
        # dH/dlog(beta) = -Var_p(beta*z)
        step = np.where(var_a > 1e-300, err / np.maximum(var_a, 1e-300), 0.0)
        cand = lb + step
        bad = (cand <= lo) | (cand >= hi) | (var_a <= 1e-300)
        lb = np.where(bad, 0.5 * (lo + hi), cand)
    return 1.0 / np.exp(lb)


def peak_rows(rows: np.ndarray, p_top: float) -> np.ndarray:
    """Raise each row's argmax so that its softmax probability is p_top."""
    out = rows.copy()
    a = rows.argmax(axis=1)
    for i in range(rows.shape[0]):
        rest = np.delete(rows[i], a[i])
        m = rest.max()
        lse_rest = m + math.log(np.exp(rest - m).sum())
        out[i, a[i]] = math.log(p_top) - math.log(1.0 - p_top) + lse_rest
    return out


def adaptive_round(seed: int, batch: int, B: int, V: int, var: float = 3.0,
                   p_top: float = 0.95, entropy: float = 6.0,
                   ctx_lo: int = 512, ctx_hi: int = 32768, req0: int = 0):
    """Marginal block logits with per-request drafter confidence.
    Returns (L [batch][B][V] fp32, peaked [batch] bool, ctx_len [batch])."""
    L = np.empty((batch, B, V), dtype=np.float32)
    peaked = np.zeros(batch, dtype=bool)
    reqs = np.arange(req0, req0 + batch, dtype=np.uint64)
    regime = uniform(seed, TAG_REGIME, reqs)
    ctxu = uniform(seed, TAG_CTX, reqs)
    ctx = np.rint(np.exp(math.log(ctx_lo) + ctxu * (math.log(ctx_hi)
                                                     - math.log(ctx_lo))))
    for q in range(batch):
        rows = base_rows(seed, req0 + q, B, V, var)
        if regime[q] < 0.5:
            peaked[q] = True
            rows = peak_rows(rows, p_top)
        else:
            T = flatten_to_entropy(rows, entropy)
            rows = rows / T[:, None]
        L[q] = rows.astype(np.float32)
    return L, peaked, ctx.astype(np.int32)


def context_lengths(seed: int, batch: int, lo: int = 512, hi: int = 32768,
                    req0: int = 0) -> np.ndarray:
    """Context length per request, log-uniform over [lo, hi] (the same draw
    as adaptive_round's)."""
    reqs = np.arange(req0, req0 + batch, dtype=np.uint64)
    ctxu = uniform(seed, TAG_CTX, reqs)
    return np.rint(np.exp(math.log(lo) + ctxu * (math.log(hi) -
                                                 math.log(lo)))).astype(
        np.int32)


# --------------------------------------------------------------------------
# synthetic target tokens for the acceptance walk

def _path_hashes(tok, parent, n, anchor):
    """Per node, a 64-bit hash of its token path from the anchor."""
    h = np.zeros(n + 1, dtype=np.uint64)  # index 0 = root
    h[0] = _sm(np.array([anchor & 0xFFFFFFFF], dtype=np.uint64))[0]
    for i in range(n):
        p = int(parent[i])
        h[i + 1] = _sm(np.array([int(h[p + 1]) ^ (int(tok[i]) + 1)],
                                dtype=np.uint64))[0]
    return h


def targets_from_tree(seed: int, tok, parent, depth, n_nodes, anchor, V: int,
                      B: int, q_of_depth, req0: int = 0) -> np.ndarray:
    """target [batch][N+1]: index 0 is the target's token after the root,
    1+i after node i.  A node with children agrees with its first child (in
    output order) with probability q(depth); otherwise, and at leaves, the
    target picks a uniform random token.  Draws are keyed by the node's token
    path, so equal trees get equal targets."""
    tok = np.asarray(tok)
    batch, N = tok.shape
    out = np.empty((batch, N + 1), dtype=np.int32)
    key = np.uint64(stream_key(seed, TAG_TARGET))
    for q in range(batch):
        n = int(n_nodes[q])
        first_child = np.full(n + 1, -1, dtype=np.int64)
        for i in range(n - 1, -1, -1):
            first_child[int(parent[q, i]) + 1] = i
        h = _path_hashes(tok[q], parent[q], n, int(anchor[q]))
        hq = _sm(h ^ key ^ np.uint64(req0 + q))
        u_agree = ((_sm(hq ^ np.uint64(1)) >> np.uint64(11)).astype(np.float64)
                   + 0.5) * 2.0 ** -53
        u_tok = ((_sm(hq ^ np.uint64(2)) >> np.uint64(11)).astype(np.float64)
                 + 0.5) * 2.0 ** -53
        rnd = np.minimum((u_tok * V).astype(np.int64), V - 1)
        d_of = np.zeros(n + 1, dtype=np.int64)
        d_of[1:] = np.asarray(depth[q, :n])
        for u in range(n + 1):
            fc = first_child[u]
            if fc >= 0 and u_agree[u] < q_of_depth(int(d_of[u])):
                out[q, u] = tok[q, fc]
            else:
                out[q, u] = rnd[u]
        out[q, n + 1:] = -1
    return out


def round_agreement(B: int):
    """Agreement that decays linearly from 0.9 at the root to 0.6 at depth
    B-1."""
    return lambda d: 0.9 - 0.3 * d / max(B - 1, 1)


# --------------------------------------------------------------------------
# named workloads

@dataclass
class TreeWorkload:
    name: str
    seed: int
    batch: int
    B: int
    V: int
    k: int
    beam_w: int
    N: int
    r: int
    bf16: bool
    var: float
    temp_range: tuple | None
    agreement: float | None = None
    extra: dict = field(default_factory=dict)


TREE_WORKLOADS = {
    "tiny": TreeWorkload("tiny", 1001, 1, 4, 1000, 4, 4, 16, 16, False, 2.0,
                         None, agreement=0.7),
    "b7": TreeWorkload("b7", 2001, 1, 7, 151936, 8, 8, 64, 256, True, 3.0,
                       None),
    "b16": TreeWorkload("b16", 3001, 32, 16, 151936, 8, 16, 256, 256, True,
                        3.0, (0.5, 2.0)),
    "round": TreeWorkload("round", 5001, 128, 16, 151936, 8, 16, 512, 256,
                          True, 3.0, (0.5, 2.0)),
}

ADAPTIVE = dict(name="adaptive", seed=4001, batch=64, B=16, V=151936,
                n_max=1024, C_d=1.0, c0=2.0, c1=0.004, c2=2e-6, c_ell=1e-5)


def tree_inputs(w: TreeWorkload, batch: int | None = None, req0: int = 0,
                seed: int | None = None):
    """L, U, W, anchor for a tree workload (optionally a slice of requests
    req0..req0+batch-1; U and W are shared by all requests)."""
    sd = w.seed if seed is None else seed
    nb = w.batch if batch is None else batch
    L = drafter_logits(sd, nb, w.B, w.V, w.var, w.temp_range, req0=req0)
    U, W = markov_factors(sd, w.V, w.r, w.bf16)
    A = anchors(sd, nb, w.V, req0=req0)
    return L, U, W, A
