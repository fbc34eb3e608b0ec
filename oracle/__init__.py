"""ctypes front-end of the CPU oracle (pct_oracle.c).

TEST INFRASTRUCTURE ONLY: the oracle is a plain, slow, single-threaded C
implementation used to check the GPU library.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the
product path never does.

The library is built with gcc (-O2 -ffp-contract=off, no fast-math) by
build(); load() builds it only when no built copy exists.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pct_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1

_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", LIB + ".tmp",
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class TreeShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("B", C.c_int32), ("V", C.c_int32),
                ("r", C.c_int32), ("k", C.c_int32), ("beam_w", C.c_int32),
                ("N", C.c_int32), ("uw_dtype", C.c_int32)]


class CostModel(C.Structure):
    _fields_ = [("C_d", C.c_double), ("c0", C.c_double), ("c1", C.c_double),
                ("c2", C.c_double), ("c_ell", C.c_double)]


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = C.CDLL(LIB)
    P = C.c_void_p
    i32 = C.c_int32
    lib.ref_markov_row.argtypes = [P, P, i32, i32, i32, i32, P]
    lib.ref_row_stats.argtypes = [P, P, i32, i32, P, P, P, P]
    lib.ref_pool_size.argtypes = [C.POINTER(TreeShape)]
    lib.ref_pool_size.restype = C.c_int64
    lib.ref_build_tree.argtypes = [C.POINTER(TreeShape), P, P, P, P, P, P, P,
                                   P, P, P, P, P, P, P, P]
    lib.ref_greedy_chain.argtypes = [i32, i32, i32, P, P, P, i32, i32, P]
    lib.ref_bestfirst.argtypes = [i32, i32, i32, P, P, P, i32, i32, i32, P, P,
                                  P, P, P, P]
    lib.ref_adaptive.argtypes = [i32, i32, i32, i32, P, P, P, i32, i32, i32,
                                 C.POINTER(CostModel), P, P, P, P, P, P, P, P,
                                 P]
    lib.ref_stop.argtypes = [i32, P, i32, C.POINTER(CostModel), P, P, P, P]
    lib.ref_throughput_curve.argtypes = [i32, P, i32, C.POINTER(CostModel),
                                         P]
    lib.ref_uniform.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
    lib.ref_uniform.restype = C.c_double
    lib.ref_sample_targets.argtypes = [i32, i32, P, C.c_double, C.c_uint64,
                                       C.c_uint64, P, P]
    lib.ref_mask.argtypes = [i32, i32, P, P]
    lib.ref_mask.restype = None
    lib.ref_accept.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _factors(U, W):
    if U is None:
        return None, None, F32
    if U.dtype == np.uint16:
        return (np.ascontiguousarray(U), np.ascontiguousarray(W, np.uint16),
                BF16)
    return _f32(U), _f32(W), F32


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def markov_row(U, W, tok: int) -> np.ndarray:
    U, W, dt = _factors(U, W)
    V, r = U.shape
    out = np.empty(V, dtype=np.float32)
    _check(load().ref_markov_row(_p(U), _p(W), dt, V, r, tok, _p(out)),
           "markov_row")
    return out


def row_stats(Lrow, Mrow, k: int):
    """Returns (lse, topk_tok, topk_z, min_gap)."""
    Lrow = _f32(Lrow)
    Mrow = None if Mrow is None else _f32(Mrow)
    V = Lrow.shape[0]
    lse = np.empty(1, np.float32)
    tt = np.empty(k, np.int32)
    tz = np.empty(k, np.float32)
    g = np.empty(1, np.float64)
    _check(load().ref_row_stats(_p(Lrow), _p(Mrow), V, k, _p(lse), _p(tt),
                                _p(tz), _p(g)), "row_stats")
    return float(lse[0]), tt, tz, float(g[0])


def shape(batch, B, V, r, k, beam_w, N, bf16=False) -> TreeShape:
    return TreeShape(batch, B, V, r, k, beam_w, N, BF16 if bf16 else F32)


def pool_size(batch, B, V, r, k, beam_w, N) -> int:
    sh = shape(batch, B, V, r, k, beam_w, N)
    return int(load().ref_pool_size(C.byref(sh)))


def build_tree(L, U, W, anchor, k: int, beam_w: int, N: int,
               diagnostics: bool = False):
    """PCTree on [batch][B][V] logits.  Returns a dict with tok, parent,
    depth, score [batch][N], n_nodes [batch], min_gap [batch], depth_gap
    [batch][B+1] (beam-boundary gap per depth, then the top-N boundary gap)
    and, with diagnostics, pool_tok/pool_ppid/pool_score [batch][pool] and
    beam_pid [batch][B][beam_w]."""
    L = _f32(L)
    batch, B, V = L.shape
    U, W, dt = _factors(U, W)
    r = 0 if U is None else U.shape[1]
    sh = TreeShape(batch, B, V, r, k, beam_w, N, dt)
    lib = load()
    pool = int(lib.ref_pool_size(C.byref(sh)))
    out = dict(tok=np.empty((batch, N), np.int32),
               parent=np.empty((batch, N), np.int32),
               depth=np.empty((batch, N), np.int32),
               score=np.empty((batch, N), np.float32),
               n_nodes=np.empty(batch, np.int32),
               min_gap=np.empty(batch, np.float64),
               depth_gap=np.empty((batch, B + 1), np.float64))
    if diagnostics:
        out["pool_tok"] = np.empty((batch, pool), np.int32)
        out["pool_ppid"] = np.empty((batch, pool), np.int32)
        out["pool_score"] = np.empty((batch, pool), np.float32)
        out["beam_pid"] = np.empty((batch, B, beam_w), np.int32)
    A = _i32(anchor)
    rc = lib.ref_build_tree(
        C.byref(sh), _p(L), _p(U), _p(W), _p(A), _p(out["tok"]),
        _p(out["parent"]), _p(out["depth"]), _p(out["score"]),
        _p(out["n_nodes"]), _p(out["min_gap"]), _p(out.get("pool_tok")),
        _p(out.get("pool_ppid")), _p(out.get("pool_score")),
        _p(out.get("beam_pid")), _p(out["depth_gap"]))
    _check(rc, "build_tree")
    return out


def greedy_chain(L, U, W, anchor: int) -> np.ndarray:
    L = _f32(L)
    B, V = L.shape
    U, W, dt = _factors(U, W)
    r = 0 if U is None else U.shape[1]
    out = np.empty(B, np.int32)
    _check(load().ref_greedy_chain(B, V, r, _p(L), _p(U), _p(W), dt, anchor,
                                   _p(out)), "greedy_chain")
    return out


def bestfirst(L, U, W, anchor: int, n_max: int):
    """One request's best-first tree ([B][V] logits).  Returns dict with
    tok, parent, depth, score [n_max], n, min_gap."""
    L = _f32(L)
    B, V = L.shape
    U, W, dt = _factors(U, W)
    r = 0 if U is None else U.shape[1]
    out = dict(tok=np.empty(n_max, np.int32), parent=np.empty(n_max, np.int32),
               depth=np.empty(n_max, np.int32),
               score=np.empty(n_max, np.float32))
    n = np.empty(1, np.int32)
    g = np.empty(1, np.float64)
    rc = load().ref_bestfirst(B, V, r, _p(L), _p(U), _p(W), dt, anchor, n_max,
                              _p(out["tok"]), _p(out["parent"]),
                              _p(out["depth"]), _p(out["score"]), _p(n), _p(g))
    _check(rc, "bestfirst")
    out["n"] = int(n[0])
    out["min_gap"] = float(g[0])
    return out


def _cost(cost):
    return None if cost is None else CostModel(cost["C_d"], cost["c0"],
                                               cost["c1"], cost["c2"],
                                               cost["c_ell"])


def adaptive(L, n_max: int, ctx_len: int, cost: dict | None, U=None, W=None,
             anchor: int = 0):
    """One request's adaptive best-first tree ([B][V] logits): marginal rows
    without U/W, parent-conditioned rows from `anchor` with them.
    cost: dict(C_d, c0, c1, c2, c_ell) or None for a fixed budget n_max."""
    L = _f32(L)
    B, V = L.shape
    U, W, dt = _factors(U, W)
    r = 0 if U is None else U.shape[1]
    out = dict(tok=np.empty(n_max, np.int32), parent=np.empty(n_max, np.int32),
               depth=np.empty(n_max, np.int32),
               score=np.empty(n_max, np.float32))
    ns = np.empty(1, np.int32)
    phi = np.empty(1, np.float64)
    thr = np.empty(1, np.float64)
    g = np.empty(1, np.float64)
    gm = np.empty(1, np.float64)
    cm = _cost(cost)
    rc = load().ref_adaptive(B, V, r, n_max, _p(L), _p(U), _p(W), dt,
                             int(anchor), int(ctx_len),
                             None if cm is None else C.byref(cm),
                             _p(out["tok"]), _p(out["parent"]),
                             _p(out["depth"]), _p(out["score"]), _p(ns),
                             _p(phi), _p(thr), _p(g), _p(gm))
    _check(rc, "adaptive")
    out.update(n_star=int(ns[0]), phi=float(phi[0]), throughput=float(thr[0]),
               min_gap=float(g[0]), gain_margin=float(gm[0]))
    return out


def stop(score, n_avail: int, ctx_len: int, cost: dict | None):
    """Throughput stop over best-first-ordered scores.  Returns dict with
    n_star, phi, throughput, gain_margin."""
    sc = _f32(score)
    ns = np.empty(1, np.int32)
    phi = np.empty(1, np.float64)
    thr = np.empty(1, np.float64)
    gm = np.empty(1, np.float64)
    cm = _cost(cost)
    _check(load().ref_stop(int(n_avail), _p(sc), int(ctx_len),
                           None if cm is None else C.byref(cm), _p(ns),
                           _p(phi), _p(thr), _p(gm)), "stop")
    return dict(n_star=int(ns[0]), phi=float(phi[0]),
                throughput=float(thr[0]), gain_margin=float(gm[0]))


def throughput_curve(score, n_avail: int, ctx_len: int, cost: dict | None):
    """f(n) = (1 + Phi_n) / D(n) for n = 0..n_avail."""
    sc = _f32(score)
    f = np.empty(int(n_avail) + 1, np.float64)
    cm = _cost(cost)
    _check(load().ref_throughput_curve(int(n_avail), _p(sc), int(ctx_len),
                                       None if cm is None else C.byref(cm),
                                       _p(f)), "throughput_curve")
    return f


def mask(parent, n_nodes: int, N: int) -> np.ndarray:
    parent = _i32(parent)
    words = (N + 63) // 64
    out = np.empty((N, words), np.uint64)
    load().ref_mask(N, n_nodes, _p(parent), _p(out))
    return out


def accept(tok, parent, n_nodes: int, B: int, target):
    """Returns (tau, accept_node [B], accept_tok [B+1])."""
    tok = _i32(tok)
    parent = _i32(parent)
    target = _i32(target)
    N = tok.shape[0]
    tau = np.empty(1, np.int32)
    an = np.empty(B, np.int32)
    at = np.empty(B + 1, np.int32)
    _check(load().ref_accept(N, n_nodes, B, _p(tok), _p(parent), _p(target),
                             _p(tau), _p(an), _p(at)), "accept")
    return int(tau[0]), an, at


def uniform(seed: int, stream: int, idx: int) -> float:
    return float(load().ref_uniform(seed, stream, idx))


def sample_targets(logits, temperature: float, seed: int, stream0: int = 0):
    """Sampled target tokens of the rows of logits [n_rows][V].  Returns
    (tokens [n_rows], key_gap [n_rows])."""
    z = _f32(logits)
    n, V = z.shape
    out = np.empty(n, np.int32)
    gap = np.empty(n, np.float64)
    _check(load().ref_sample_targets(n, V, _p(z), float(temperature),
                                     int(seed), int(stream0), _p(out),
                                     _p(gap)), "sample_targets")
    return out, gap

