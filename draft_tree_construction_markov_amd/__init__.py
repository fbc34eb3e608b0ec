"""libpctree: draft-tree construction and checking on MI355X (gfx950).

A thin ctypes binding over the C-ABI declared in include/pctree.h.  It only
marshals arguments: torch provides device memory and the current stream;
every step of the computation runs in the library's HIP kernels.  If the
built library is missing the import of any entry point fails loudly: there
is no CPU fallback.

Build it with ``python -m draft_tree_construction_markov_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpctree.so")

PCT_F32, PCT_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
           3: "workspace too small", 4: "HIP error"}


class PCTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpctree: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class TreeShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("B", C.c_int32), ("V", C.c_int32),
                ("r", C.c_int32), ("k", C.c_int32), ("beam_w", C.c_int32),
                ("N", C.c_int32), ("uw_dtype", C.c_int32)]


class CostModel(C.Structure):
    _fields_ = [("C_d", C.c_double), ("c0", C.c_double), ("c1", C.c_double),
                ("c2", C.c_double), ("c_ell", C.c_double)]


_lib = None


def lib():
    """Load libpctree.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m draft_tree_construction_markov_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    L.pct_markov_logits.argtypes = [P, i64, i32, P, P, i32, i32, i32, P, P,
                                    i32, i32, P, P, P, P, P, sz, P]
    L.pct_markov_logits_workspace.argtypes = [i32, i32, i32]
    L.pct_markov_logits_workspace.restype = sz
    L.pct_build_tree.argtypes = [C.POINTER(TreeShape), P, P, P, P, P, P, P, P,
                                 P, P, P, sz, P]
    L.pct_build_tree_workspace.argtypes = [C.POINTER(TreeShape)]
    L.pct_build_tree_workspace.restype = sz
    L.pct_tree_mask.argtypes = [i32, i32, P, P, P, P]
    L.pct_verify_accept.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                    P]
    if hasattr(L, "pct_build_tree_adaptive"):
        L.pct_build_tree_adaptive.argtypes = [
            i32, i32, i32, i32, P, P, C.POINTER(CostModel), P, P, P, P, P, P,
            P, P, P, sz, P]
        L.pct_build_tree_adaptive_workspace.argtypes = [i32, i32, i32, i32]
        L.pct_build_tree_adaptive_workspace.restype = sz
    L.pct_build_tree_adaptive_pc.argtypes = [
        C.POINTER(TreeShape), P, P, P, P, P, C.POINTER(CostModel), P, P, P, P,
        P, P, P, P, P, sz, P]
    L.pct_build_tree_adaptive_pc_workspace.argtypes = [C.POINTER(TreeShape)]
    L.pct_build_tree_adaptive_pc_workspace.restype = sz
    L.pct_throughput_curve.argtypes = [i32, i32, P, P, P,
                                       C.POINTER(CostModel), P, P]
    L.pct_verify_sample.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P,
                                    C.c_double, C.c_uint64, P, P, P, P, P,
                                    sz, P]
    L.pct_verify_sample_workspace.argtypes = [i32, i32, i32]
    L.pct_verify_sample_workspace.restype = sz
    L.pct_profile_enable.argtypes = [i32]
    L.pct_profile_reset.argtypes = []
    L.pct_profile_read.argtypes = [i32, i64, C.POINTER(C.c_double),
                                   C.POINTER(C.c_int64)]
    L.pct_last_error.restype = C.c_char_p
    L.pct_status_string.restype = C.c_char_p
    _lib = L
    return L


def exported_symbols():
    """Names of the C-ABI entry points the header declares."""
    return ["pct_markov_logits", "pct_markov_logits_workspace",
            "pct_build_tree", "pct_build_tree_workspace",
            "pct_build_tree_adaptive", "pct_build_tree_adaptive_workspace",
            "pct_build_tree_adaptive_pc",
            "pct_build_tree_adaptive_pc_workspace", "pct_throughput_curve",
            "pct_build_tree_noalloc", "pct_verify_sample",
            "pct_verify_sample_workspace",
            "pct_tree_mask", "pct_verify_accept", "pct_profile_enable",
            "pct_profile_reset", "pct_profile_read", "pct_status_string",
            "pct_last_error"]


PROF_MARKOV, PROF_EXPAND, PROF_TOPN, PROF_MASK, PROF_ACCEPT, PROF_ROWTOP, \
    PROF_INIT, PROF_ROWSTATS, PROF_BESTFIRST, PROF_FINALIZE, PROF_STOP, \
    PROF_SAMPLE = range(12)


def profile_enable(on: bool = True):
    _check(lib().pct_profile_enable(1 if on else 0))


def profile_reset():
    _check(lib().pct_profile_reset())


def profile_read(kind: int, units: int = -1):
    """(total milliseconds, launches) recorded for one kernel kind."""
    ms = C.c_double()
    n = C.c_int64()
    _check(lib().pct_profile_read(kind, units, C.byref(ms), C.byref(n)))
    return ms.value, n.value


def _check(rc: int):
    if rc != 0:
        raise PCTError(rc, lib().pct_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("libpctree needs device tensors")
    return t.device


def _factors(U, W):
    if U is None and W is None:
        return None, None, PCT_F32, 0
    if U is None or W is None:
        raise ValueError("U and W must both be given or both None")
    if U.dtype != W.dtype or U.shape != W.shape or U.dim() != 2:
        raise ValueError("U and W must be [V][r] tensors of the same dtype")
    if U.dtype == torch.bfloat16:
        dt = PCT_BF16
    elif U.dtype == torch.float32:
        dt = PCT_F32
    else:
        raise ValueError("U/W must be bfloat16 or float32")
    return U.contiguous(), W.contiguous(), dt, int(U.shape[1])


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# pct_markov_logits

def markov_logits(L, U, W, parent_tok, parent_Lrow, k: int,
                  want_z: bool = False, V: int | None = None):
    """Per-parent lse and top-k of z = L[row] + U[tok] . W[v].
    L: [rows][V] float32 or None; U, W: [V][r] or None.
    Returns (lse [P], topk_tok [P][k], topk_logp [P][k], z [P][V] or None)."""
    dev = _dev(parent_tok)
    U, W, dt, r = _factors(U, W)
    if L is not None:
        L = L.contiguous()
        V = int(L.shape[-1])
        stride = V
        rows = int(L.numel() // V)
    else:
        V = int(U.shape[0])
        stride = 0
        rows = 0
    P = int(parent_tok.numel())
    lse = torch.empty(P, dtype=torch.float32, device=dev)
    tt = torch.empty(P, k, dtype=torch.int32, device=dev)
    tl = torch.empty(P, k, dtype=torch.float32, device=dev)
    z = torch.empty(P, V, dtype=torch.float32, device=dev) if want_z else None
    nbytes = lib().pct_markov_logits_workspace(P, V, k)
    ws = _workspace(nbytes, dev)
    pt = parent_tok.to(torch.int32).contiguous()
    pr = None if parent_Lrow is None else parent_Lrow.to(torch.int32).contiguous()
    _check(lib().pct_markov_logits(
        _ptr(L), stride, rows, _ptr(U), _ptr(W), dt, V, r, _ptr(pt), _ptr(pr), P, k,
        _ptr(lse), _ptr(tt), _ptr(tl), _ptr(z), _ptr(ws), ws.numel(),
        _stream(dev)))
    return lse, tt, tl, z


# ---------------------------------------------------------------------------
# pct_build_tree

@dataclass
class TreeOutputs:
    tok: torch.Tensor
    parent: torch.Tensor
    depth: torch.Tensor
    score: torch.Tensor
    n_nodes: torch.Tensor
    mask: torch.Tensor | None

    def numpy(self):
        out = {k: getattr(self, k).cpu().numpy()
               for k in ("tok", "parent", "depth", "score", "n_nodes")}
        if self.mask is not None:
            out["mask"] = self.mask.cpu().numpy().view("uint64")
        return out


class TreeBuilder:
    """A parent-conditioned build of fixed shape with its workspace and
    outputs allocated once; run() only enqueues kernels."""

    def __init__(self, batch: int, B: int, V: int, k: int, beam_w: int,
                 N: int, r: int = 0, bf16: bool = True, mask: bool = False,
                 device="cuda"):
        self.shape = TreeShape(batch, B, V, r, k, beam_w, N,
                               PCT_BF16 if bf16 else PCT_F32)
        self.device = torch.device(device)
        nbytes = lib().pct_build_tree_workspace(C.byref(self.shape))
        if nbytes == 0:
            raise PCTError(1, lib().pct_last_error().decode())
        self.ws = _workspace(nbytes, self.device)
        dev = self.device
        words = (N + 63) // 64
        self.out = TreeOutputs(
            tok=torch.empty(batch, N, dtype=torch.int32, device=dev),
            parent=torch.empty(batch, N, dtype=torch.int32, device=dev),
            depth=torch.empty(batch, N, dtype=torch.int32, device=dev),
            score=torch.empty(batch, N, dtype=torch.float32, device=dev),
            n_nodes=torch.empty(batch, dtype=torch.int32, device=dev),
            mask=(torch.empty(batch, N, words, dtype=torch.int64, device=dev)
                  if mask else None))

    def run(self, L, U, W, anchor) -> TreeOutputs:
        o = self.out
        _check(lib().pct_build_tree(
            C.byref(self.shape), _ptr(L), _ptr(U), _ptr(W), _ptr(anchor),
            _ptr(o.tok), _ptr(o.parent), _ptr(o.depth), _ptr(o.score),
            _ptr(o.n_nodes), _ptr(o.mask), _ptr(self.ws), self.ws.numel(),
            _stream(self.device)))
        return o


def build_tree(L, U, W, anchor, k: int, beam_w: int, N: int,
               mask: bool = False) -> TreeOutputs:
    """PCTree on L [batch][B][V] float32 with factors U, W [V][r] (bf16 or
    fp32) or None; anchor [batch] int32."""
    dev = _dev(L)
    batch, B, V = (int(x) for x in L.shape)
    U, W, dt, r = _factors(U, W)
    tb = TreeBuilder(batch, B, V, k, beam_w, N, r=r, bf16=(dt == PCT_BF16),
                     mask=mask, device=dev)
    return tb.run(L.contiguous(), U, W, anchor.to(torch.int32).contiguous())


# ---------------------------------------------------------------------------
# pct_build_tree_adaptive

class AdaptiveBuilder:
    """CaDDTree best-first build with the throughput stop, fixed shape."""

    def __init__(self, batch: int, B: int, V: int, n_max: int,
                 cost: dict | None, mask: bool = False, device="cuda"):
        self.batch, self.B, self.V, self.n_max = batch, B, V, n_max
        self.cost = None if cost is None else CostModel(
            cost["C_d"], cost["c0"], cost["c1"], cost["c2"], cost["c_ell"])
        self.device = torch.device(device)
        nbytes = lib().pct_build_tree_adaptive_workspace(batch, B, V, n_max)
        if nbytes == 0:
            raise PCTError(1, lib().pct_last_error().decode())
        self.ws = _workspace(nbytes, self.device)
        dev = self.device
        words = (n_max + 63) // 64
        self.tok = torch.empty(batch, n_max, dtype=torch.int32, device=dev)
        self.parent = torch.empty_like(self.tok)
        self.depth = torch.empty_like(self.tok)
        self.score = torch.empty(batch, n_max, dtype=torch.float32, device=dev)
        self.n_star = torch.empty(batch, dtype=torch.int32, device=dev)
        self.phi = torch.empty(batch, dtype=torch.float64, device=dev)
        self.throughput = torch.empty(batch, dtype=torch.float64, device=dev)
        self.mask = (torch.empty(batch, n_max, words, dtype=torch.int64,
                                 device=dev) if mask else None)

    def run(self, L, ctx_len):
        _check(lib().pct_build_tree_adaptive(
            self.batch, self.B, self.V, self.n_max, _ptr(L), _ptr(ctx_len),
            None if self.cost is None else C.byref(self.cost),
            _ptr(self.tok), _ptr(self.parent), _ptr(self.depth),
            _ptr(self.score), _ptr(self.n_star), _ptr(self.phi),
            _ptr(self.throughput), _ptr(self.mask), _ptr(self.ws),
            self.ws.numel(), _stream(self.device)))
        return self

    def numpy(self):
        out = {k: getattr(self, k).cpu().numpy()
               for k in ("tok", "parent", "depth", "score", "n_star", "phi",
                         "throughput")}
        if self.mask is not None:
            out["mask"] = self.mask.cpu().numpy().view("uint64")
        return out


def build_tree_adaptive(L, ctx_len, n_max: int, cost: dict | None,
                        mask: bool = False) -> AdaptiveBuilder:
    batch, B, V = (int(x) for x in L.shape)
    ab = AdaptiveBuilder(batch, B, V, n_max, cost, mask=mask,
                         device=_dev(L))
    return ab.run(L.contiguous(), ctx_len.to(torch.int32).contiguous())


# ---------------------------------------------------------------------------
# pct_build_tree_adaptive_pc / pct_throughput_curve

def _cost_struct(cost):
    return None if cost is None else CostModel(
        cost["C_d"], cost["c0"], cost["c1"], cost["c2"], cost["c_ell"])


class AdaptivePCBuilder:
    """Throughput stop on the parent-conditioned tree, fixed shape (N is
    the largest tree considered)."""

    def __init__(self, batch: int, B: int, V: int, k: int, beam_w: int,
                 n_max: int, cost: dict | None, r: int = 0,
                 bf16: bool = True, mask: bool = False, device="cuda"):
        self.shape = TreeShape(batch, B, V, r, k, beam_w, n_max,
                               PCT_BF16 if bf16 else PCT_F32)
        self.cost = _cost_struct(cost)
        self.device = torch.device(device)
        nbytes = lib().pct_build_tree_adaptive_pc_workspace(
            C.byref(self.shape))
        if nbytes == 0:
            raise PCTError(1, lib().pct_last_error().decode())
        self.ws = _workspace(nbytes, self.device)
        dev = self.device
        words = (n_max + 63) // 64
        self.tok = torch.empty(batch, n_max, dtype=torch.int32, device=dev)
        self.parent = torch.empty_like(self.tok)
        self.depth = torch.empty_like(self.tok)
        self.score = torch.empty(batch, n_max, dtype=torch.float32, device=dev)
        self.n_star = torch.empty(batch, dtype=torch.int32, device=dev)
        self.phi = torch.empty(batch, dtype=torch.float64, device=dev)
        self.throughput = torch.empty(batch, dtype=torch.float64, device=dev)
        self.mask = (torch.empty(batch, n_max, words, dtype=torch.int64,
                                 device=dev) if mask else None)

    def run(self, L, U, W, anchor, ctx_len):
        _check(lib().pct_build_tree_adaptive_pc(
            C.byref(self.shape), _ptr(L), _ptr(U), _ptr(W), _ptr(anchor),
            _ptr(ctx_len), None if self.cost is None else C.byref(self.cost),
            _ptr(self.tok), _ptr(self.parent), _ptr(self.depth),
            _ptr(self.score), _ptr(self.n_star), _ptr(self.phi),
            _ptr(self.throughput), _ptr(self.mask), _ptr(self.ws),
            self.ws.numel(), _stream(self.device)))
        return self

    def numpy(self):
        out = {k: getattr(self, k).cpu().numpy()
               for k in ("tok", "parent", "depth", "score", "n_star", "phi",
                         "throughput")}
        if self.mask is not None:
            out["mask"] = self.mask.cpu().numpy().view("uint64")
        return out


def build_tree_adaptive_pc(L, U, W, anchor, ctx_len, k: int, beam_w: int,
                           n_max: int, cost: dict | None,
                           mask: bool = False) -> AdaptivePCBuilder:
    dev = _dev(L)
    batch, B, V = (int(x) for x in L.shape)
    U, W, dt, r = _factors(U, W)
    ab = AdaptivePCBuilder(batch, B, V, k, beam_w, n_max, cost, r=r,
                           bf16=(dt == PCT_BF16), mask=mask, device=dev)
    return ab.run(L.contiguous(), U, W, anchor.to(torch.int32).contiguous(),
                  ctx_len.to(torch.int32).contiguous())


def throughput_curve(score, n_nodes, ctx_len, cost: dict | None):
    """f(n) = (1 + Phi_n) / D(n) for n = 0..N of best-first-ordered scores
    [batch][N]; returns [batch][N+1] float64."""
    dev = _dev(score)
    batch, N = (int(x) for x in score.shape)
    f = torch.empty(batch, N + 1, dtype=torch.float64, device=dev)
    cm = _cost_struct(cost)
    _check(lib().pct_throughput_curve(
        batch, N, _ptr(score.contiguous()), _ptr(n_nodes.contiguous()),
        _ptr(None if ctx_len is None else ctx_len.contiguous()),
        None if cm is None else C.byref(cm), _ptr(f), _stream(dev)))
    return f


# ---------------------------------------------------------------------------
# pct_tree_mask / pct_verify_accept

def tree_mask(parent, n_nodes, out=None) -> torch.Tensor:
    """parent [batch][N] int32, n_nodes [batch] -> mask [batch][N][words]
    (int64 storage of the uint64 words), into `out` when given."""
    dev = _dev(parent)
    batch, N = (int(x) for x in parent.shape)
    words = (N + 63) // 64
    mask = out if out is not None else torch.empty(
        batch, N, words, dtype=torch.int64, device=dev)
    if tuple(mask.shape) != (batch, N, words) or mask.dtype != torch.int64:
        raise ValueError("mask must be int64 [batch][N][ceil(N/64)]")
    _check(lib().pct_tree_mask(batch, N, _ptr(parent.contiguous()),
                               _ptr(n_nodes.contiguous()), _ptr(mask),
                               _stream(dev)))
    return mask


def verify_accept(tok, parent, depth, n_nodes, target, B: int, out=None,
                  mask=None):
    """Greedy acceptance walk; with the tree's packed ancestry mask the
    acceptance test uses it.  Returns (tau [batch], accept_node [batch][B],
    accept_tok [batch][B+1])."""
    dev = _dev(tok)
    batch, N = (int(x) for x in tok.shape)
    if out is None:
        out = (torch.empty(batch, dtype=torch.int32, device=dev),
               torch.empty(batch, B, dtype=torch.int32, device=dev),
               torch.empty(batch, B + 1, dtype=torch.int32, device=dev))
    if mask is not None and tuple(mask.shape) != (batch, N, (N + 63) // 64):
        raise ValueError("mask must be [batch][N][ceil(N/64)]")
    tau, an, at = out
    _check(lib().pct_verify_accept(
        batch, N, B, _ptr(tok), _ptr(parent), _ptr(depth), _ptr(n_nodes),
        _ptr(mask), _ptr(target), _ptr(tau), _ptr(an), _ptr(at),
        _stream(dev)))
    return tau, an, at


def verify_sample(tok, parent, depth, n_nodes, target_logits, B: int,
                  temperature: float, seed: int, mask=None, out=None,
                  workspace=None):
    """Verification with temperature sampling: target_logits
    [batch][N+1][V] float32.  Returns (sampled [batch][N+1], tau [batch],
    accept_node [batch][B], accept_tok [batch][B+1]).  workspace: an
    optional uint8 device tensor reused across calls."""
    dev = _dev(tok)
    batch, N = (int(x) for x in tok.shape)
    V = int(target_logits.shape[-1])
    if tuple(target_logits.shape) != (batch, N + 1, V):
        raise ValueError("target_logits must be [batch][N+1][V]")
    if out is None:
        out = (torch.empty(batch, N + 1, dtype=torch.int32, device=dev),
               torch.empty(batch, dtype=torch.int32, device=dev),
               torch.empty(batch, B, dtype=torch.int32, device=dev),
               torch.empty(batch, B + 1, dtype=torch.int32, device=dev))
    sm, tau, an, at = out
    nb = int(lib().pct_verify_sample_workspace(batch, N, V))
    if workspace is None or workspace.numel() < nb:
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib().pct_verify_sample(
        batch, N, B, V, _ptr(tok), _ptr(parent), _ptr(depth), _ptr(n_nodes),
        _ptr(mask), _ptr(target_logits.contiguous()), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(sm), _ptr(tau), _ptr(an),
        _ptr(at), _ptr(workspace), workspace.numel(), _stream(dev)))
    return sm, tau, an, at


def bf16_tensor(bits, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> a bfloat16 device tensor."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)
