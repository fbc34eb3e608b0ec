"""GPU check of pct_build_tree_noalloc (the build with its workspace in the
library's own fixed device array) through the C ABI: two calls in a row,
the second on a smaller input, each equal to pct_build_tree with a
caller-owned workspace on the same inputs; a shape whose workspace exceeds
the array is rejected before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

import draft_tree_construction_markov_amd as pct
import synth
from gpu_util import announce, dev_f32, dev_factors, dev_i32

pytestmark = pytest.mark.gpu


def _lib():
    lib = pct.lib()
    P = C.c_void_p
    lib.pct_build_tree_noalloc.argtypes = [C.POINTER(pct.TreeShape), P, P, P,
                                           P, P, P, P, P, P, P, P]
    return lib


def _inputs(seed, batch, B, V, r):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(batch, B, V)) * 1.7).astype(np.float32)
    U, W = synth.markov_factors(seed, V, r, True)
    A = rng.integers(0, V, size=batch).astype(np.int32)
    return L, U, W, A


def _noalloc(lib, sh, dL, dU, dW, dA, N):
    batch = sh.batch
    dev = dL.device
    out = dict(tok=torch.empty(batch, N, dtype=torch.int32, device=dev),
               parent=torch.empty(batch, N, dtype=torch.int32, device=dev),
               depth=torch.empty(batch, N, dtype=torch.int32, device=dev),
               score=torch.empty(batch, N, dtype=torch.float32, device=dev),
               n_nodes=torch.empty(batch, dtype=torch.int32, device=dev),
               mask=torch.empty(batch, N, (N + 63) // 64, dtype=torch.int64,
                                device=dev))
    p = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.pct_build_tree_noalloc(
        C.byref(sh), p(dL), p(dU), p(dW), p(dA), p(out["tok"]),
        p(out["parent"]), p(out["depth"]), p(out["score"]),
        p(out["n_nodes"]), p(out["mask"]),
        C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.pct_last_error()
    return out


@pytest.mark.parametrize("calls", [[(3, 8, 5, 20000, 256, 8, 16, 128),
                                    (4, 3, 3, 3000, 64, 4, 6, 40)]])
def test_noalloc_matches_workspace_build(calls):
    lib = _lib()
    for seed, batch, B, V, r, k, beam, N in calls:
        L, U, W, A = _inputs(seed, batch, B, V, r)
        dL, dA = dev_f32(L), dev_i32(A)
        dU, dW = dev_factors(U, W)
        sh = pct.TreeShape(batch, B, V, r, k, beam, N, pct.PCT_BF16)
        announce("noalloc", dict(batch=batch, B=B, V=V, r=r, k=k, N=N))
        got = _noalloc(lib, sh, dL, dU, dW, dA, N)
        ref = pct.build_tree(dL, dU, dW, dA, k, beam, N, mask=True)
        torch.cuda.synchronize()
        for key in ("tok", "parent", "depth", "n_nodes", "score", "mask"):
            assert torch.equal(got[key], getattr(ref, key)), key
        assert int(got["n_nodes"].min()) > 0


def test_noalloc_rejects_workspace_above_the_array():
    lib = _lib()
    sh = pct.TreeShape(4096, 16, 151936, 256, 8, 16, 256, pct.PCT_BF16)
    assert lib.pct_build_tree_workspace(C.byref(sh)) > 32 << 20
    d = C.c_void_p(256)
    rc = lib.pct_build_tree_noalloc(C.byref(sh), d, d, d, d, d, d, d, d, d,
                                    None, None)
    assert rc == 2
    assert b"exceeds" in lib.pct_last_error()
