"""Helpers for the GPU parity tests (device tensors from the seeded inputs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import draft_tree_construction_markov_amd as pct


def announce(*what):
    """Name the case before a GPU step (flushed, so a fault still shows)."""
    print("[gpu-case]", *what, flush=True)
    sys.stdout.flush()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def dev_factors(U, W):
    if U is None:
        return None, None
    if U.dtype == np.uint16:
        return pct.bf16_tensor(U), pct.bf16_tensor(W)
    return dev_f32(U), dev_f32(W)


def tree_numpy(out):
    d = out.numpy()
    d["min_gap"] = None
    return d
