"""Writes the CPU oracle's trees for every request of the full-size tree
workloads, for the GPU parity tests to compare against.

    python tests/golden/make_golden.py b16 round [--procs 8]

Each request is built by the oracle (oracle/) from the seeded inputs of
synth/ in its own worker process; nothing here computes any part of the
method.  Output: tests/golden/<workload>_trees.npz with, per request, the
tree (tok, parent, depth, score), n_nodes, the oracle's smallest selection
gap (min_gap) and its per-depth beam / top-N boundary gaps (depth_gap), and
the workload's shape in `shape` (seed, batch, B, V, k, beam_w, N, r).
"""
from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

_W = {}


def _init(name):
    w = synth.TREE_WORKLOADS[name]
    _W["w"] = w
    _W["UW"] = synth.markov_factors(w.seed, w.V, w.r, w.bf16)


def _one(q):
    w = _W["w"]
    U, W = _W["UW"]
    L = synth.drafter_logits(w.seed, 1, w.B, w.V, w.var, w.temp_range, req0=q)
    A = synth.anchors(w.seed, 1, w.V, req0=q)
    o = oracle.build_tree(L, U, W, A, w.k, w.beam_w, w.N)
    return q, {k: v[0] for k, v in o.items()}


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"{name}_trees.npz")


def make(name: str, procs: int):
    w = synth.TREE_WORKLOADS[name]
    t0 = time.time()
    out = {"tok": np.empty((w.batch, w.N), np.int32),
           "parent": np.empty((w.batch, w.N), np.int32),
           "depth": np.empty((w.batch, w.N), np.int32),
           "score": np.empty((w.batch, w.N), np.float32),
           "n_nodes": np.empty(w.batch, np.int32),
           "min_gap": np.empty(w.batch, np.float64),
           "depth_gap": np.empty((w.batch, w.B + 1), np.float64)}
    ctx = mp.get_context("fork")
    with ctx.Pool(procs, initializer=_init, initargs=(name,)) as pool:
        for q, o in pool.imap_unordered(_one, range(w.batch)):
            for k in out:
                out[k][q] = o[k]
            print(f"{name}: request {q} done ({time.time() - t0:.0f}s)",
                  flush=True)
    shape = np.array([w.seed, w.batch, w.B, w.V, w.k, w.beam_w, w.N, w.r],
                     np.int64)
    np.savez_compressed(golden_path(name), shape=shape, **out)
    print(f"wrote {golden_path(name)} in {time.time() - t0:.0f}s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+", choices=["b16", "round"])
    ap.add_argument("--procs", type=int, default=8)
    args = ap.parse_args()
    for name in args.workloads:
        make(name, args.procs)


if __name__ == "__main__":
    main()
