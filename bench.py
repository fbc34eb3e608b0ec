"""Benchmark of libpctree on one MI355X.

One step = one pass of the whole hot path over one batch of the "b16"
workload (batch 32, V = 151936, B = 16, k = 8, beam 16, N = 256, rank-256
bf16 Markov factors): the parent-conditioned tree build (seed pre-pass, 16
depths of fused Markov / log-sum-exp / top-k + per-request expand, global
top-N), its packed ancestry mask, and the acceptance walk against synthetic
target tokens (prepared before the timed region).  Inputs are resident in
HBM before timing starts.

Prints one JSON line (rank 0):
  value        draft trees per second (whole job)
  roofline     the fused Markov kernel at 512 parents per launch (depths 3..16)
               against bf16 dense MFMA peak.  Its launch durations come from
               HIP events that the library records on the launch stream
               around every launch, over a second pass of the same K steps
               (so that `value` is timed without events); `traffic` is the
               counted HBM bytes per launch from profiles/, or null when the
               kernel changed since the counters were taken
  markov_memory_bound_depths
               the fused kernel's launches at depths 1 and 2 (32 and 256
               parents) against HBM peak: W once + the launch's L rows +
               the parents' U rows, per launch
  step_ms      median / p10 / p90 of per-step HIP-event times (a separate
               pass with one event pair per step)
  cpu_baseline the CPU oracle on a bounded sample of the same workload, on
               one pinned host core; cpu_baselines adds the tiny, b7 and
               adaptive workloads timed in full
  round        batch 128, N = 512: build, 512x512 masks and the acceptance
               walk timed separately and summed (medians of per-step events)
  b7_latency   batch 1, B = 7, N = 64 build + mask latency, and
               verification of that tree with temperature sampling
  adaptive     the adaptive best-first build (batch 64, n_max 1024) with its
               row-statistics kernels (single-read pieces, their merge and
               the full-length pass) against HBM peak
  adaptive_pc  the throughput stop on the parent-conditioned tree (the b16
               inputs, k = beam = N = 20, the adaptive workload's cost model)
  budget_grid  fixed budgets of every size (one build without a cost model
               + the throughput curve) against the adaptive budget
  cost_model   a fit of the verification cost from synthetic latency samples
               and the throughput lost to fitted or perturbed cost models
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0


# Kernel sources whose HBM traffic was counted (profiles/*_traffic.md); a
# recorded figure is used only while the digest of these files still matches.
TRAFFIC_SOURCES = {
    "markov": ("k_markov_impl.h", "k_markov.hip", "k_markov_r16s.hip",
               "pct_internal.h", "pct_device.h"),
    "rowsel": ("k_adaptive.hip", "pct_internal.h", "pct_device.h"),
}
TRAFFIC_FILES = {"markov": "markov_topk_mfma_b16_traffic.md",
                 "rowsel": "rowsel_adaptive_traffic.md"}


def source_digest(kernel):
    """sha256 of the kernel's sources with comments and blank space removed
    (editing a comment does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kernel]:
        with open(os.path.join(ROOT, "draft_tree_construction_markov_amd",
                               "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def traffic_of(kernel, launches=1):
    """HBM bytes per launch (times `launches`) from the committed counter
    summary, or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILES[kernel])
    try:
        fields = {}
        for line in open(path):
            if ":" in line and line.split(":", 1)[0] in (
                    "source_digest", "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                fields[k] = v.strip().strip("`")
        if fields.get("source_digest") != source_digest(kernel):
            return None
        return float(fields["traffic_bytes_per_launch"]) * launches
    except (OSError, KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-requests", type=int, default=2,
                    help="requests of the workload timed on the CPU oracle")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-adaptive", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the b16 workload (profiling runs)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run a plain device copy of this size first "
                         "(traffic-counter calibration)")
    return ap.parse_args()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                          "--gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    import draft_tree_construction_markov_amd as pct
    import synth

    dev = torch.device("cuda:0")
    w = synth.TREE_WORKLOADS["b16"]
    t0 = time.time()
    L, U, W, A = synth.tree_inputs(w)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    dL = torch.from_numpy(L).to(dev)
    dU, dW = pct.bf16_tensor(U, dev), pct.bf16_tensor(W, dev)
    dA = torch.from_numpy(A).to(dev)
    tb = pct.TreeBuilder(w.batch, w.B, w.V, w.k, w.beam_w, w.N, r=w.r,
                         bf16=True, mask=True, device=dev)
    out = tb.run(dL, dU, dW, dA)
    torch.cuda.synchronize()
    g = out.numpy()
    tgt = synth.targets_from_tree(w.seed, g["tok"], g["parent"], g["depth"],
                                  g["n_nodes"], A, w.V, w.B,
                                  synth.round_agreement(w.B))
    dT = torch.from_numpy(tgt).to(dev)
    vout = (torch.empty(w.batch, dtype=torch.int32, device=dev),
            torch.empty(w.batch, w.B, dtype=torch.int32, device=dev),
            torch.empty(w.batch, w.B + 1, dtype=torch.int32, device=dev))

    def step():
        o = tb.run(dL, dU, dW, dA)
        pct.verify_accept(o.tok, o.parent, o.depth, o.n_nodes, dT, w.B,
                          out=vout, mask=o.mask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.calib_copy_mb:
        # a plain device copy of known size, for scaling traffic counters
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: K steps, inputs resident, no instrumentation
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t1) * 1e3 / args.steps

    # the same K steps again with HIP events around every launch (on the
    # launch stream, recorded by the library) for per-kernel durations
    pct.profile_reset()
    pct.profile_enable(True)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step_ev = (time.perf_counter() - t3) * 1e3 / args.steps
    pct.profile_enable(False)
    step_ms = step_stats(torch, step, args.steps)
    P_steady = w.batch * w.beam_w
    k1_ms, k1_n = pct.profile_read(pct.PROF_MARKOV, P_steady)
    k1_all_ms, k1_all_n = pct.profile_read(pct.PROF_MARKOV, -1)
    # the memory-bound depths: 1 (the anchors, one parent per request) and
    # 2 (the anchors' children that the beam keeps); algorithmic bytes =
    # W once + the launch's L rows (one per request) + the parents' U rows
    shallow = {}
    for d, P in ((1, w.batch), (2, w.batch * min(w.k, w.beam_w))):
        ms, nl = pct.profile_read(pct.PROF_MARKOV, P)
        if nl:
            byts = 2.0 * w.V * w.r + w.batch * 4.0 * w.V + P * 2.0 * w.r
            gbs = byts / (ms / nl * 1e-3) / 1e9
            shallow[f"depth{d}"] = {"parents": P, "avg_launch_ms": round(ms / nl, 5),
                                    "bytes": int(byts), "achieved_GBs": round(gbs, 1),
                                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    kinds = {"markov": pct.PROF_MARKOV, "expand": pct.PROF_EXPAND,
             "topn": pct.PROF_TOPN, "mask": pct.PROF_MASK,
             "accept": pct.PROF_ACCEPT, "rowtop": pct.PROF_ROWTOP,
             "init": pct.PROF_INIT}
    per_kind = {}
    for name, kd in kinds.items():
        ms, n = pct.profile_read(kd, -1)
        per_kind[name] = round(ms / args.steps, 4)
    pct.profile_reset()

    trees_s = w.batch / (ms_step / 1e3)
    nodes_s = w.batch * w.N / (ms_step / 1e3)
    tau = vout[0].cpu().numpy()

    flop_per_parent = 2.0 * w.r * w.V
    k1_avg_ms = k1_ms / max(k1_n, 1)
    achieved = P_steady * flop_per_parent / (k1_avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_of("markov"),
                "kernel": "markov_topk_mfma<2,8,16> (512 parents/launch)",
                "avg_launch_ms": round(k1_avg_ms, 5),
                "launches": k1_n}

    res = {
        "metric": "draft trees/sec & nodes/sec (V=151936,B=16,N=256,"
                  "batch 32); % HBM/MFMA peak",
        "value": round(trees_s, 1),
        "unit": "trees/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-mfma/fp32",
        "data": "synthetic",
        "config": {"workload": "b16: batch 32, V=151936, B=16, k=8, beam 16,"
                               " N=256, r=256 bf16 Markov factors; build + "
                               "mask + acceptance walk",
                   "global_batch": w.batch, "parallelism": "none (1 GPU)"},
        "nodes_per_sec": round(nodes_s, 1),
        "step_ms": step_ms,
        "ms_per_step_with_events": round(ms_step_ev, 4),
        "kernel_ms_per_step": per_kind,
        "markov_all_launches": {"ms_per_step": round(k1_all_ms / args.steps, 4),
                                "launches_per_step": k1_all_n // args.steps},
        "markov_memory_bound_depths": shallow,
        "mean_tau": float(np.mean(tau)),
        "roofline": roofline,
    }

    if not args.no_extra:
        res["round"] = bench_round(args, pct, synth, torch, dev)
        res["b7_latency"] = bench_b7(args, pct, synth, torch, dev)
        res["adaptive_pc"] = bench_adaptive_pc(args, pct, synth, torch, dev,
                                               dL, dU, dW, dA)
    if not args.no_adaptive:
        res["adaptive"], extra = bench_adaptive(args, pct, synth, torch, dev)
        if not args.no_extra:
            res["budget_grid"], res["cost_model"] = extra

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args, w, L, U, W, A)
        if not args.no_extra:
            res["cpu_baselines"] = cpu_baselines(synth)
    print(json.dumps(res), flush=True)


def pct_stats(xs):
    xs = np.sort(np.asarray(xs, np.float64))
    return {"median": round(float(np.median(xs)), 5),
            "p10": round(float(np.percentile(xs, 10)), 5),
            "p90": round(float(np.percentile(xs, 90)), 5)}


def step_stats(torch, fn, steps):
    """Per-step HIP-event times (ms) of fn on the current stream."""
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return pct_stats([a.elapsed_time(b) for a, b in ev])


def bench_round(args, pct, synth, torch, dev):
    """The full round: batch 128, N = 512 build, masks, acceptance walk."""
    w = synth.TREE_WORKLOADS["round"]
    t0 = time.time()
    L, U, W, A = synth.tree_inputs(w)
    log(f"round inputs in {time.time() - t0:.1f}s")
    dL = torch.from_numpy(L).to(dev)
    dU, dW = pct.bf16_tensor(U, dev), pct.bf16_tensor(W, dev)
    dA = torch.from_numpy(A).to(dev)
    del L
    tb = pct.TreeBuilder(w.batch, w.B, w.V, w.k, w.beam_w, w.N, r=w.r,
                         bf16=True, mask=False, device=dev)
    o = tb.run(dL, dU, dW, dA)
    torch.cuda.synchronize()
    g = o.numpy()
    tgt = torch.from_numpy(synth.targets_from_tree(
        w.seed, g["tok"], g["parent"], g["depth"], g["n_nodes"], A, w.V, w.B,
        synth.round_agreement(w.B))).to(dev)
    words = (w.N + 63) // 64
    mask = torch.empty(w.batch, w.N, words, dtype=torch.int64, device=dev)
    vout = (torch.empty(w.batch, dtype=torch.int32, device=dev),
            torch.empty(w.batch, w.B, dtype=torch.int32, device=dev),
            torch.empty(w.batch, w.B + 1, dtype=torch.int32, device=dev))
    parts = {
        "build": lambda: tb.run(dL, dU, dW, dA),
        "mask": lambda: pct.tree_mask(o.parent, o.n_nodes, out=mask),
        "verify": lambda: pct.verify_accept(o.tok, o.parent, o.depth,
                                            o.n_nodes, tgt, w.B, out=vout,
                                            mask=mask),
    }
    for _ in range(args.warmup):
        for f in parts.values():
            f()
    ev = {k: [] for k in parts}
    torch.cuda.synchronize()
    for _ in range(args.steps):
        for k, f in parts.items():
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            ev[k].append((a, b))
    torch.cuda.synchronize()
    out = {k: pct_stats([a.elapsed_time(b) for a, b in v])
           for k, v in ev.items()}
    total = sum(out[k]["median"] for k in parts)
    tau = vout[0].cpu().numpy()
    return {"workload": "round: batch 128, V=151936, B=16, k=8, beam 16, "
                        "N=512, r=256 bf16; build + 512x512 masks + walk",
            "ms": out, "round_ms_median_sum": round(total, 5),
            "trees_per_sec": round(w.batch / (total / 1e3), 1),
            "nodes_per_sec": round(w.batch * w.N / (total / 1e3), 1),
            "mean_tau": float(tau.mean())}


def bench_b7(args, pct, synth, torch, dev):
    """Latency of one batch-1, B = 7, N = 64 build with its 64x64 mask."""
    w = synth.TREE_WORKLOADS["b7"]
    L, U, W, A = synth.tree_inputs(w)
    dL = torch.from_numpy(L).to(dev)
    dU, dW = pct.bf16_tensor(U, dev), pct.bf16_tensor(W, dev)
    dA = torch.from_numpy(A).to(dev)
    tb = pct.TreeBuilder(w.batch, w.B, w.V, w.k, w.beam_w, w.N, r=w.r,
                         bf16=True, mask=True, device=dev)
    for _ in range(args.warmup):
        tb.run(dL, dU, dW, dA)
    st = step_stats(torch, lambda: tb.run(dL, dU, dW, dA), max(args.steps, 20))
    # verification with temperature sampling on this tree: the target's
    # logits after the root and after each of the 64 nodes (synthetic,
    # generated before timing), Gumbel-max samples, then the walk
    tl = torch.from_numpy(synth.drafter_logits(w.seed + 17, 1, w.N + 1, w.V,
                                               3.0)).to(dev)
    o = tb.out
    outs = (torch.empty(1, w.N + 1, dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int32, device=dev),
            torch.empty(1, w.B, dtype=torch.int32, device=dev),
            torch.empty(1, w.B + 1, dtype=torch.int32, device=dev))
    sws = torch.empty(max(1, int(pct.lib().pct_verify_sample_workspace(
        1, w.N, w.V))), dtype=torch.uint8, device=dev)
    sv = lambda: pct.verify_sample(o.tok, o.parent, o.depth, o.n_nodes, tl,  # noqa: E731
                                   w.B, 0.8, 12345, mask=o.mask, out=outs,
                                   workspace=sws)
    sv()
    ss = step_stats(torch, sv, max(args.steps, 20))
    rows = w.N + 1
    return {"workload": "b7: batch 1, V=151936, B=7, k=8, beam 8, N=64, "
                        "r=256 bf16; build + 64x64 mask",
            "latency_ms": st,
            "verify_sample": {"what": "65 rows of V=151936 target logits, "
                                      "T = 0.8: Gumbel-max samples in "
                                      "double + acceptance walk",
                              "latency_ms": ss,
                              "logits_GBs": round(rows * w.V * 4 /
                                                  (ss["median"] * 1e-3) /
                                                  1e9, 1)}}


def bench_adaptive_pc(args, pct, synth, torch, dev, dL, dU, dW, dA):
    """Throughput stop on the parent-conditioned tree over the b16 inputs."""
    w = synth.TREE_WORKLOADS["b16"]
    a = synth.ADAPTIVE
    cost = {k: a[k] for k in ("C_d", "c0", "c1", "c2", "c_ell")}
    ctx = torch.from_numpy(synth.context_lengths(w.seed, w.batch)).to(dev)
    kk = 20
    ab = pct.AdaptivePCBuilder(w.batch, w.B, w.V, kk, kk, kk, cost, r=w.r,
                               bf16=True, mask=True, device=dev)
    for _ in range(args.warmup):
        ab.run(dL, dU, dW, dA, ctx)
    st = step_stats(torch, lambda: ab.run(dL, dU, dW, dA, ctx), args.steps)
    ns = ab.n_star.cpu().numpy()
    med = st["median"]
    return {"workload": "b16 inputs (batch 32, V=151936, B=16, r=256) with "
                        "k = beam = N = 20 (the kept tree is the best-first "
                        "tree when n* <= 20), adaptive cost model",
            "step_ms": st, "trees_per_sec": round(w.batch / (med / 1e3), 1),
            "n_star_mean": float(ns.mean()), "n_star_std": float(ns.std()),
            "n_star_max": int(ns.max())}


def grid_and_cost(pct, torch, dL, dC, a, cost, ab_star):
    """Budget grid search (DDTree-style fixed budgets) and the cost-model
    fit / robustness sweep, on the adaptive workload's curves."""
    from draft_tree_construction_markov_amd import costmodel as cm
    fixed = pct.AdaptiveBuilder(a["batch"], a["B"], a["V"], a["n_max"], None,
                                device=dL.device).run(dL, dC)

    def curve(c):
        return pct.throughput_curve(fixed.score, fixed.n_star, dC,
                                    c).cpu().numpy()
    f = curve(cost)
    rows = np.arange(f.shape[0])
    mean_f = f.mean(axis=0)
    n_fix = int(np.argmax(mean_f))
    f_ad = f[rows, ab_star]
    grid = {"fixed_budgets": "every n in 0..1024 (one build, n_max 1024, "
                             "no cost model; f from pct_throughput_curve)",
            "best_fixed_budget": n_fix,
            "mean_f_best_fixed": round(float(mean_f[n_fix]), 6),
            "mean_f_adaptive": round(float(f_ad.mean()), 6),
            "adaptive_gain": round(float(f_ad.mean() / mean_f[n_fix] - 1), 6),
            "mean_f_oracle_budget_per_round": round(float(f.max(1).mean()),
                                                    6),
            "n_star_mean": float(ab_star.mean()),
            "n_star_std": float(ab_star.std())}
    rng = np.random.default_rng(7)
    n = rng.integers(1, 1025, size=600)
    ell = np.rint(np.exp(rng.uniform(np.log(512), np.log(32768), size=600)))
    y = cm.predict(cost, n, ell) * (1 + 0.05 * rng.normal(size=600))
    fit = cm.fit(n, ell, y, weights=1.0 / y ** 2)
    models = {"fitted": fit.cost(cost["C_d"]),
              "c1 x2": cm.perturbed(cost, {"c1": 2.0}),
              "c_ell x0.5": cm.perturbed(cost, {"c_ell": 0.5}),
              "c0 x0.5": cm.perturbed(cost, {"c0": 0.5}),
              "all x1.5": cm.perturbed(cost, {k: 1.5 for k in cm.FEATURES})}
    rob = cm.robustness(curve, cost, models)
    costm = {"samples": "600 synthetic (n, l) latencies of the adaptive "
                        "workload's cost model with 5% noise",
             "fitted": {k: getattr(fit, k) for k in cm.FEATURES},
             "true": {k: cost[k] for k in cm.FEATURES},
             "robustness_rel_loss": {k: round(v["rel_loss"], 6)
                                     for k, v in rob.items()}}
    return grid, costm


def bench_adaptive(args, pct, synth, torch, dev):
    a = synth.ADAPTIVE
    t0 = time.time()
    L, peaked, ctx = synth.adaptive_round(a["seed"], a["batch"], a["B"],
                                          a["V"])
    log(f"adaptive inputs in {time.time() - t0:.1f}s")
    dL = torch.from_numpy(L).to(dev)
    dC = torch.from_numpy(ctx).to(dev)
    cost = {k: a[k] for k in ("C_d", "c0", "c1", "c2", "c_ell")}
    ab = pct.AdaptiveBuilder(a["batch"], a["B"], a["V"], a["n_max"], cost,
                             mask=True, device=dev)
    for _ in range(args.warmup):
        ab.run(dL, dC)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        ab.run(dL, dC)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    # the same steps again with per-launch events: the row-statistics time
    # of a step is every row-statistics launch in it (the full-length pass
    # only touches rows of requests that outgrew the short lists)
    pct.profile_reset()
    pct.profile_enable(True)
    for _ in range(args.steps):
        ab.run(dL, dC)
    torch.cuda.synchronize()
    pct.profile_enable(False)
    rs_ms, rs_n = pct.profile_read(pct.PROF_ROWSTATS, -1)
    bf_ms, _ = pct.profile_read(pct.PROF_BESTFIRST, -1)
    pct.profile_reset()
    st = step_stats(torch, lambda: ab.run(dL, dC), args.steps)
    ns = ab.n_star.cpu().numpy()
    extra = grid_and_cost(pct, torch, dL, dC, a, cost, ns)
    bytes_rows = float(L.nbytes)
    rs_step = rs_ms / args.steps
    gbs = bytes_rows / (rs_step * 1e-3) / 1e9
    return {"workload": "adaptive: batch 64, V=151936, B=16, n_max=1024, "
                        "marginal rows, half peaked / half flat",
            "trees_per_sec": round(a["batch"] / (ms / 1e3), 1),
            "nodes_per_sec": round(float(ns.sum()) / (ms / 1e3), 1),
            "ms_per_step": round(ms, 4), "step_ms": st,
            "n_star_mean": float(ns.mean()), "n_star_std": float(ns.std()),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_of("rowsel"),  # per step
                         "kernel": "row statistics: rowpart_kernel + "
                                   "rowmerge_kernel + full-length "
                                   "rowsel_kernel pass (1024 rows/step)",
                         "ms_per_step": round(rs_step, 5),
                         "launches_per_step": rs_n // args.steps},
            "bestfirst_ms_per_step": round(bf_ms / args.steps, 5)}, extra


class one_core:
    """Pin this process to one host core while the oracle runs."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.core = min(self.saved)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def cpu_baseline(args, w, L, U, W, A):
    import oracle
    n = args.cpu_requests
    with one_core() as c:
        t0 = time.perf_counter()
        oracle.build_tree(L[:n], U, W, A[:n], w.k, w.beam_w, w.N)
        el = time.perf_counter() - t0
    return {"value": round(n / el, 4), "unit": "trees/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {n} requests of the b16 workload, tree build "
                      f"only, single-threaded C oracle ({el:.1f}s) pinned to "
                      f"core {c.core} of {cpu_model()}, "
                      f"nproc={os.cpu_count()}"}


def cpu_baselines(synth):
    """The oracle on the tiny, b7 and adaptive workloads in full, on one
    pinned core (inputs drawn before the clock starts)."""
    import oracle
    out = {}
    for name in ("tiny", "b7"):
        w = synth.TREE_WORKLOADS[name]
        L, U, W, A = synth.tree_inputs(w)
        with one_core():
            t0 = time.perf_counter()
            oracle.build_tree(L, U, W, A, w.k, w.beam_w, w.N)
            el = time.perf_counter() - t0
        out[name] = {"requests": w.batch, "seconds": round(el, 4),
                     "trees_per_sec": round(w.batch / el, 4)}
    a = synth.ADAPTIVE
    L, peaked, ctx = synth.adaptive_round(a["seed"], a["batch"], a["B"],
                                          a["V"])
    cost = {k: a[k] for k in ("C_d", "c0", "c1", "c2", "c_ell")}
    with one_core():
        t0 = time.perf_counter()
        for q in range(a["batch"]):
            oracle.adaptive(L[q], a["n_max"], int(ctx[q]), cost)
        el = time.perf_counter() - t0
    out["adaptive"] = {"requests": a["batch"], "seconds": round(el, 4),
                       "trees_per_sec": round(a["batch"] / el, 4)}
    out["cores"] = 1
    return out


if __name__ == "__main__":
    main()
