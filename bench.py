"""Benchmark of the ManifoldKV eviction hot path on one MI355X.

Workload (default): a Llama-3.1-8B-shaped KV cache, 32 layers x 8 KV heads
(256 slices), head dim 128, batch 1, S = 16384 tokens, bf16 K/V drawn with
per-channel offsets, lognormal norm scales and 64 planted x4 outliers per
head; global-centroid L2 scoring, 50% eviction (keep 8192 per head) and
compaction of K and V.  One step = score every key + select + compact.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line: head-tokens scored+compacted per second, the roofline
of the dominant kernel (algorithmic bytes / its average launch time, from HIP
events on the launch stream) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every slice is "
              "independent; sharding is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from token_scoring_eviction_amd import kvc, pipeline

    kvc.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L, H, S, keep = 32, 8, 16384, 8192
    G = L * H
    K, V, _ = synth.manifold_global(L, 1, H, S, planted=64, device=dev)
    buf = pipeline.alloc_eviction(G, S, keep, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        kvc.kvc_score_l2(K, scores=buf.scores)
        if ev is not None:
            ev[1].record()
        kvc.kvc_topk_compact(buf.scores, keep, K, V, idx_out=buf.idx, K_out=buf.K_out, V_out=buf.V_out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing: K steps between two synchronizations
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps

    # per-entry-point timing with events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    score_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    topk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    head_tokens = G * S
    # algorithmic (compulsory) bytes
    by_score = G * S * (128 * 2 + 4)                       # K read once, fp32 score written
    by_topk = G * S * 4 + 2 * G * keep * 128 * 2 * 2 + G * keep * 4  # scores, kept K/V rows r+w, idx
    by_step = G * S * 128 * 2 + G * keep * 128 * 2 + 2 * G * keep * 128 * 2 + G * S * 4 + G * keep * 4
    ops = {
        "kvc_score_l2": {"ms": score_ms, "bytes": by_score, "GBs": by_score / score_ms / 1e6},
        "kvc_topk_compact": {"ms": topk_ms, "bytes": by_topk, "GBs": by_topk / topk_ms / 1e6},
    }
    dom = max(ops, key=lambda n: ops[n]["ms"])
    achieved = ops[dom]["GBs"]
    line = {
        "metric": "KV head-tokens scored+compacted/s",
        "value": head_tokens / (ms_step / 1e3),
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ManifoldKV global-L2 eviction, 32 layers x 8 KV heads x d_h 128, "
                               "batch 1, S=16384, keep 8192 (50%)",
                   "slices": G, "seq_len": S, "keep": keep, "head_dim": 128},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "step_hbm": {"algorithmic_bytes": by_step, "GBs": by_step / ms_step / 1e6,
                     "frac": by_step / ms_step / 1e6 / HBM_PEAK_GBS},
        "ops": ops,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(K, V, keep, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def cpu_baseline(K, V, keep, budget_s):
    """The oracle (single-threaded C, fp64) on the first slices of the same
    workload, as many as fit in about budget_s seconds."""
    import numpy as np

    import oracle
    import synth
    G, S, _ = K.shape
    done = 0
    t = 0.0
    while done < G and t < budget_s:
        kb = synth.bf16_bits(K[done:done + 1])
        vb = synth.bf16_bits(V[done:done + 1])
        t0 = time.perf_counter()
        sc, _ = oracle.score_l2(kb)
        idx = oracle.topk(sc.astype(np.float32), keep)
        oracle.gather(kb, idx)
        oracle.gather(vb, idx)
        t += time.perf_counter() - t0
        done += 1
    return {"value": done * S / t, "unit": "head-tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d of %d slices (S=%d each) of the same workload, %.1f s" % (done, G, S, t)}


if __name__ == "__main__":
    main()
