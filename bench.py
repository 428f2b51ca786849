"""Benchmark of the KV-cache scoring / compaction hot path on one MI355X.

Default workload (the headline): ManifoldKV eviction of a Llama-3.1-8B-shaped
KV cache -- 32 layers x 8 KV heads (256 slices), head dim 128, batch 1,
S = 16384 tokens, bf16 K/V drawn with per-channel offsets, lognormal norm
scales and 64 planted x4 outliers per head -- scored against the global key
centroid, 50% evicted (keep 8192 per head), K and V compacted.  One step =
score every key + select + compact.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--no-cpu-baseline]

--config 0..4 measures the other synthetic workloads instead (0: 8 slices at
S=4096 keep 3277; 2: windowed W=4096 at S=65536 keep 49152; 3: OjaKV prefill
compression B=4, S=32768, r=64 with 5% anchors; 4: the OjaKV prefill + 256
decode-step loop at S=131072).  Prints one JSON line: head-tokens/s; the
roofline of the whole step (its algorithmic bytes -- K read once, kept V rows
read, kept K/V written, scores and indices written, low-rank outputs written --
over the step's time, HIP events on the launch stream), with the dominant
kernel named; per entry point, its share of those bytes and its time; and the
CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0    # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_digest(path):
    import hashlib
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(entry_point, workload):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of an entry point on a
    workload ("config<N>" or "refine"), as recorded from rocprofv3 counter runs
    (profiles/hbm_traffic.json); None when absent or when the kernel source
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["entries"]["%s/%s" % (entry_point, workload)]
    except (OSError, KeyError, ValueError):
        return None
    if any(source_digest(p) != h for p, h in rec["sources"].items()):
        return None
    return rec["bytes_per_launch"]


def step_traffic(ops, workload):
    """Counter bytes of one step: the sum over its entry points, or None unless every
    one of them has a current record."""
    parts = [measured_traffic(op.name, workload) for op in ops]
    return None if any(x is None for x in parts) else sum(parts)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--metric", choices=["l2", "cosine"], default="l2",
                    help="centroid score of configs 0-2: ManifoldKV's L2 distance (the workload) "
                         "or the cosine-dissimilarity baseline")
    ap.add_argument("--budgets", choices=["uniform", "ripple"], default="uniform",
                    help="configs 0-2: every slice keeps the same k (the workload) or per-layer "
                         "RippleKV budgets (seeded sensitivity profile, r=8, gamma=4) with the same total")
    ap.add_argument("--storage", choices=["fp32", "bf16"], default="fp32",
                    help="OjaKV configs 3-4: compressed cache (K~, V~, K^, V^) in fp32 (the "
                         "workload) or bf16 (the memory-saving layout)")
    ap.add_argument("--refine", action="store_true",
                    help="time RefineKV cluster summaries (10-key clusters) and risk scores (4 queries "
                         "per kv head) on a 32-layer x 8-kv-head cache of 131072 tokens instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="only time a plain device-to-device copy of MIB MiB (the reference "
                         "kernel for scaling HBM traffic counters) and exit")
    return ap.parse_args()


def time_device_copy(mib, reps):
    """A plain device-to-device copy of MIB MiB: (ms per copy, GB/s read + write)."""
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    return ms, 2 * n / ms / 1e6


def copy_reference(mib, reps):
    ms, gbs = time_device_copy(mib, reps)
    print(json.dumps({"copy_bytes": mib << 20, "ms": ms, "GBs_read_plus_write": gbs}), flush=True)


def host_cpu():
    """Model name of the host CPU and the threads the OS reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def run_cpu_baseline(cpu, seconds):
    """The oracle on one host core: this thread is pinned to the core it runs on
    for the sample, then its affinity is restored."""
    before = None
    try:
        before = os.sched_getaffinity(0)
        core = sorted(before)[0]
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        core = None
    try:
        n, t, sample = cpu(seconds)
    finally:
        if before is not None:
            os.sched_setaffinity(0, before)
    model, threads = host_cpu()
    return {"value": n / t, "unit": "head-tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s, %.1f s" % (sample, t), "pinned_core": core, "host_cpu": model,
            "host_threads": threads}


class Op:
    """An entry-point call inside a step.  nbytes: its share of the step's
    algorithmic bytes (what the method must move: K once, kept V rows, kept K/V
    written, scores, indices, low-rank outputs); moved: the bytes this
    implementation has to move for it (adds re-reads, e.g. the selection's read of
    the scores and the copy's read of the kept K rows); flops: the method's own
    dense-contraction flops (no split-operand passes)."""

    def __init__(self, name, fn, nbytes, flops=0, kernel=None, moved=None):
        self.name, self.fn, self.nbytes, self.flops = name, fn, nbytes, flops
        self.kernel = kernel or name
        self.moved = nbytes if moved is None else moved
        self.ms = []


def manifold_workload(cfg, dev, metric="l2", budgets="uniform"):
    import torch

    import synth
    from token_scoring_eviction_amd import kvc, pipeline
    if cfg == 0:
        L, H, S, keep, W = 1, 8, 4096, 3277, None
        K, V, _ = synth.manifold_global(L, 1, H, S, planted=16, device=dev)
        desc = "ManifoldKV global-L2 eviction, 1 layer x 8 KV heads x d_h 128, S=4096, keep 3277 (drop 20%)"
    elif cfg == 1:
        L, H, S, keep, W = 32, 8, 16384, 8192, None
        K, V, _ = synth.manifold_global(L, 1, H, S, planted=64, device=dev)
        desc = ("ManifoldKV global-L2 eviction, 32 layers x 8 KV heads x d_h 128, batch 1, "
                "S=16384, keep 8192 (50%)")
    else:
        L, H, S, keep, W = 32, 8, 65536, 49152, 4096
        K, V = synth.manifold_drifting(L, 1, H, S, device=dev)
        desc = ("Windowed ManifoldKV eviction, 32 layers x 8 KV heads x d_h 128, batch 1, "
                "S=65536, W=4096, keep 49152 (25% evicted)")
    G = L * H
    buf = pipeline.alloc_eviction(G, S, keep, device=dev)
    if metric == "cosine":
        score = lambda: kvc.kvc_score_centroid(K, W=W, metric="cosine", scores=buf.scores)
        score_name = "kvc_score_centroid"
        desc = desc.replace("ManifoldKV", "cosine-to-centroid").replace("global-L2", "global")
    elif W is None:
        score, score_name = (lambda: kvc.kvc_score_l2(K, scores=buf.scores)), "kvc_score_l2"
    else:
        score, score_name = (lambda: kvc.kvc_score_l2_windowed(K, W, scores=buf.scores)), "kvc_score_l2_windowed"
    # caches under 12 MiB of keys take the three-launch scoring path (second read from
    # the caches); larger ones the single-read kernel and its repair launch
    small = G * S * 256 < (12 << 20)
    score_kernel = ("centroid_partial+centroid_final+" + ("cosine_distance" if metric == "cosine" else "l2_distance")
                    if small else "l2_fused+l2_repair")
    # algorithmic bytes: K read once and the scores written (scoring); kept V rows read,
    # kept K and V rows written, indices written (compaction).  The selection's read of
    # the scores and the copy's read of the kept K rows are the implementation's own.
    ops = [Op(score_name, score, G * S * (256 + 4), kernel=score_kernel)]
    if budgets == "ripple":
        # per-layer budgets from a seeded sensitivity profile, same total as keep per slice
        import numpy as np
        sens = np.random.default_rng(20261202 + cfg).gamma(2.0, 1.0, L)
        kl = kvc.kvc_layer_budgets(sens, 8.0, 4.0, L * keep, S)
        ks = np.repeat(kl, H)
        total = int(ks.sum())
        kd = torch.from_numpy(ks.astype(np.int64)).to(dev)  # the budgets live on the device
        rbuf = (torch.empty(total, dtype=torch.int32, device=dev),
                torch.empty((total, 128), dtype=torch.bfloat16, device=dev),
                torch.empty((total, 128), dtype=torch.bfloat16, device=dev))
        ops.append(Op("kvc_topk_compact_ragged",
                      lambda: kvc.kvc_topk_compact_ragged(buf.scores, kd, K, V, idx_out=rbuf[0],
                                                          K_out=rbuf[1], V_out=rbuf[2], k_max=int(ks.max()),
                                                          k_total=total),
                      total * (3 * 256 + 4), moved=G * S * 4 + total * (4 * 256 + 4),
                      kernel="ragged_offsets+select_compact+gather_rows"))
        desc += "; RippleKV per-layer budgets %d..%d (r=8, gamma=4)" % (kl.min(), kl.max())
        kept = total
    else:
        ops.append(Op("kvc_topk_compact",
                      lambda: kvc.kvc_topk_compact(buf.scores, keep, K, V, idx_out=buf.idx, K_out=buf.K_out,
                                                   V_out=buf.V_out),
                      G * keep * (3 * 256 + 4), moved=G * S * 4 + G * keep * (4 * 256 + 4),
                      kernel="select_compact+gather_rows"))
        kept = G * keep
    algo = G * S * (256 + 4) + kept * (3 * 256 + 4)
    config = {"workload": desc, "slices": G, "seq_len": S, "keep": keep, "head_dim": 128,
              "window": W, "metric": metric, "budgets": budgets}

    def cpu(budget):
        import numpy as np
        import oracle
        done, t = 0, 0.0
        while t < budget and done < 64 * G:
            g = done % G
            kb = synth.bf16_bits(K[g:g + 1])
            vb = synth.bf16_bits(V[g:g + 1])
            t0 = time.perf_counter()
            if metric == "cosine":
                sc, _ = oracle.score_cosine_windowed(kb, W or S)
            else:
                sc, _ = oracle.score_l2(kb) if W is None else oracle.score_l2_windowed(kb, W)
            idx = oracle.topk(sc.astype(np.float32), keep)
            oracle.gather(kb, idx)
            oracle.gather(vb, idx)
            t += time.perf_counter() - t0
            done += 1
        return done * S, t, "%d slice passes (S=%d each; the workload has %d slices, taken in order)" % (
            done, S, G)

    return ops, G * S, algo, config, cpu


def refine_workload(dev):
    import torch

    import synth
    from token_scoring_eviction_amd import kvc
    L, H, S, c, nq = 32, 8, 131072, 10, 4
    G, nC = L * H, -(-S // c)
    K, V, _ = synth.manifold_global(L, 1, H, S, planted=64, device=dev)
    Q = torch.randn((G, nq, 128), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    summ = [torch.empty((G, nC, 128), **f32), torch.empty((G, nC, 128), **f32), torch.empty((G, nC), **f32),
            torch.empty((G, nC), **f32)]
    rc = torch.empty((G, nq, nC), **f32)

    def summaries():
        lib = kvc.load()
        kvc._check("kvc_cluster_summaries", lib.kvc_cluster_summaries(
            kvc._ptr(K), kvc._ptr(V), G, S, 128, c, *[kvc._ptr(t) for t in summ], kvc._stream()))

    # algorithmic bytes: K and V read once, summaries written; the risk pass reads the
    # mean keys, radii and value norms and writes one score per (query, cluster)
    ops = [Op("kvc_cluster_summaries", summaries, G * S * 512 + G * nC * (2 * 512 + 8),
              kernel="cluster_summary_kernel"),
           Op("kvc_refine_risk", lambda: kvc.kvc_refine_risk(summ[0], summ[2], summ[3], S, c, Q, rc=rc),
              G * nC * (512 + 8 + nq * 4), moved=G * nC * (512 + 8 + 3 * nq * 4),
              kernel="risk_partial_kernel+risk_final_kernel")]
    algo = sum(op.nbytes for op in ops)
    config = {"workload": "RefineKV cluster summaries (contiguous 10-key clusters: mean key, mean value, "
                          "key radius, value norm) and risk scores of every cluster for the 4 query heads "
                          "of each kv head, 32 layers x 8 KV heads x d_h 128, S=131072",
              "slices": G, "seq_len": S, "cluster": c, "queries": nq}

    def cpu(budget):
        import numpy as np
        import oracle
        done, t = 0, 0.0
        while t < budget and done < G:
            kb, vb = synth.bf16_bits(K[done:done + 1, :16384]), synth.bf16_bits(V[done:done + 1, :16384])
            qb = synth.bf16_bits(Q[done:done + 1])
            t0 = time.perf_counter()
            mk, _, rad, vn = oracle.cluster_summaries(kb, vb, c)
            oracle.refine_risk(mk, rad, vn, 16384, c, qb)
            t += time.perf_counter() - t0
            done += 1
        return done * 16384, t, "%d slices truncated to their first 16384 tokens" % done

    return ops, G * S, algo, config, cpu


def oja_workload(dev, storage="fp32"):
    import synth
    from token_scoring_eviction_amd import kvc, pipeline
    L, B, Hkv, Hq, S, R, Wq = 32, 4, 8, 32, 32768, 64, 32
    inp = synth.oja_inputs(L, B, Hkv, Hq, S, R=R, Wq=Wq, device=dev)
    G = L * B * Hkv
    k = pipeline.anchor_count(S)
    st = pipeline.alloc_hybrid(G, S, R, device=dev, max_anchor=k, with_hat=False, storage=storage)
    ob = 2 if storage == "bf16" else 4  # bytes per stored K~ / V~ element
    compress = kvc.kvc_lowrank_compress_bf16 if storage == "bf16" else kvc.kvc_lowrank_compress
    # the method's dense contractions per head-token: K~ = K U_k (2*128*R), the residual
    # r = k - U_k K~ (2*R*128), the window's products q.r over g*W_q queries
    # (2*128*g*W_q), V~ = V U_v (2*128*R): 81,920 flop at R = 64, g*W_q = 128
    flops_per_token = 2 * 128 * R + 2 * R * 128 + 2 * 128 * (Hq // Hkv) * Wq + 2 * 128 * R
    ops = [
        Op("kvc_lowrank_compress" + ("_bf16" if storage == "bf16" else ""),
           lambda: compress(inp.K, inp.V, inp.Q, inp.Uk, inp.Uv, L, B, Hkv,
                            K_tilde=st.Kt, V_tilde=st.Vt, err=st.err),
           G * S * (2 * 256 + 2 * R * ob + 4), flops=G * S * flops_per_token,
           kernel="prep_query_kernel+project_kernel"),
        Op("kvc_topk_compact",
           lambda: kvc.kvc_topk_compact(st.err, k, inp.K, inp.V, idx_out=st.idx, K_out=st.K_anchor,
                                        V_out=st.V_anchor),
           G * k * (3 * 256 + 4), moved=G * S * 4 + G * k * (4 * 256 + 4),
           kernel="select_compact+gather_rows"),
    ]
    algo = sum(op.nbytes for op in ops)
    config = {"workload": "OjaKV hybrid low-rank prefill compression, 32 layers x batch 4 x 8 KV heads "
                          "(32 query heads), d_h 128, S=32768, r=64, 32-query window, 5% anchors",
              "slices": G, "seq_len": S, "rank": R, "anchors": k, "storage": storage}

    def cpu(budget):
        import numpy as np
        import oracle
        done, t = 0, 0.0
        Uk, Uv = inp.Uk.cpu().numpy(), inp.Uv.cpu().numpy()
        while done < G and t < budget:
            g = done
            l, b, h = g // (B * Hkv), (g // Hkv) % B, g % Hkv
            kb, vb = synth.bf16_bits(inp.K[g:g + 1]), synth.bf16_bits(inp.V[g:g + 1])
            q = synth.bf16_bits(inp.Q[l:l + 1, b:b + 1, 4 * h:4 * h + 4])
            t0 = time.perf_counter()
            _, _, e = oracle.lowrank_compress(kb, vb, q, Uk[l:l + 1, h:h + 1], Uv[l:l + 1, h:h + 1],
                                              1, 1, 1, 4)
            idx = oracle.topk(e.astype(np.float32), k)
            oracle.gather(kb, idx)
            oracle.gather(vb, idx)
            t += time.perf_counter() - t0
            done += 1
        return done * S, t, "%d of %d slices (S=%d each) of the same workload" % (done, G, S)

    return ops, G * S, algo, config, cpu


def run_loop_config(args, dev):
    """Config 4: one step = the whole OjaKV loop (prefill + 256 decode steps, 8 updates)."""
    import torch

    import synth
    from token_scoring_eviction_amd import pipeline
    L, B, Hkv, Hq, S0, R, Wq, steps, T = 32, 1, 8, 32, 131072, 64, 32, 256, 32
    inp = synth.oja_inputs(L, B, Hkv, Hq, S0, R=R, Wq=Wq, S_cap=S0 + steps, device=dev)
    G = L * B * Hkv
    toks = [synth.decode_token(inp, s) for s in range(steps)]
    Uk0, Uv0 = inp.Uk.clone(), inp.Uv.clone()

    # the loop's dominant call, timed in place: HIP events on the launch stream around
    # every fused compression + reconstruction (K and V sides) of the timed loops
    from token_scoring_eviction_amd import kvc
    fused_name = ("kvc_lowrank_compress_reconstruct_bf16" if args.storage == "bf16"
                  else "kvc_lowrank_compress_reconstruct")
    fused_fn = getattr(kvc, fused_name)
    fused_calls = []  # (start event, end event, head-tokens) while recording
    recording = [False]

    def timed_fused(K, V, *a, **kw):
        if not recording[0]:
            return fused_fn(K, V, *a, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fused_fn(K, V, *a, **kw)
        e1.record()
        fused_calls.append((e0, e1, K.shape[0] * kw["S"]))
        return out

    setattr(kvc, fused_name, timed_fused)

    def loop(times=None):
        Uk, Uv = Uk0.clone(), Uv0.clone()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        st = pipeline.ojakv_prefill(inp.K, inp.V, inp.Q, Uk, Uv, L, B, Hkv, S0, T=T, pool=32, eta=1e-3,
                                    storage=args.storage)
        e[1].record()
        upd = []
        for s in range(steps):
            k, v, q = toks[s]
            if (s + 1) % T == 0:
                a = torch.cuda.Event(enable_timing=True)
                a.record()
            if pipeline.ojakv_decode_step(st, inp.K, inp.V, k, v, q, L, B, Hkv, T=T, eta=1e-3):
                b = torch.cuda.Event(enable_timing=True)
                b.record()
                upd.append((a, b))
        if times is not None:
            times.append((e, upd))
        return st

    # each loop allocates the hybrid state (about 70 GB at this size) in its prefill; the
    # previous loop's state is released first, so the caching allocator hands back the same
    # blocks instead of mapping new memory inside the timed region
    for _ in range(max(1, args.warmup // 5)):
        st = None
        st = loop()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 25)
    times = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    recording[0] = True
    st = None
    t0.record()
    for _ in range(reps):
        st = None
        st = loop(times)
    t1.record()
    torch.cuda.synchronize()
    recording[0] = False
    setattr(kvc, fused_name, fused_fn)
    ms = t0.elapsed_time(t1) / reps
    pre = sum(e[0].elapsed_time(e[1]) for e, _ in times) / reps
    upd = sum(sum(a.elapsed_time(b) for a, b in u) for _, u in times) / reps / 8
    scorings = G * sum(S0 + T * j for j in range(9))
    ob = 2 if args.storage == "bf16" else 4  # bytes per stored K~, V~, K^, V^ element
    per_pass = lambda S: (G * S * (2 * 256 + 2 * R * ob + 4 + 2 * 128 * ob)
                          + G * pipeline.anchor_count(S) * 1028)
    algo = G * S0 * 256 * 2 + sum(per_pass(S0 + T * j) for j in range(9))
    line = base_line(args, "KV head-tokens scored+compacted/s", scorings / (ms / 1e3), ms, reps,
                     {"workload": "OjaKV full loop: 32 layers x batch 1 x 8 KV heads (32 query heads), "
                                  "d_h 128, S=131072 prefill pooled by 32 + 256 decode steps, update "
                                  "every 32 (eta 1e-3, r=64, 5% anchors, K^/V^ rebuilt per update)",
                      "slices": G, "seq_len": S0, "decode_steps": steps, "updates": 8,
                      "storage": args.storage})
    line["phases_ms"] = {"prefill": pre, "per_update": upd, "whole_loop": ms}
    # algorithmic bytes of one fused call: K and V read, K~/V~ and K^/V^ written, e written
    fused_ms = sum(a.elapsed_time(b) for a, b, _ in fused_calls)
    fused_bytes = sum(n * (2 * 256 + 2 * R * ob + 2 * 128 * ob + 4) for _, _, n in fused_calls)
    ncalls = max(1, len(fused_calls))
    fused_per_loop = fused_bytes / reps
    # the roofline of the whole loop (pooling pass, 9 compression + reconstruction passes,
    # anchors, appends); the fused pass is the dominant entry point
    achieved = algo / ms / 1e6
    line["roofline"] = {"bound": "hbm", "scope": "step (the whole loop)", "achieved": achieved,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                        "traffic": None, "algorithmic_bytes": algo,
                        "dominant": {"entry_point": fused_name, "kernels": "project_kernel (fused reconstruction)",
                                     "ms": fused_ms / ncalls, "calls_per_loop": len(fused_calls) / reps,
                                     "frac": fused_bytes / fused_ms / 1e6 / HBM_PEAK_GBS,
                                     "algorithmic_share": fused_per_loop / algo}}
    line["ops"] = {fused_name: {"ms": fused_ms / ncalls, "algorithmic_bytes": fused_bytes / ncalls,
                                "GBs": fused_bytes / fused_ms / 1e6,
                                "frac": fused_bytes / fused_ms / 1e6 / HBM_PEAK_GBS,
                                "traffic": measured_traffic(fused_name, "config4"),
                                "mfma": {"flops_per_head_token": 81920 + 2 * 2 * 128 * R,
                                         "TFLOPs": sum(n for _, _, n in fused_calls) * (81920 + 4 * 128 * R)
                                         / fused_ms / 1e9}}}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = loop_cpu_baseline(inp, toks, S0, T, G, R)
    print(json.dumps(line), flush=True)


def loop_cpu_baseline(inp, toks, S0, T, G, R):
    """The oracle's loop on one slice (layer 0, kv head 0), pinned to one core: the
    pooled prefill update and pass, then the first decode update and pass (two
    passes over ~131K tokens).  Reported as oracle scorings/s; the time of the whole
    workload on one core is extrapolated from it."""
    import numpy as np
    import torch

    import oracle
    import synth
    grp = inp.Hq // inp.Hkv
    K = synth.bf16_bits(inp.K[0, :S0 + T])
    V = synth.bf16_bits(inp.V[0, :S0 + T])
    Qp = synth.bf16_bits(inp.Q[0, 0, :grp])
    Qd = synth.bf16_bits(torch.stack([q[0, 0, :grp] for _, _, q in toks[:T]]).to(torch.bfloat16))
    Uk, Uv = inp.Uk[0, 0].cpu().numpy(), inp.Uv[0, 0].cpu().numpy()

    def cpu(_budget):
        t0 = time.perf_counter()
        res = oracle.full_loop_slice(K, V, Qp, Qd, Uk, Uv, S0, T, T, 32, 1e-3)
        t = time.perf_counter() - t0
        return sum(st["S"] for st in res), t, ("layer 0 / kv head 0: the pooled prefill update and pass over "
                                               "%d tokens, then the first decode update and pass over %d" % (S0, S0 + T))

    rec = run_cpu_baseline(cpu, 0.0)
    rec["unit"] = "scorings/s"
    scorings = G * sum(S0 + T * j for j in range(9))
    rec["extrapolated_full_workload_s"] = scorings / rec["value"]
    rec["extrapolation"] = ("%d scorings (256 slices x 9 passes) at the sample's rate on one core; "
                            "not measured" % scorings)
    del np
    return rec


def base_line(args, metric, value, ms_step, steps, config):
    # the path takes bf16 K/V/Q and computes in fp32 (scores, centroids, low-rank outputs)
    return {"metric": metric, "value": value, "unit": "head-tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp32 (bf16 inputs)", "data": "synthetic",
            "config": config}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every slice is "
              "independent, so slices would shard across GPUs without communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from token_scoring_eviction_amd import kvc

    if args.copy_ref:
        return copy_reference(args.copy_ref, args.steps)
    kvc.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.config == 4 and not args.refine:
        return run_loop_config(args, dev)
    if args.refine:
        ops, head_tokens, algo, config, cpu = refine_workload(dev)
    elif args.config == 3:
        ops, head_tokens, algo, config, cpu = oja_workload(dev, args.storage)
    else:
        ops, head_tokens, algo, config, cpu = manifold_workload(args.config, dev, args.metric, args.budgets)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()
    # The timed region: the steps back to back, bracketed by two events on the stream the
    # kernels are launched on (torch's current stream, which the binding passes to libkvc).
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        for op in ops:
            op.fn()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    # The breakdown: the same steps again, every entry point bracketed by its own events
    # (a separate pass, because an event between two launches adds a few microseconds
    # to the step: 0.629 vs 0.611 ms at 256 x 16384)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(args.steps)]
    for i in range(args.steps):
        for op, (a, b) in zip(ops, ev[i]):
            a.record()
            op.fn()
            b.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        for op, (a, b) in zip(ops, ev[i]):
            op.ms.append(a.elapsed_time(b))
    workload = "refine" if args.refine else "config%d" % args.config
    per_op = {}
    for op in ops:
        ms = sum(op.ms) / len(op.ms)
        rec = {"ms": ms, "algorithmic_bytes": op.nbytes, "algorithmic_share": op.nbytes / algo,
               "GBs": op.nbytes / ms / 1e6, "frac": op.nbytes / ms / 1e6 / HBM_PEAK_GBS,
               "moved_bytes": op.moved, "moved_GBs": op.moved / ms / 1e6, "kernels": op.kernel,
               "traffic": measured_traffic(op.name, workload)}
        if op.flops:
            rec["mfma"] = {"flops": op.flops, "TFLOPs": op.flops / ms / 1e9,
                           "frac": op.flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}
        per_op[op.name] = rec
    dom = max(per_op, key=lambda n: per_op[n]["ms"])
    line = base_line(args, "KV head-tokens scored+compacted/s", head_tokens / (ms_step / 1e3),
                     ms_step, args.steps, config)
    # the roofline of the whole step: its algorithmic bytes over its time; the entry
    # point that takes longest is named with its kernels and its own fraction
    achieved = algo / ms_step / 1e6
    line["roofline"] = {"bound": "hbm", "scope": "step", "achieved": achieved, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": step_traffic(ops, workload),
                        "algorithmic_bytes": algo,
                        "dominant": {"entry_point": dom, "kernels": per_op[dom]["kernels"],
                                     "ms": per_op[dom]["ms"], "frac": per_op[dom]["frac"],
                                     "algorithmic_share": per_op[dom]["algorithmic_share"]}}
    mf = [r["mfma"] for r in per_op.values() if "mfma" in r]
    if mf:
        line["roofline"]["mfma"] = mf[0]
    line["ops"] = per_op
    # context for the fraction: what a plain 1 GiB device copy reaches on this GPU
    copy_ms, copy_gbs = time_device_copy(1024, 10)
    line["context"] = {"device_copy_GBs": copy_gbs, "device_copy_frac": copy_gbs / HBM_PEAK_GBS}
    if not args.no_cpu_baseline:
        rec = run_cpu_baseline(cpu, args.cpu_seconds)
        rec["extrapolated_full_workload_s"] = head_tokens / rec["value"]
        rec["extrapolation"] = "the whole workload at the sample's rate on one core; not measured"
        line["cpu_baseline"] = rec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
