"""Benchmark: one verification step of a LLaMA-7B-shaped attention layer on one
MI355X -- ancestor mask -> tree attention over a 4096-token prefix for a
64-node tree (32 heads, head dim 128, bf16) -> greedy acceptance over a
32000-token vocab -> KV compaction -- on seeded synthetic inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: verified tree tokens/s (tree nodes verified per second),
the per-call times, the attention kernel's roofline entry and the CPU oracle's
rate on a bounded sample.  Inputs are cycled over replicas totalling >= 1 GiB,
so the 256 MB Infinity Cache cannot serve them between steps.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, published
REPLICA_BYTES = 1 << 30        # cycle at least this much input per step round


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--traffic", default=None,
                    help="traffic summary (default profiles/attention_<workload>_traffic.md); "
                         "used only if it was taken from the current attention sources")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def algorithmic_attention_bytes(wl) -> int:
    """K and V rows of every request read once (prefix + tree keys), the
    queries read and the outputs written once."""
    s = wl.elem_bytes
    n = 0
    for b in range(wl.B):
        N = int(wl.node_off[b + 1] - wl.node_off[b])
        P = int(wl.prefix_len[b])
        n += (P + N) * wl.Hkv * wl.D * 2 * s + 2 * N * wl.Hq * wl.D * s
    return n


def algorithmic_attention_flops(wl) -> int:
    """Useful matrix work: every query row against the keys it attends (the
    request's prefix plus the node's root path), 2 flops per multiply-add in
    Q K^T and again in P V."""
    n = 0
    for b in range(wl.B):
        lo, hi = int(wl.node_off[b]), int(wl.node_off[b + 1])
        P = int(wl.prefix_len[b])
        depth = [0] * (hi - lo)
        for i in range(1, hi - lo):
            depth[i] = depth[int(wl.parent[lo + i])] + 1
        n += wl.Hq * ((hi - lo) * P + sum(depth) + (hi - lo)) * wl.D * 4
    return n


def cpu_baseline(wl, budget_s: float, stochastic: bool):
    """The oracle as it stands, timed on the host: full steps of the same
    workload, repeated until the time budget is used."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    W = (wl.max_nodes + 63) // 64
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.tree_mask(wl.node_off, wl.parent, W)
        oracle.tree_attention(wl.q, wl.k_cache, wl.v_cache, wl.dtype, wl.Hq, wl.Hkv, wl.node_off,
                              wl.parent, wl.prefix_len)
        if wl.V:
            if stochastic:
                res = oracle.verify_stochastic(wl.node_off, wl.parent, wl.tokens, wl.logits,
                                               wl.draft_logits, wl.V, wl.temperature,
                                               wl.rng_seed, wl.rng_offset, wl.max_depth)
            else:
                res = oracle.verify_greedy(wl.node_off, wl.parent, wl.tokens, wl.logits, wl.V,
                                           wl.max_depth)
            oracle.kv_compact(wl.k_cache, wl.v_cache, wl.prefix_len, res["accept_len"],
                              res["accept_nodes"], wl.max_depth + 1)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 1000:
            break
    per = el / runs
    return {"value": wl.T / per, "unit": "verified tree tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{runs} full oracle step(s) of the same workload "
            f"(mask, fp64 attention, acceptance, compaction) in {el:.1f} s; "
            f"{per * 1e3:.1f} ms per step", "seconds_per_step": per}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    from synth import make_workload
    from token_tree_verification_st_amd import load_library, to_device
    from token_tree_verification_st_amd import step as stp

    load_library()
    torch.cuda.set_device(0)
    wl = make_workload(args.workload, args.seed)
    stochastic = "stochastic" in wl.steps
    footprint = (wl.q.nbytes + wl.k_cache.nbytes + wl.v_cache.nbytes +
                 (0 if wl.logits is None else wl.logits.nbytes) +
                 (0 if wl.draft_logits is None else wl.draft_logits.nbytes))
    R = max(1, math.ceil(REPLICA_BYTES / footprint))
    reps = [to_device(wl) for _ in range(R)]
    print(f"# workload {wl.name}: T={wl.T} footprint {footprint / 1e6:.1f} MB, {R} replicas",
          file=sys.stderr, flush=True)

    calls = ["mask", "attention"] + (["verify", "compact"] if wl.V else [])
    fns = {"mask": stp.run_mask, "attention": stp.run_attention,
           "verify": lambda d: stp.run_verify(d, stochastic), "compact": stp.run_compact}

    for i in range(args.warmup):
        stp.verification_step(reps[i % R], stochastic=stochastic)
    torch.cuda.synchronize()

    # The K timed steps are captured into one HIP graph (replica i % R for step
    # i), so host launch cost does not pace the GPU; events on the stream
    # bracket its replay.  Each call is then timed the same way from a graph
    # of K back-to-back launches of that call alone (same replicas, same
    # stream), which gives its average launch duration.
    K = args.steps

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(reps[i % R])
        return g

    def timed_replay(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t, e0.elapsed_time(e1)

    step_fn = lambda d: stp.verification_step(d, stochastic=stochastic)
    if args.eager:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(K):
            step_fn(reps[i % R])
        e1.record()
        torch.cuda.synchronize()
        wall, gpu_span_ms = time.perf_counter() - t0, e0.elapsed_time(e1)
    else:
        g_step = capture(step_fn)
        wall, gpu_span_ms = timed_replay(g_step)
    ms_per_step = wall / K * 1e3
    per_call = {}
    for c in calls:
        _, ms = timed_replay(capture(fns[c]))
        per_call[c] = ms / K * 1e3  # us per launch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    st_words = [int(r.buf["status"].item()) for r in reps]
    assert not any(st_words), f"device status {st_words}"

    attn_bytes = algorithmic_attention_bytes(wl)
    attn_us = per_call["attention"]
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    from token_tree_verification_st_amd.profiling import read_traffic
    traffic = read_traffic(args.traffic or os.path.join(
        ROOT, "profiles", f"attention_{wl.name}_traffic.md"))
    attn_flops = algorithmic_attention_flops(wl)
    tflops = attn_flops / (attn_us * 1e-6) / 1e12
    peak_tf = MFMA_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    # the bound is whichever of the two ideal times is longer
    mfma_bound = attn_flops / (peak_tf * 1e12) > attn_bytes / (HBM_PEAK_GBS * 1e9)
    roof = {"bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(tflops if mfma_bound else achieved, 1),
            "peak": peak_tf if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / peak_tf if mfma_bound else achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "st_tree_attention", "algorithmic_bytes": attn_bytes,
            "algorithmic_flops": attn_flops, "hbm_gbs": round(achieved, 1),
            "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / peak_tf, 4),
            "avg_launch_us": round(attn_us, 3),
            "timing": f"HIP events around a graph of {K} back-to-back st_tree_attention calls"}
    al = reps[0].buf["accept_len"].cpu().numpy() if wl.V else np.zeros(wl.B)
    line = {
        "metric": "verified tree tokens/s (7B-shaped layer, 64-node tree, 4K prefix); % HBM peak",
        "value": round(wl.T / (ms_per_step * 1e-3), 1),
        "unit": "verified tree tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "gpu_ms_per_step": round(gpu_span_ms / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded PCG64, N(0,1) q/k/v, N(0,3) logits)",
        "config": {"workload": wl.name, "requests": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "prefix": [int(x) for x in wl.prefix_len][:8],
                   "tree_nodes": int(wl.T), "vocab": wl.V,
                   "acceptance": "stochastic" if stochastic else "greedy",
                   "replicas": R, "launch": "eager" if args.eager else "hip graph"},
        "per_call_us": {c: round(v, 3) for c, v in per_call.items()},
        "hbm_frac_step": round(attn_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "accepted_tokens_per_step": int((al + 1).sum()),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, stochastic)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
