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
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="stochastic workloads: nucleus sampling on target and draft")
    ap.add_argument("--draft-probs", action="store_true",
                    help="stochastic workloads: pass the draft as probabilities")
    ap.add_argument("--traffic", default=None,
                    help="traffic summary (default profiles/attention_<workload>_traffic.md); "
                         "used only if it was taken from the current attention sources")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="also time st_tree_attention_paged with this block size")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--only", default=None, choices=("attention", "verify", "step"),
                    help="for counter runs: launch only this call (warm-up, then a graph of "
                         "--steps calls), print its per-call time and exit")
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


def cpu_baseline_layer(host, cfg, wl, budget_s: float):
    """The oracle's layer step (fp64 model layer, greedy acceptance,
    compaction) on the host, repeated until the time budget is used."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    from oracle.attention import decode_values
    kc = decode_values(wl.k_cache, "bf16")
    vc = decode_values(wl.v_cache, "bf16")
    runs, t0 = 0, time.perf_counter()
    while True:
        out = oracle.tree_layer(host, cfg, wl.tokens, wl.node_off, wl.parent, wl.prefix_len,
                                kc, vc)
        res = oracle.verify_greedy(wl.node_off, wl.parent, wl.tokens, out["logits"], cfg["V"],
                                   wl.max_depth)
        oracle.kv_compact(out["k_cache"], out["v_cache"], wl.prefix_len, res["accept_len"],
                          res["accept_nodes"], wl.max_depth + 1)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 100:
            break
    per = el / runs
    return {"value": wl.T / per, "unit": "verified tree tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{runs} full oracle layer step(s) of the same workload "
            f"(fp64 projections, rotary, attention, acceptance, compaction) in {el:.1f} s; "
            f"{per * 1e3:.1f} ms per step", "seconds_per_step": per}


def bench_layer(args):
    """One model layer verifying the llama7b tree: embedding, q/k/v projection,
    rotary + append, tree attention, output projection with residual,
    vocabulary projection, greedy acceptance, compaction (d = 4096, 32/32
    heads, D = 128, V = 32000, prefix 4096, 64 nodes)."""
    import numpy as np
    import torch

    from synth import make_workload, model_config, model_weights
    from token_tree_verification_st_amd import Tree, load_library
    from token_tree_verification_st_amd.layer import (LayerWeights, layer_buffers, layer_step)
    from token_tree_verification_st_amd.binding import (st_embed, st_linear,
                                                        st_tree_attention, st_tree_rope_append,
                                                        st_verify_greedy, st_kv_compact)

    load_library()
    torch.cuda.set_device(0)
    wl = make_workload("llama7b", args.seed)
    cfg = model_config(V=wl.V, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D)
    wb = model_weights(args.seed, cfg)
    w_bytes = sum(v.nbytes for k, v in wb.items() if k != "E")

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()

    RW = 2                        # weight replicas: 2 x 396 MB cycles past the Infinity Cache
    ws = [LayerWeights(E=dev(wb["E"]), Wqkv=dev(wb["Wqkv"]), Wo=dev(wb["Wo"]),
                       Wlm=dev(wb["Wlm"]), Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"])
          for _ in range(RW)]
    kv_bytes = wl.k_cache.nbytes + wl.v_cache.nbytes
    R = max(RW, math.ceil(REPLICA_BYTES / kv_bytes))
    tree = Tree(torch.from_numpy(wl.node_off).cuda(), torch.from_numpy(wl.parent).cuda(),
                wl.max_nodes, wl.max_depth)
    tokens = torch.from_numpy(wl.tokens).cuda()
    prefix = torch.from_numpy(wl.prefix_len).cuda()
    P = int(wl.prefix_len.max())
    caches = [(dev(wl.k_cache), dev(wl.v_cache)) for _ in range(R)]
    bufs = [layer_buffers(ws[0], tree, P) for _ in range(R)]
    print(f"# workload llama7b_layer: T={wl.T} weights {w_bytes / 1e6:.0f} MB x {RW}, "
          f"kv {kv_bytes / 1e6:.1f} MB x {R}", file=sys.stderr, flush=True)

    def step(i):
        kc, vc = caches[i % R]
        layer_step(ws[i % RW], tree, tokens, prefix, P, kc, vc, bufs[i % R])

    T, d, V = wl.T, cfg["d"], cfg["V"]
    HD, QKV = cfg["Hq"] * cfg["D"], (cfg["Hq"] + 2 * cfg["Hkv"]) * cfg["D"]
    calls = {
        "embed": lambda i: st_embed(tokens, ws[i % RW].E, bufs[i % R].buf["x"],
                                    bufs[i % R].buf["status"]),
        "qkv_proj": lambda i: st_linear(bufs[i % R].buf["x"], ws[i % RW].Wqkv,
                                        bufs[i % R].buf["qkv"], workspace=bufs[i % R].buf["ws_qkv"]),
        "rope_append": lambda i: st_tree_rope_append(
            tree, bufs[i % R].buf["qkv"], cfg["Hq"], cfg["Hkv"], prefix, P, bufs[i % R].buf["q"],
            caches[i % R][0], caches[i % R][1], status=bufs[i % R].buf["status"]),
        "attention": lambda i: st_tree_attention(
            tree, bufs[i % R].buf["q"], caches[i % R][0], caches[i % R][1], prefix, P, None,
            bufs[i % R].buf["attn"], None, bufs[i % R].buf["ws_attn"],
            status=bufs[i % R].buf["status"]),
        "o_proj": lambda i: st_linear(bufs[i % R].buf["attn"].view(T, HD), ws[i % RW].Wo,
                                      bufs[i % R].buf["h"], residual=bufs[i % R].buf["x"],
                                      workspace=bufs[i % R].buf["ws_o"]),
        "lm_head": lambda i: st_linear(bufs[i % R].buf["h"], ws[i % RW].Wlm,
                                       bufs[i % R].buf["logits"],
                                       workspace=bufs[i % R].buf["ws_lm"]),
        "verify": lambda i: st_verify_greedy(
            tree, tokens, bufs[i % R].buf["logits"], bufs[i % R].buf["accept_len"],
            bufs[i % R].buf["accept_nodes"], bufs[i % R].buf["out_tokens"],
            bufs[i % R].buf["ws_verify"], bufs[i % R].buf["status"]),
        "compact": lambda i: st_kv_compact(
            caches[i % R][0], caches[i % R][1], prefix, bufs[i % R].buf["accept_len"],
            bufs[i % R].buf["accept_nodes"], bufs[i % R].buf["src_slot"],
            bufs[i % R].buf["new_len"], bufs[i % R].buf["status"]),
    }
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                fn(i)
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

    wall, gpu_ms = timed_replay(capture(step))
    ms_per_step = wall / K * 1e3
    per_call = {}
    for name, fn in calls.items():
        _, ms = timed_replay(capture(fn))
        per_call[name] = ms / K * 1e3
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    st_words = [int(b.buf["status"].item()) for b in bufs]
    assert not any(st_words), f"device status {st_words}"

    lm_bytes = V * d * 2 + T * d * 2 + T * V * 4
    lm_us = per_call["lm_head"]
    achieved = lm_bytes / (lm_us * 1e-6) / 1e9
    proj_bytes = (QKV * d + d * HD + V * d) * 2
    proj_us = per_call["qkv_proj"] + per_call["o_proj"] + per_call["lm_head"]
    from token_tree_verification_st_amd.profiling import read_linear_traffic
    traffic = read_linear_traffic(os.path.join(ROOT, "profiles",
                                               "linear_llama7b_layer_traffic.md"))
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "st_linear (vocabulary projection, 32000 x 4096)",
            "algorithmic_bytes": lm_bytes, "avg_launch_us": round(lm_us, 3),
            "projections_gbs": round(proj_bytes / (proj_us * 1e-6) / 1e9, 1),
            "timing": f"HIP events around a graph of {K} back-to-back calls"}
    al = bufs[0].buf["accept_len"].cpu().numpy()
    line = {
        "metric": "verified tree tokens/s (7B-shaped layer step with projections, 64-node tree, "
                  "4K prefix)",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "verified tree tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "gpu_ms_per_step": round(gpu_ms / K, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded PCG64: bf16 weights N(0, 1/d), N(0,1) prefix K/V)",
        "config": {"workload": "llama7b_layer", "requests": 1, "d_model": d,
                   "q_heads": cfg["Hq"], "kv_heads": cfg["Hkv"], "head_dim": cfg["D"],
                   "prefix": [P], "tree_nodes": T, "vocab": V, "acceptance": "greedy",
                   "weight_replicas": RW, "kv_replicas": R, "launch": "hip graph"},
        "per_call_us": {c: round(v, 3) for c, v in per_call.items()},
        "accepted_tokens_per_step": int((al + 1).sum()),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle.attention import decode_values
        host = {k: (decode_values(v, "bf16") if k != "E" else None) for k, v in wb.items()}
        # the oracle gathers embedding rows; decode only the rows it reads
        E = np.zeros((V, d))
        rows = np.unique(wl.tokens)
        E[rows] = decode_values(wb["E"][rows], "bf16")
        host["E"] = E
        line["cpu_baseline"] = cpu_baseline_layer(host, cfg, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def bench_tree_build(args):
    """Token-tree construction: 16 requests, 16 candidate continuations of up
    to 8 tokens each (shared prefixes of random length), vocab 32000, trees of
    at most 128 nodes, merged and packed into the st_tree layout per call."""
    import numpy as np
    import torch

    from synth import TREE_BUILD_CASE, make_candidates
    from token_tree_verification_st_amd import load_library, st_tree_build

    load_library()
    torch.cuda.set_device(0)
    c = TREE_BUILD_CASE
    B, K, Lmax, V, cap = c["B"], c["K"], c["Lmax"], c["V"], c["cap"]
    R = 64   # input and output replicas, cycled (they are small; this spreads the launches)
    cands = [make_candidates(args.seed + r, B, K, Lmax, V) for r in range(R)]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    ins = [tuple(dev(a) for a in cd) for cd in cands]
    outs = [{k: torch.empty(n, dtype=torch.int32, device="cuda") for k, n in
             (("n_nodes", B), ("parent", B * cap), ("tokens", B * cap), ("depth", B * cap),
              ("node_off", B + 1), ("parent_packed", B * cap), ("tokens_packed", B * cap),
              ("status", 1))} for _ in range(R)]

    def call(i):
        root, seqs, lens = ins[i % R]
        o = outs[i % R]
        st_tree_build(root, seqs, lens, V, cap, o["n_nodes"], o["parent"], o["tokens"],
                      o["depth"], node_off=o["node_off"], parent_packed=o["parent_packed"],
                      tokens_packed=o["tokens_packed"], status=o["status"])

    for o in outs:
        o["status"].zero_()
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    Ks = args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(Ks):
            call(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    us = e0.elapsed_time(e1) / Ks * 1e3
    assert not any(int(o["status"].item()) for o in outs), "device status set"
    nodes = int(outs[0]["node_off"][B].item())
    in_bytes = (B * K * Lmax + B * K + B) * 4
    out_bytes = (B * cap * 3 + B + (B + 1) + 2 * nodes) * 4
    gbs = (in_bytes + out_bytes) / (us * 1e-6) / 1e9
    line = {
        "metric": "token trees built per second (16 requests x 16 candidates x 8 tokens)",
        "value": round(B / (wall / Ks), 1), "unit": "trees/s", "n_gpus": 1, "steps": Ks,
        "warmup": args.warmup, "ms_per_step": round(wall / Ks * 1e3, 5),
        "gpu_ms_per_step": round(us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32",
        "data": "synthetic (seeded PCG64 candidates with shared prefixes of random length)",
        "config": {"workload": "tree_build", **c, "nodes_first_replica": nodes,
                   "launch": "hip graph"},
        "per_call_us": {"tree_build": round(us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                     "kernel": "st_tree_build (latency-bound: two launches, a few barriers "
                               "per level)", "algorithmic_bytes": in_bytes + out_bytes,
                     "avg_launch_us": round(us, 3),
                     "timing": f"HIP events around a graph of {Ks} back-to-back calls"},
    }
    if not args.no_cpu_baseline:
        import oracle
        runs, t0 = 0, time.perf_counter()
        while True:
            root, seqs, lens = cands[runs % R]
            r = oracle.build_tree(root, seqs, lens, V, cap)
            oracle.pack_trees(r["n_nodes"], r["parent"], r["tokens"])
            runs += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0) or runs >= 10000:
                break
        line["cpu_baseline"] = {"value": round(B * runs / el, 1), "unit": "trees/s", "cores": 1,
                                "kind": "oracle", "sample": f"{runs} oracle merges of the same "
                                f"case (pure Python, one thread) in {el:.1f} s"}
    print(json.dumps(line), flush=True)


def only(args, reps, R, fns, one_step):
    """One call alone, for counter runs: warm-up, a graph of K launches (events
    around its replay), then the calibration copy; every dispatch of the
    call's kernels in the process is one of these."""
    import torch
    fn = one_step if args.only == "step" else fns[args.only]
    for i in range(args.warmup):
        fn(reps[i % R])
    torch.cuda.synchronize()
    K = args.steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            fn(reps[i % R])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    st_words = [int(r.buf["status"].item()) for r in reps]
    assert not any(st_words), f"device status {st_words}"
    print(json.dumps({"only": args.only, "workload": args.workload, "calls": K,
                      "us_per_call": round(e0.elapsed_time(e1) / K * 1e3, 3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the verification path runs on one GPU (no sharding across GPUs); --gpus must be 1"}))
        sys.exit(2)
    if args.workload == "llama7b_layer":
        bench_layer(args)
        return
    if args.workload == "tree_build":
        bench_tree_build(args)
        return
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
    ext = stochastic and (args.top_p < 1.0 or args.draft_probs)
    if ext and args.draft_probs:
        z = wl.draft_logits.astype(np.float64) / wl.temperature
        pr = np.exp(z - z.max(axis=1, keepdims=True))
        pr = (pr / pr.sum(axis=1, keepdims=True)).astype(np.float32)
        for d in reps:
            d.buf["draft_probs"] = torch.from_numpy(pr).cuda()

    def verify(d):
        if ext:
            stp.run_verify(d, True, top_p=args.top_p, draft=d.buf.get("draft_probs"))
        else:
            stp.run_verify(d, stochastic)

    fns = {"mask": stp.run_mask, "attention": stp.run_attention, "verify": verify,
           "compact": stp.run_compact}

    def one_step(d):
        if ext:
            stp.verification_step(d, stochastic=True, top_p=args.top_p,
                                  draft=d.buf.get("draft_probs"))
        else:
            stp.verification_step(d, stochastic=stochastic)

    if args.only:
        only(args, reps, R, fns, one_step)
        return

    for i in range(args.warmup):
        one_step(reps[i % R])
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

    step_fn = one_step
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
    spread = {}
    if not args.eager:
        # four more replays of the same graph: the spread of the per-step time
        reps_ms = [gpu_span_ms / K] + [timed_replay(g_step)[1] / K for _ in range(4)]
        q = np.percentile(reps_ms, [10, 50, 90])
        spread = {"replays": len(reps_ms), "p10_us": round(q[0] * 1e3, 3),
                  "p50_us": round(q[1] * 1e3, 3), "p90_us": round(q[2] * 1e3, 3)}
    # one step after a 1 GiB write has pushed every input out of the caches,
    # events around that step only (median of 5)
    flush = torch.empty(REPLICA_BYTES // 4, dtype=torch.float32, device="cuda")
    single = []
    for i in range(5):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step_fn(reps[i % R])
        e1.record()
        torch.cuda.synchronize()
        single.append(e0.elapsed_time(e1) * 1e3)
    del flush
    per_call = {}
    for c in calls:
        _, ms = timed_replay(capture(fns[c]))
        per_call[c] = ms / K * 1e3  # us per launch
    if args.paged:
        # the same attention over a paged pool (blocks scattered by a seeded
        # permutation), one pool per replica
        from synth import make_paged
        from token_tree_verification_st_amd import st_tree_attention_paged

        def dev16(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
            return torch.from_numpy(a).cuda()

        kp_h, vp_h, bt_h = make_paged(args.seed, wl.k_cache, wl.v_cache, args.paged)
        pools = [(dev16(kp_h), dev16(vp_h)) for _ in range(R)]
        bt = torch.from_numpy(bt_h).cuda()

        def paged_call(d, i=[0]):
            kp, vp = pools[i[0] % R]
            i[0] += 1
            st_tree_attention_paged(d.tree, d.q, kp, vp, bt, d.prefix_len, d.max_prefix,
                                    d.buf["mask"], d.buf["out"], d.buf["lse"], d.buf["attn_ws"],
                                    status=d.buf["status"])

        _, ms = timed_replay(capture(paged_call))
        per_call["attention_paged"] = ms / K * 1e3
        del pools
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
    # practical ceiling: a plain read-only pass over as many bytes as the
    # attention's algorithmic traffic, cycled over cold buffers
    from token_tree_verification_st_amd import st_stream_read
    nbuf = max(2, math.ceil(REPLICA_BYTES / attn_bytes))
    bufs = [torch.ones(attn_bytes // 4, dtype=torch.int32, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for i in range(3):
        st_stream_read(bufs[i % nbuf], sink)
    g_read = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_read):
        for i in range(K):
            st_stream_read(bufs[i % nbuf], sink)
    _, ms = timed_replay(g_read)
    ceiling_us = ms / K * 1e3
    del g_read, bufs
    attn_us = per_call["attention"]
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    from token_tree_verification_st_amd.profiling import read_traffic
    traffic_md = args.traffic or os.path.join(ROOT, "profiles", f"attention_{wl.name}_traffic.md")
    traffic = read_traffic(traffic_md)
    traffic_partials = read_traffic(traffic_md, "split_partial_bytes")
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
            "traffic": traffic, "traffic_split_partials": traffic_partials,
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
                   **({"top_p": args.top_p, "draft": "probabilities" if args.draft_probs
                       else "logits"} if ext else {}),
                   "replicas": R, "launch": "eager" if args.eager else "hip graph",
                   **({"paged_block": args.paged} if args.paged else {})},
        "per_call_us": {c: round(v, 3) for c, v in per_call.items()},
        "hbm_frac_step": round(attn_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_spread": spread,
        "stream_ceiling": {"kernel": "st_stream_read (read-only)", "bytes": attn_bytes,
                           "us": round(ceiling_us, 3),
                           "gbs": round(attn_bytes / (ceiling_us * 1e-6) / 1e9, 1)},
        "single_step_us_after_flush": round(float(np.median(single)), 3),
        "accepted_tokens_per_step": int((al + 1).sum()),
        "roofline": roof,
    }
    if stochastic:
        # comparisons on the taken paths within 1e-6 of the acceptance bound (and
        # replacement draws within 1e-6 of a bin edge), summed over requests
        line["near_ties_per_step"] = int(reps[0].buf["near_ties"].sum().item())
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, stochastic)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
