"""Benchmark: scored+compressed KV tokens/s per layer on one MI355X.

One step is one pass of the whole path over one layer's cache already resident in HBM:
kvc_row_lse -> kvc_score_tokens(SUM) -> kvc_channel_weights -> kvc_allocate_bits(V tokens)
-> kvc_allocate_bits(K channels) -> kvc_quantize_pack.  The workload is the Llama-3-8B-like
prefill layer (32 query heads / 8 KV heads, d = 128, N = Nq = 8192, causal, bf16, 4 outlier
K channels per head, 3 bits/element).  value = N / (mean step time).

Prints ONE JSON line.  `roofline` is for the dominant kernel, timed with events on the stream
its call is enqueued on; `cpu_baseline` times the float64 oracle on a bounded sample on the
host cores.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scored+compressed KV tokens/s per layer; % bf16 MFMA peak & % HBM BW"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak (published)


def visible_elements(N, Nq, causal=True):
    if not causal:
        return N * Nq
    return Nq * (N - Nq) + Nq * (Nq + 1) // 2


def cpu_baseline(cfg_index):
    """The oracle as it stands on one KV head of the layer (its G query heads, all rows),
    every step of the path; the layer takes H_kv times as long."""
    import numpy as np
    import oracle
    from workloads import get_config, make_config_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:
        blas_threads = 0
    cfg = get_config(cfg_index)
    x = make_config_inputs(cfg)
    G = cfg.gqa
    q1 = np.ascontiguousarray(x["q"][:G])
    k1 = np.ascontiguousarray(x["k"][:1])
    v1 = np.ascontiguousarray(x["v"][:1])
    t0 = time.perf_counter()
    lse = oracle.row_lse(q1, k1)
    w = oracle.token_scores_sum(q1, k1, lse)
    wc = oracle.channel_weights(q1, k1)
    bv, _ = oracle.allocate_v_tokens(w.astype(np.float32), cfg.avg_bits, cfg.head_dim)
    bk, _ = oracle.allocate_k_channels(wc.astype(np.float32), bv, cfg.avg_bits)
    oracle.pack_cache(k1, v1, bv, bk)
    dt = time.perf_counter() - t0
    layer_s = dt * cfg.n_kv_heads
    cores = len(os.sched_getaffinity(0))
    return {
        "value": cfg.n_keys / layer_s, "unit": "tokens/s", "cores": cores,
        "blas_threads": blas_threads, "kind": "oracle",
        "sample": (f"1 of {cfg.n_kv_heads} KV heads ({G} query heads x {cfg.n_queries} rows x "
                   f"{cfg.n_keys} keys), all six steps, float64 numpy: {dt:.2f} s; layer time "
                   f"taken as {cfg.n_kv_heads} x sample"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this path runs on a single GPU; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kv_cache_compression_pass_amd as kvc
    from workloads import get_config, make_config_inputs

    cfg = get_config(args.config)
    if cfg.mode != "sum":
        print("bench.py times the sum-score path (configs 0, 1, 2, 4)", file=sys.stderr)
        sys.exit(2)
    kvc.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    hq, hkv, d, N, Nq = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries
    x = make_config_inputs(cfg)
    q, k, v = (kvc.bf16_tensor(x[n], dev) for n in ("q", "k", "v"))
    del x
    desc = kvc.make_desc(hq, hkv, d, N, Nq, True)
    lse = torch.empty(hq, Nq, dtype=torch.float32, device=dev)
    w = torch.empty(hkv, N, dtype=torch.float32, device=dev)
    wc = torch.empty(hkv, d, dtype=torch.float32, device=dev)
    bv = torch.empty(hkv, N, dtype=torch.uint8, device=dev)
    bk = torch.empty(hkv, d, dtype=torch.uint8, device=dev)
    ws_l = kvc.workspace(kvc.OP_ROW_LSE, desc, 0, dev)
    ws_s = kvc.workspace(kvc.OP_SCORE_TOKENS, desc, kvc.SCORE_SUM, dev)
    ws_c = kvc.workspace(kvc.OP_CHANNEL_WEIGHTS, desc, 0, dev)
    ws_v = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_V_TOKENS, dev)
    ws_k = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_K_CHANNELS, dev)
    ws_p = kvc.workspace(kvc.OP_QUANTIZE_PACK, desc, 0, dev)
    res_v = kvc.alloc_result_buffer(dev)
    res_k = kvc.alloc_result_buffer(dev)
    cache = kvc.PackedCache(desc, dev)
    stream = torch.cuda.current_stream()

    calls = [
        ("row_lse", lambda: kvc.kvc_row_lse(desc, q, k, lse, ws_l, stream=stream)),
        ("score_tokens", lambda: kvc.kvc_score_tokens(desc, kvc.SCORE_SUM, q, k, lse, w, ws_s, stream=stream)),
        ("channel_weights", lambda: kvc.kvc_channel_weights(desc, q, k, wc, ws_c, stream=stream)),
        ("allocate_v", lambda: kvc.kvc_allocate_bits(desc, kvc.ALLOC_V_TOKENS, w, bv, ws_v,
                                                     avg_bits=cfg.avg_bits, result=res_v, stream=stream)),
        ("allocate_k", lambda: kvc.kvc_allocate_bits(desc, kvc.ALLOC_K_CHANNELS, wc, bk, ws_k, bits_v=bv,
                                                     avg_bits=cfg.avg_bits, result=res_k, stream=stream)),
        ("quantize_pack", lambda: kvc.kvc_quantize_pack(desc, k, v, bv, bk, cache, ws_p, stream=stream)),
    ]

    def step(events=None):
        for i, (_, fn) in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: whole steps only
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # per-call durations over the same number of steps (events around each call's launches)
    per_call = {name: 0.0 for name, _ in calls}
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
        step(ev)
        torch.cuda.synchronize()
        for (name, _), (a, b) in zip(calls, ev):
            per_call[name] += a.elapsed_time(b) / args.steps

    alloc_v = kvc.decode_alloc_result(res_v)
    alloc_k = kvc.decode_alloc_result(res_k)
    hdr = cache.header()

    # dominant kernel: pass 1.  For this workload (1024 head x row-tile blocks) kvc_row_lse
    # is a single launch of lse_partial, so events around the call time that kernel.
    flops = 2.0 * d * visible_elements(N, Nq) * hq
    lse_ms = per_call["row_lse"]
    achieved = flops / (lse_ms * 1e-3) / 1e12
    roofline = {
        "kernel": "lse_partial", "bound": "mfma", "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": None,
        "flops_per_launch": flops, "avg_launch_ms": round(lse_ms, 5),
    }
    score_flops = flops
    out = {
        "metric": METRIC,
        "value": round(N / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_q_heads": hq, "n_kv_heads": hkv, "head_dim": d,
                   "n_keys": N, "n_queries": Nq, "causal": True, "avg_bits": cfg.avg_bits},
        "roofline": roofline,
        "per_call_ms": {n: round(t, 5) for n, t in per_call.items()},
        "score_pass2_call_tflops": round(score_flops / (per_call["score_tokens"] * 1e-3) / 1e12, 2),
        "alloc": {"v_lambda": alloc_v["lam"], "v_used_bits": alloc_v["used"], "v_budget": alloc_v["budget"],
                  "k_lambda": alloc_k["lam"], "k_used_bits": alloc_k["used"], "k_budget": alloc_k["budget"],
                  "retained_tokens": int(hdr[7])},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
