"""Benchmark: scored+compressed KV tokens/s per layer on one MI355X.

One step is one pass of the whole path over one layer's cache already resident in HBM:
  sum configs (0, 1, 2, 4): kvc_row_lse -> kvc_score_tokens(SUM) -> kvc_channel_weights
                            -> kvc_allocate_bits(V tokens) -> kvc_allocate_bits(K channels)
                            -> kvc_quantize_pack
  max config (3):           kvc_row_lse -> kvc_score_tokens(MAX) -> kvc_allocate_bits(TOPK)
                            -> kvc_quantize_pack
The default workload is the largest single-GPU one: the decode-time 128k cache (32 query heads /
8 KV heads, d = 128, N = 131072 cached keys, the last Nq = 512 positions as query rows, causal,
bf16, 4 outlier K channels per KV head, 2 bits/element), whose 512 MiB of K and V do not fit the
Infinity Cache, so its pack and attend figures are HBM figures.
value = N / (mean step time over the timed steps).

Prints ONE JSON line.  `roofline` is for the dominant kernel (pass 1 of the scorer,
lse_partial), timed with HIP events recorded on the stream its call is enqueued on, inside
the timed region.  The fidelity attend is timed after the timed region and reported apart
(`attend`), together with a single-decode-row slice whose HBM traffic is the packed cache.
`cpu_baseline` times the float64 oracle on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]
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
CPU_SAMPLE_SECONDS = 12.0      # oracle sample: KV heads are added until this much CPU time

# HBM bytes per launch of the dominant kernel, from rocprofv3 FETCH_SIZE and WRITE_SIZE runs
# scaled by the same counters on a plain copy of known size (profiles/hbm_counters_*.md).
# A figure holds only for the scorer source it was measured on; otherwise traffic is null.
MEASURED_TRAFFIC = {
    "decode_cache_n131072_q512": {"bytes": 309878618,
                                  "score_src_sha256": "5fc095335bdb6081bf714a3488036e0375c138f3f88d532c6d0332666af39cbf"},
}


def visible_elements(N, Nq, causal=True):
    """Visible (query row, key) pairs of one query head, row i at position N - Nq + i."""
    if not causal:
        return N * Nq
    return Nq * (N - Nq) + Nq * (Nq + 1) // 2


def cpu_baseline(cfg):
    """The oracle as it stands, every step of the timed path, on whole KV heads (each with
    its G query heads and all rows) until about CPU_SAMPLE_SECONDS have passed; the layer
    time is the per-head time times H_kv."""
    import numpy as np
    import oracle
    from workloads import make_config_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:
        blas_threads = 0
    x = make_config_inputs(cfg)
    G = cfg.gqa
    heads = 0
    dt = 0.0
    for g in range(cfg.n_kv_heads):
        q1 = np.ascontiguousarray(x["q"][g * G:(g + 1) * G])
        k1 = np.ascontiguousarray(x["k"][g:g + 1])
        v1 = np.ascontiguousarray(x["v"][g:g + 1])
        t0 = time.perf_counter()
        lse = oracle.row_lse(q1, k1)
        if cfg.mode == "sum":
            w = oracle.token_scores_sum(q1, k1, lse)
            wc = oracle.channel_weights(q1, k1)
            bv, _ = oracle.allocate_v_tokens(w.astype(np.float32), cfg.avg_bits, cfg.head_dim)
            bk, _ = oracle.allocate_k_channels(wc.astype(np.float32), bv, cfg.avg_bits)
        else:
            w_o = x["w_o"][:, g * G * cfg.head_dim:(g + 1) * G * cfg.head_dim]
            s = oracle.token_scores_max(q1, k1, lse, x["hidden"], np.ascontiguousarray(w_o), v1)
            bv = oracle.topk_keep(s.astype(np.float32), cfg.keep_fraction, 16)
            bk = np.full((1, cfg.head_dim), 16, dtype=np.uint8)
        oracle.pack_cache(k1, v1, bv, bk)
        dt += time.perf_counter() - t0
        heads += 1
        if dt >= CPU_SAMPLE_SECONDS:
            break
    layer_s = dt / heads * cfg.n_kv_heads
    return {
        "value": round(cfg.n_keys / layer_s, 1), "unit": "tokens/s",
        "cores": max(1, blas_threads), "kind": "oracle",
        "sample": (f"{heads} of {cfg.n_kv_heads} KV heads of {cfg.name} (each: {G} query heads x "
                   f"{cfg.n_queries} rows x {cfg.n_keys} keys), every step of the timed path in "
                   f"float64 numpy, {dt:.2f} s; layer time = per-head time x {cfg.n_kv_heads}; "
                   f"BLAS threads {blas_threads}, host cpus {len(os.sched_getaffinity(0))}"),
    }


def measured_traffic(workload):
    import hashlib
    m = MEASURED_TRAFFIC.get(workload)
    if m is None:
        return None
    src = os.path.join(ROOT, "kv_cache_compression_pass_amd", "csrc", "score.hip")
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m["score_src_sha256"]:
            return None
    return m["bytes"]


def packed_bytes_read_by_attend(hdr):
    """Bytes of the packed cache one attend launch streams: value words and (scale, zero)
    pairs, key words and pairs, the retained-token list and its value locations."""
    return int(4 * hdr[5] + 8 * hdr[6] + 8 * hdr[7] + 4 * hdr[8] + 8 * hdr[9])


def pack_algorithmic_bytes(hdr, k_width, d):
    """Bytes kvc_quantize_pack must move: bf16 elements of retained V tokens and of retained
    tokens in K channels of nonzero width (read), codes, (scale, zero) pairs and the index
    lists (written).  Returns the K part (pack_k) and the V part (pack_v)."""
    hkv = int(hdr[0])
    k_read = 0
    for g in range(hkv):
        r_g = int(hdr[16 + 24 * g + 4])
        k_read += 2 * r_g * int((k_width[g] > 0).sum())
    v_read = 2 * d * int(hdr[4])
    v_write = 4 * int(hdr[5]) + 8 * int(hdr[6]) + 4 * int(hdr[4])
    k_write = 4 * int(hdr[8]) + 8 * int(hdr[9]) + 8 * int(hdr[7])
    return {"k": k_read + k_write, "v": v_read + v_write}


# KVSculpt's setting (Qwen2.5-1.5B-like layer, 2048-token context): 12 query heads, 2 KV heads,
# d = 128; the 512 most recent tokens are kept, the older 1536 are fitted by n_c = 768 pairs
# (ratio 0.5), with 1024 training query rows per query head that see every key.
RIDGE_SHAPE = {"n_q_heads": 12, "n_kv_heads": 2, "head_dim": 128, "n_compressed": 768, "n_retained": 512,
               "n_queries": 1024, "lambda": 1e-3}


def ridge_algorithmic_flops(hq, hkv, d, nc, m, nq):
    """Per call: logits 2 R n d, retained product 2 R m d, the normal matrix by symmetry
    R n_c (n_c + 1), its right side 2 R n_c d, Cholesky n_c^3 / 3, two solves 2 n_c^2 d (per KV
    head, R = G Nq stacked rows, n = n_c + m keys)."""
    R = (hq // hkv) * nq
    n = nc + m
    per = 2 * R * n * d + 2 * R * m * d + R * nc * (nc + 1) + 2 * R * nc * d + nc ** 3 / 3 + 2 * nc * nc * d
    return hkv * per


def ridge_figure(args, stream, dev):
    import numpy as np
    import torch
    import kv_cache_compression_pass_amd as kvc
    from workloads import make_inputs
    sh = RIDGE_SHAPE
    hq, hkv, d, nc, m, nq = (sh["n_q_heads"], sh["n_kv_heads"], sh["head_dim"], sh["n_compressed"],
                             sh["n_retained"], sh["n_queries"])
    x = make_inputs(hq, hkv, d, nc + m, nq, seed=4321)
    q = kvc.bf16_tensor(x["q"], dev)
    k = kvc.bf16_tensor(x["k"], dev)
    v_r = kvc.bf16_tensor(np.ascontiguousarray(x["v"][:, nc:]), dev)
    y = torch.randn(hq, nq, d, dtype=torch.float32, device=dev, generator=torch.Generator(device=dev).manual_seed(7))
    desc = kvc.make_desc(hq, hkv, d, nc + m, nq, False)
    ws = kvc.workspace(kvc.OP_RIDGE_FIT, desc, nc, dev)
    v_c = torch.empty(hkv, nc, d, dtype=torch.float32, device=dev)
    fn = lambda: kvc.kvc_ridge_value_fit(desc, nc, q, k, v_r, y, sh["lambda"], v_c, ws, stream=stream)
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    reps = max(min(args.steps, 20), 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = ridge_algorithmic_flops(hq, hkv, d, nc, m, nq)
    return {"shape": dict(sh), "ms": round(ms, 4), "flops": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "status": kvc.kvc_get_device_status(ws)}


def copy_rate(stream, dev, mib=512, reps=10):
    """The streaming rate this GPU sustains in the same run: a plain device copy of MIB MiB
    (reads MIB, writes MIB), median of REPS launches.  Context for the pack's HBM figure: the
    published 8 TB/s is a peak that no streaming kernel reaches."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    ms = ts[len(ts) // 2]
    del src, dst
    return 2.0 * 4 * n / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the bench: run a plain elementwise copy of MIB MiB (read MIB, "
                         "write MIB) five times, the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path runs "
              "on a single GPU (sharding by KV head or key range is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(5):
            torch.neg(src, out=dst)
        a1.record()
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / 5
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "ms": round(ms, 5), "gbs": round(8 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    import kv_cache_compression_pass_amd as kvc
    from workloads import get_config, make_config_inputs

    cfg = get_config(args.config)
    kvc.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    hq, hkv, d, N, Nq = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries
    x = make_config_inputs(cfg)
    q, k, v = (kvc.bf16_tensor(x[n], dev) for n in ("q", "k", "v"))
    hidden = w_o = None
    if cfg.mode == "max":
        hidden = kvc.bf16_tensor(x["hidden"], dev)
        w_o = kvc.bf16_tensor(x["w_o"], dev)
    del x
    desc = kvc.make_desc(hq, hkv, d, N, Nq, True)
    lse = torch.empty(hq, Nq, dtype=torch.float32, device=dev)
    w = torch.empty(hkv, N, dtype=torch.float32, device=dev)
    wc = torch.empty(hkv, d, dtype=torch.float32, device=dev)
    bv = torch.empty(hkv, N, dtype=torch.uint8, device=dev)
    bk = torch.empty(hkv, d, dtype=torch.uint8, device=dev)
    mode = kvc.SCORE_SUM if cfg.mode == "sum" else kvc.SCORE_MAX
    ws_l = kvc.workspace(kvc.OP_ROW_LSE, desc, 0, dev)
    ws_s = kvc.workspace(kvc.OP_SCORE_TOKENS, desc, mode, dev)
    ws_p = kvc.workspace(kvc.OP_QUANTIZE_PACK, desc, 0, dev)
    res_v = kvc.alloc_result_buffer(dev)
    res_k = kvc.alloc_result_buffer(dev)
    cache = kvc.PackedCache(desc, dev)
    stream = torch.cuda.current_stream()

    calls = [("row_lse", lambda: kvc.kvc_row_lse(desc, q, k, lse, ws_l, stream=stream))]
    if cfg.mode == "sum":
        ws_c = kvc.workspace(kvc.OP_CHANNEL_WEIGHTS, desc, 0, dev)
        ws_v = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_V_TOKENS, dev)
        ws_k = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_K_CHANNELS, dev)
        calls += [
            ("score_tokens", lambda: kvc.kvc_score_tokens(desc, mode, q, k, lse, w, ws_s, stream=stream)),
            ("channel_weights", lambda: kvc.kvc_channel_weights(desc, q, k, wc, ws_c, stream=stream)),
            ("allocate_v", lambda: kvc.kvc_allocate_bits(desc, kvc.ALLOC_V_TOKENS, w, bv, ws_v,
                                                         avg_bits=cfg.avg_bits, result=res_v, stream=stream)),
            ("allocate_k", lambda: kvc.kvc_allocate_bits(desc, kvc.ALLOC_K_CHANNELS, wc, bk, ws_k, bits_v=bv,
                                                         avg_bits=cfg.avg_bits, result=res_k, stream=stream)),
        ]
    else:
        ws_t = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_TOPK, dev)
        bk.fill_(16)
        calls += [
            ("score_tokens", lambda: kvc.kvc_score_tokens(desc, mode, q, k, lse, w, ws_s, hidden=hidden,
                                                          w_o=w_o, v=v, stream=stream)),
            ("allocate_topk", lambda: kvc.kvc_allocate_bits(desc, kvc.ALLOC_TOPK, w, bv, ws_t,
                                                            keep_fraction=cfg.keep_fraction, keep_bits=16,
                                                            result=res_v, stream=stream)),
        ]
    calls.append(("quantize_pack", lambda: kvc.kvc_quantize_pack(desc, k, v, bv, bk, cache, ws_p, stream=stream)))

    def step(events=None):
        for i, (_, fn) in enumerate(calls):
            if events is not None and events[i] is not None:
                events[i][0].record(stream)
            fn()
            if events is not None and events[i] is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps; events around the dominant call (row_lse) of every step
    ev_dom = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        step([ev_dom[s]] + [None] * (len(calls) - 1))
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    lse_ms = sum(a.elapsed_time(b) for a, b in ev_dom) / args.steps

    # per-call breakdown and per-step median over the same number of steps (not timed above)
    per_call = {name: [] for name, _ in calls}
    step_ms = []
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
        step(ev)
        torch.cuda.synchronize()
        for (name, _), (a, b) in zip(calls, ev):
            per_call[name].append(a.elapsed_time(b))
        step_ms.append(ev[0][0].elapsed_time(ev[-1][1]))

    hdr = cache.header()
    flops = 2.0 * d * visible_elements(N, Nq) * hq
    achieved = flops / (lse_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(cfg.name),
        "kernel": "lse_partial<128, 0>", "flops_per_launch": flops, "avg_launch_ms": round(lse_ms, 5),
    }

    # fidelity attend on the configuration's fidelity rows (the last rows of Q), and a
    # single-decode-row slice: one row per query head over the whole packed cache
    bv_h = bv.cpu().numpy()
    attend = {}
    for label, rows in (("fidelity", cfg.fidelity_rows), ("decode_row", 1)):
        rows = min(rows, Nq)
        desc_f = kvc.make_desc(hq, hkv, d, N, rows, True)
        q_f = q[:, Nq - rows:, :].contiguous()
        out_f = torch.empty(hq, rows, d, dtype=torch.float32, device=dev)
        lse_f = torch.empty(hq, rows, dtype=torch.float32, device=dev)
        ws_a = kvc.workspace(kvc.OP_COMPRESSED_ATTEND, desc_f, 0, dev)
        fn = lambda: kvc.kvc_compressed_attend(desc_f, q_f, cache, out_f, lse_f, ws_a, stream=stream)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        reps = max(args.steps, 10)
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / reps
        # retained keys visible to each row, per KV head: rows at positions N - rows + i
        ret = np.cumsum(bv_h > 0, axis=1)
        pos = np.arange(N - rows, N)
        vis = int(ret[:, pos].sum()) * (hq // hkv)
        a_flops = 4.0 * d * vis
        a_bytes = packed_bytes_read_by_attend(hdr) + 2 * q_f.numel() + 4 * (out_f.numel() + lse_f.numel())
        attend[label] = {"rows": rows, "ms": round(ms, 5),
                         "tflops": round(a_flops / (ms * 1e-3) / 1e12, 2),
                         "gbs": round(a_bytes / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(a_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "bytes": a_bytes, "flops": a_flops}

    # one decode row per query head over the packed cache plus an append buffer of 128 new
    # tokens (raw bf16; the last 128 keys and values stand in for them)
    n_new = min(128, N)
    kn = k[:, N - n_new:, :].contiguous()
    vn = v[:, N - n_new:, :].contiguous()
    desc_a = kvc.make_desc(hq, hkv, d, N, 1, True)
    q_a = q[:, Nq - 1:, :].contiguous()
    out_a = torch.empty(hq, 1, d, dtype=torch.float32, device=dev)
    lse_a = torch.empty(hq, 1, dtype=torch.float32, device=dev)
    ws_aa = kvc.workspace(kvc.OP_COMPRESSED_ATTEND, desc_a, 0, dev)
    afn = lambda: kvc.kvc_compressed_attend_append(desc_a, q_a, cache, kn, vn, out_a, lse_a, ws_aa, stream=stream)
    for _ in range(3):
        afn()
    torch.cuda.synchronize()
    reps = max(args.steps, 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        afn()
    e1.record(stream)
    torch.cuda.synchronize()
    ap_ms = e0.elapsed_time(e1) / reps
    ap_bytes = packed_bytes_read_by_attend(hdr) + 2 * kn.numel() * 2 + 2 * q_a.numel() + 4 * (out_a.numel() + lse_a.numel())
    attend["decode_row_append128"] = {"rows": 1, "n_new": n_new, "ms": round(ap_ms, 5),
                                      "gbs": round(ap_bytes / (ap_ms * 1e-3) / 1e9, 1),
                                      "hbm_frac": round(ap_bytes / (ap_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                      "bytes": ap_bytes}

    # threshold-and-window keep over this step's token scores (reported apart): the threshold is
    # the 75th percentile of the scores, the window the pages' 128 tokens
    w_h = w.cpu().numpy()
    thr = float(np.percentile(w_h[np.isfinite(w_h)], 75.0))
    bits_t = torch.empty(hkv, N, dtype=torch.uint8, device=dev)
    kept_t = torch.empty(hkv, dtype=torch.int64, device=dev)
    kfn = lambda: kvc.kvc_keep_threshold(desc, w, thr, bits_t, window=128, keep_bits=16, kept=kept_t,
                                         stream=stream)
    for _ in range(3):
        kfn()
    torch.cuda.synchronize()
    reps = max(args.steps, 10)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(reps):
        kfn()
    k1.record(stream)
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / reps
    k_bytes = 5 * hkv * N + 8 * hkv
    keep_thr = {"ms": round(k_ms, 5), "bytes": k_bytes, "gbs": round(k_bytes / (k_ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(k_bytes / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "kept_fraction": round(float(kept_t.sum().item()) / (hkv * N), 4)}

    ridge = ridge_figure(args, stream, dev)

    pb = pack_algorithmic_bytes(hdr, bk.cpu().numpy(), d)
    pack_ms = float(np.mean(per_call["quantize_pack"]))
    pack_gbs = (pb["k"] + pb["v"]) / (pack_ms * 1e-3) / 1e9
    copy_gbs = copy_rate(stream, dev)
    pack = {"ms": round(pack_ms, 5), "bytes_k": pb["k"], "bytes_v": pb["v"],
            "gbs": round(pack_gbs, 1),
            "hbm_frac": round(pack_gbs / PEAK_HBM_GBS, 4),
            "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(pack_gbs / copy_gbs, 4)}

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
                   "n_keys": N, "n_queries": Nq, "causal": True, "score": cfg.mode,
                   "avg_bits": cfg.avg_bits, "keep_fraction": cfg.keep_fraction},
        "roofline": roofline,
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "per_call_ms": {n: round(float(np.mean(t)), 5) for n, t in per_call.items()},
        "score_pass2_call_tflops": round(flops / (np.mean(per_call["score_tokens"]) * 1e-3) / 1e12, 2),
        "attend": attend,
        "pack": pack,
        "keep_threshold": keep_thr,
        "ridge_fit": ridge,
        "retained_tokens": int(hdr[7]),
    }
    if cfg.mode == "sum":
        av, ak = kvc.decode_alloc_result(res_v), kvc.decode_alloc_result(res_k)
        out["alloc"] = {"v_lambda": av["lam"], "v_used_bits": av["used"], "v_budget": av["budget"],
                        "k_lambda": ak["lam"], "k_used_bits": ak["used"], "k_budget": ak["budget"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
