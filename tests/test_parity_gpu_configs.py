"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark
times.  Where the float64 oracle cannot redo the whole layer in seconds, it checks outputs it
can compute exactly on their own (sampled rows; the last key columns, which only the last
rows see; one KV head) plus properties that hold at any size (every attention row sums to
one, so sum_t w[g,t] = G * Nq)."""

import math

import numpy as np
import pytest
import torch

import kv_cache_compression_pass_amd as kvc
import oracle
from workloads import get_config, make_config_inputs
from tests import gpu_helpers as H
from tests import oracle_blocks as OB

pytestmark = pytest.mark.gpu

TAIL = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    kvc.load()


def _sampled_rows(x, cfg, lse_g, rng, n=12):
    """Oracle LSE of single rows: row i only depends on q_i and the keys up to its position."""
    N, Nq, G = cfg.n_keys, cfg.n_queries, cfg.gqa
    picks = [(0, 0), (cfg.n_q_heads - 1, Nq - 1)]
    picks += [(int(rng.integers(cfg.n_q_heads)), int(rng.integers(Nq))) for _ in range(n)]
    for h, i in picks:
        p = N - Nq + i
        ref = oracle.row_lse(x["q"][h:h + 1, i:i + 1], x["k"][h // G:h // G + 1, :p + 1])[0, 0]
        assert abs(float(lse_g[h, i]) - ref) <= 1e-4, (h, i, float(lse_g[h, i]), ref)


def _tail_scores(x, cfg):
    """Exact oracle w[:, t] for the last TAIL keys: only the last TAIL rows see them."""
    Nq = cfg.n_queries
    r0 = Nq - TAIL
    q_sub = np.ascontiguousarray(x["q"][:, r0:, :])
    lse_sub = oracle.row_lse(q_sub, x["k"])
    w_sub = oracle.token_scores_sum(q_sub, x["k"], lse_sub)
    return w_sub[:, -TAIL:]


def _synthetic_weights(shape, total_per_head, seed):
    """Seeded heavy-tailed positive weights normalised like attention column sums."""
    rng = np.random.default_rng(seed)
    w = np.exp(rng.normal(0.0, 1.5, shape))
    w *= total_per_head / w.sum(axis=1, keepdims=True)
    return w.astype(np.float32)


@pytest.mark.parametrize("ci", [1, 2, 4])
def test_sum_config_full_size(ci):
    cfg = get_config(ci)
    print(f"config {ci} ({cfg.name}): inputs", flush=True)
    x = make_config_inputs(cfg)
    hq, hkv, d, N, Nq = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    rng = np.random.default_rng(ci)

    print(f"config {ci}: row_lse + scores", flush=True)
    lse_t = H.row_lse(desc, q, k)
    lse_g = lse_t.cpu().numpy()
    _sampled_rows(x, cfg, lse_g, rng)
    w_g = H.score_sum(desc, q, k, lse_t).cpu().numpy()
    np.testing.assert_allclose(w_g.astype(np.float64).sum(axis=1), cfg.gqa * Nq, rtol=2e-5)
    H.assert_rel(w_g[:, -TAIL:], _tail_scores(x, cfg), 1e-3, what="tail token scores")
    # whole KV heads: the LSE of every row of their query heads and every score column, so the
    # many-partial column reduction the full-size launch takes is compared element by element
    G = cfg.gqa
    for g in ((0, hkv - 1) if ci == 1 else (0,)):
        print(f"config {ci}: whole KV head {g} against the oracle", flush=True)
        heads = list(range(g * G, (g + 1) * G))
        lse_r = OB.head_lse(x["q"], x["k"], heads)
        H.assert_abs(lse_g[heads], lse_r, 1e-4, f"row LSE of KV head {g}'s query heads")
        w_r = OB.group_scores_sum(x["q"], x["k"], lse_r, g)
        H.assert_rel(w_g[g], w_r, 1e-3, what=f"token scores of KV head {g}")

    print(f"config {ci}: channel weights", flush=True)
    wc_g = H.channel_weights(desc, q, k).cpu().numpy()
    H.assert_rel(wc_g, oracle.channel_weights(x["q"], x["k"]), 1e-5, what="channel weights")

    print(f"config {ci}: allocation", flush=True)
    w32 = _synthetic_weights((hkv, N), cfg.gqa * Nq, seed=100 + ci)
    bv_g, res, st = H.allocate(desc, kvc.ALLOC_V_TOKENS, H.dev_f32(w32), cfg.avg_bits)
    bv_r, info = oracle.allocate_v_tokens(w32, cfg.avg_bits, d)
    np.testing.assert_array_equal(bv_g.cpu().numpy(), bv_r)
    assert res["lam"] == info["lam"] and res["used"] == info["used"] and res["budget"] == info["budget"]
    wc32 = oracle.channel_weights(x["q"], x["k"]).astype(np.float32)
    bk_g, resk, st = H.allocate(desc, kvc.ALLOC_K_CHANNELS, H.dev_f32(wc32), cfg.avg_bits,
                                bits_v=H.dev_u8(bv_r))
    bk_r, infok = oracle.allocate_k_channels(wc32, bv_r, cfg.avg_bits)
    np.testing.assert_array_equal(bk_g.cpu().numpy(), bk_r)
    assert resk["lam"] == infok["lam"] and resk["used"] == infok["used"]

    print(f"config {ci}: pack", flush=True)
    cache, st = H.pack(desc, k, v, H.dev_u8(bv_r), H.dev_u8(bk_r))
    assert st == 0
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], bv_r, bk_r))

    print(f"config {ci}: attend", flush=True)
    nf = cfg.fidelity_rows
    heads = slice(0, cfg.gqa)          # oracle on KV head 0's query heads
    qf = np.ascontiguousarray(x["q"][:, Nq - nf:, :])
    desc_f = H.desc_of(hq, hkv, d, N, nf, True)
    out_g, lh_g, st = H.attend(desc_f, H.dev_bf16(qf), cache)
    assert st == 0
    out_r, lh_r = oracle.compressed_attend(qf[heads], x["k"][:1], x["v"][:1], bv_r[:1], bk_r[:1])
    ty, tl = H.attend_tols(qf[heads], [x["k"][:1]], [x["v"][:1]], lh_r)
    H.assert_abs(out_g.cpu().numpy()[heads], out_r, ty, "attend output")
    H.assert_abs(lh_g.cpu().numpy()[heads], lh_r, tl, "attend lse")


def test_config3_kvzip_full_size():
    cfg = get_config(3)
    print("config 3: inputs", flush=True)
    x = make_config_inputs(cfg)
    hq, hkv, d, N, Nq = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    print("config 3: row_lse + max scores", flush=True)
    lse_t = H.row_lse(desc, q, k)
    _sampled_rows(x, cfg, lse_t.cpu().numpy(), np.random.default_rng(3))
    s_g = H.score_max(desc, q, k, lse_t, H.dev_bf16(x["hidden"]), H.dev_bf16(x["w_o"]), v).cpu().numpy()
    r0 = Nq - TAIL
    q_sub = np.ascontiguousarray(x["q"][:, r0:, :])
    lse_sub = oracle.row_lse(q_sub, x["k"])
    cols = np.arange(N - TAIL, N)
    s_r = oracle.token_scores_max(q_sub, x["k"], lse_sub, x["hidden"][r0:], x["w_o"], x["v"], tokens=cols)
    H.assert_rel(s_g[:, -TAIL:], s_r, 1e-3, what="tail KVzip+ scores")
    assert np.isfinite(s_g).all() and (s_g > 0).all()
    g = hkv - 1
    print(f"config 3: whole KV head {g} against the oracle", flush=True)
    heads = list(range(g * cfg.gqa, (g + 1) * cfg.gqa))
    lse_r = OB.head_lse(x["q"], x["k"], heads)
    H.assert_abs(lse_t.cpu().numpy()[heads], lse_r, 1e-4, f"row LSE of KV head {g}'s query heads")
    s_head = OB.group_scores_max(x["q"], x["k"], lse_r, x["hidden"], x["w_o"], x["v"], g)
    H.assert_rel(s_g[g], s_head, 1e-3, what=f"KVzip+ scores of KV head {g}")
    print("config 3: top-k + pack", flush=True)
    s32 = _synthetic_weights((hkv, N), 1.0, seed=303)
    kk = math.floor(cfg.keep_fraction * N)
    for g in range(hkv):                   # plant ties straddling each head's threshold
        thr = np.sort(s32[g])[::-1][kk - 1]
        s32[g, 50 + 97 * np.arange(40)] = thr
    b_g, res, st = H.allocate(desc, kvc.ALLOC_TOPK, H.dev_f32(s32), keep_fraction=cfg.keep_fraction)
    b_r = oracle.topk_keep(s32, cfg.keep_fraction, 16)
    np.testing.assert_array_equal(b_g.cpu().numpy(), b_r)
    bk = np.full((hkv, d), 16, np.uint8)
    cache, st = H.pack(desc, k, v, H.dev_u8(b_r), H.dev_u8(bk))
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], b_r, bk))


def test_ridge_fit_at_the_bench_shape():
    """The ridge value fit at the shape bench.py times (KVSculpt's layer: 12/2 heads, 768 pairs, 512
    retained tokens, 1024 training rows), against the oracle's exact solve within the elementwise
    bounds derived from the GPU's operand precisions."""
    import bench
    sh = bench.RIDGE_SHAPE
    hq, hkv, d, nc, m, nq, lam = (sh["n_q_heads"], sh["n_kv_heads"], sh["head_dim"], sh["n_compressed"],
                                  sh["n_retained"], sh["n_queries"], sh["lambda"])
    print(f"case ridge bench shape: H_q={hq} H_kv={hkv} d={d} n_c={nc} m={m} Nq={nq} lambda={lam}", flush=True)
    from workloads import make_inputs
    x = make_inputs(hq, hkv, d, nc + m, nq, seed=4321)
    y = np.random.default_rng(7).standard_normal((hq, nq, d)).astype(np.float32)
    v_r = np.ascontiguousarray(x["v"][:, nc:])
    desc = H.desc_of(hq, hkv, d, nc + m, nq, False)
    ws = kvc.workspace(kvc.OP_RIDGE_FIT, desc, nc, H.DEV)
    v_c = torch.empty(hkv, nc, d, dtype=torch.float32, device=H.DEV)
    kvc.kvc_ridge_value_fit(desc, nc, H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(v_r), H.dev_f32(y), lam,
                            v_c, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == 0
    got = v_c.cpu().numpy().astype(np.float64)
    from tests.test_parity_gpu import _check_ridge
    _check_ridge("bench shape", x, v_r, y, nc, lam, False, got)


def test_step_replays_in_a_graph():
    """Every call of the step only enqueues kernels on its stream (no allocation, no memset, no host
    synchronisation), so the whole step can be captured in a HIP graph.  Replays, with eager work
    between them that clobbers the outputs, give results bitwise equal to the eager step."""
    cfg = get_config(1)
    print("case graph replay: llama8b_prefill_n8192 step", flush=True)
    hq, hkv, d, N, Nq = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries
    x = make_config_inputs(cfg)
    q, k, v = (H.dev_bf16(x[n]) for n in ("q", "k", "v"))
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    lse = torch.empty(hq, Nq, dtype=torch.float32, device=H.DEV)
    w = torch.empty(hkv, N, dtype=torch.float32, device=H.DEV)
    wc = torch.empty(hkv, d, dtype=torch.float32, device=H.DEV)
    bv = torch.empty(hkv, N, dtype=torch.uint8, device=H.DEV)
    bk = torch.empty(hkv, d, dtype=torch.uint8, device=H.DEV)
    ws = {op: kvc.workspace(op, desc, mode, H.DEV) for op, mode in
          ((kvc.OP_ROW_LSE, 0), (kvc.OP_SCORE_TOKENS, 0), (kvc.OP_CHANNEL_WEIGHTS, 0), (kvc.OP_QUANTIZE_PACK, 0))}
    ws_v = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_V_TOKENS, H.DEV)
    ws_k = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, kvc.ALLOC_K_CHANNELS, H.DEV)
    res_v, res_k = kvc.alloc_result_buffer(H.DEV), kvc.alloc_result_buffer(H.DEV)
    cache = kvc.PackedCache(desc, H.DEV)

    def step(s):
        kvc.kvc_row_lse(desc, q, k, lse, ws[kvc.OP_ROW_LSE], stream=s)
        kvc.kvc_score_tokens(desc, kvc.SCORE_SUM, q, k, lse, w, ws[kvc.OP_SCORE_TOKENS], stream=s)
        kvc.kvc_channel_weights(desc, q, k, wc, ws[kvc.OP_CHANNEL_WEIGHTS], stream=s)
        kvc.kvc_allocate_bits(desc, kvc.ALLOC_V_TOKENS, w, bv, ws_v, avg_bits=cfg.avg_bits, result=res_v, stream=s)
        kvc.kvc_allocate_bits(desc, kvc.ALLOC_K_CHANNELS, wc, bk, ws_k, bits_v=bv, avg_bits=cfg.avg_bits,
                              result=res_k, stream=s)
        kvc.kvc_quantize_pack(desc, k, v, bv, bk, cache, ws[kvc.OP_QUANTIZE_PACK], stream=s)

    def outputs():
        torch.cuda.synchronize()
        packed = cache.to_numpy()                      # the buffers trimmed to the lengths the header records
        return [t.cpu().numpy() for t in (lse, w, wc, bv, bk, res_v, res_k)] + [packed[n] for n in sorted(packed)]

    main = torch.cuda.current_stream()
    step(main)
    ref = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    for _ in range(3):
        w.fill_(0)
        bv.fill_(0)
        lse.fill_(0)
        cache.buffers["k_words"].fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        now = outputs()
        for a, b in zip(ref, now):
            np.testing.assert_array_equal(a, b)
