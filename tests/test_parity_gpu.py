"""GPU parity: every C-ABI call against the float64 oracle on the same seeded inputs.

Bars (derived from the arithmetic): row LSE 1e-4 abs; token scores rel 1e-3
(floor 1e-30); channel weights rel 1e-5; widths, results and packed buffers bit-exact from
identical float32 weights / widths; attention outputs and LSEs within the bounds that
gpu_helpers.attend_tols derives from the operand precisions and the inputs' magnitudes
(never looser than 2e-2 and 1e-3 abs).
"""

import math

import zlib

import numpy as np
import pytest
import torch

import kv_cache_compression_pass_amd as kvc
import oracle
from workloads import make_inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    kvc.load()


SMALL = [
    # name, H_q, H_kv, d, N, Nq, causal, avg_bits
    ("g4_d128_ragged", 8, 2, 128, 1000, 1000, True, 3.0),
    ("g1_d64_q_lt_n", 2, 2, 64, 700, 300, True, 2.5),
    ("g2_d128_noncausal", 4, 2, 128, 333, 129, False, 4.0),
    ("g4_d128_one_row", 4, 1, 128, 517, 1, True, 2.0),
    ("g1_d64_one_key", 1, 1, 64, 1, 1, True, 4.0),
    ("g3_d64_two_tiles", 6, 2, 64, 300, 257, True, 1.5),
    ("g4_d128_outliers", 8, 2, 128, 1536, 1536, True, 3.0),
]


def _pipeline(name, hq, hkv, d, N, Nq, causal, avg, seed, x=None, n_fid=64):
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} N={N} Nq={Nq} causal={causal}", flush=True)
    if x is None:
        x = make_inputs(hq, hkv, d, N, Nq, seed=seed, k_outliers=("outliers" in name))
    desc = H.desc_of(hq, hkv, d, N, Nq, causal)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])

    lse_t = H.row_lse(desc, q, k)
    lse_r = oracle.row_lse(x["q"], x["k"], causal=causal)
    H.assert_abs(lse_t.cpu().numpy(), lse_r, 1e-4, "row_lse")

    w_g = H.score_sum(desc, q, k, lse_t).cpu().numpy()
    w_r = oracle.token_scores_sum(x["q"], x["k"], lse_r, causal=causal)
    H.assert_rel(w_g, w_r, 1e-3, what="token scores (sum)")

    wc_g = H.channel_weights(desc, q, k).cpu().numpy()
    wc_r = oracle.channel_weights(x["q"], x["k"])
    H.assert_rel(wc_g, wc_r, 1e-5, what="channel weights")

    # allocation from identical float32 weights (the oracle's, rounded once)
    w32 = w_r.astype(np.float32)
    bv_g, res_v, st = H.allocate(desc, kvc.ALLOC_V_TOKENS, H.dev_f32(w32), avg)
    bv_r, info_v = oracle.allocate_v_tokens(w32, avg, d)
    assert st == 0
    np.testing.assert_array_equal(bv_g.cpu().numpy(), bv_r)
    assert res_v["lam"] == info_v["lam"] and res_v["used"] == info_v["used"]
    assert res_v["budget"] == info_v["budget"]
    assert res_v["distortion"] == pytest.approx(info_v["distortion"], rel=1e-12)
    wc32 = wc_r.astype(np.float32)
    bk_g, res_k, st = H.allocate(desc, kvc.ALLOC_K_CHANNELS, H.dev_f32(wc32), avg, bits_v=H.dev_u8(bv_r))
    bk_r, info_k = oracle.allocate_k_channels(wc32, bv_r, avg)
    assert st == 0
    np.testing.assert_array_equal(bk_g.cpu().numpy(), bk_r)
    assert res_k["lam"] == info_k["lam"] and res_k["used"] == info_k["used"]
    assert res_k["budget"] == info_k["budget"]

    # pack from identical widths: every buffer bit-exact
    cache, st = H.pack(desc, k, v, H.dev_u8(bv_r), H.dev_u8(bk_r))
    assert st == 0
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], bv_r, bk_r))

    # fidelity attend on the last rows: compressed, then the all-16 cache
    nf = min(Nq, n_fid)
    qf_bits = np.ascontiguousarray(x["q"][:, Nq - nf:, :])
    desc_f = H.desc_of(hq, hkv, d, N, nf, causal)
    out_g, lh_g, st = H.attend(desc_f, H.dev_bf16(qf_bits), cache)
    assert st == 0
    out_r, lh_r = oracle.compressed_attend(qf_bits, x["k"], x["v"], bv_r, bk_r, causal=causal)
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [x["v"]], lh_r)
    H.assert_abs(out_g.cpu().numpy(), out_r, ty, "compressed attend output")
    H.assert_abs(lh_g.cpu().numpy(), lh_r, tl, "compressed attend lse")
    full_v = np.full((hkv, N), 16, np.uint8)
    full_k = np.full((hkv, d), 16, np.uint8)
    cache16, st = H.pack(desc, k, v, H.dev_u8(full_v), H.dev_u8(full_k))
    y_g, l_g, st2 = H.attend(desc_f, H.dev_bf16(qf_bits), cache16)
    assert st == 0 and st2 == 0
    y_r, l_r = oracle.full_attend(qf_bits, x["k"], x["v"], causal=causal)
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [x["v"]], l_r)
    H.assert_abs(y_g.cpu().numpy(), y_r, ty, "full attend output")
    H.assert_abs(l_g.cpu().numpy(), l_r, tl, "full attend lse")

    # KVSculpt's loss terms per query head, from the two attends above
    terms = torch.empty(hq, 2, dtype=torch.float64, device=H.DEV)
    kvc.kvc_fidelity_terms(desc_f, out_g, lh_g, y_g, l_g, terms)
    t_r = oracle.fidelity_terms_per_head(out_g.cpu().numpy(), y_g.cpu().numpy(), lh_g.cpu().numpy(),
                                         l_g.cpu().numpy())
    np.testing.assert_allclose(terms.cpu().numpy(), t_r, rtol=1e-10, atol=0)
    return x


@pytest.mark.parametrize("step,causal", [(24.0, False), (24.0, True), (10.0, False)])
def test_row_lse_rising_maxima(step, causal):
    """Row maxima that rise by about 73 (step 24) or 31 (step 10) in the base-2 domain every
    160 keys, so the pipelined LSE must re-take its shift mid-row (a sum past 2^64) or carry
    terms up to 2^62 until it does.  Logits reach about 3.5e3 before scaling, so the bound
    adds the float32 accumulation error of a d-term dot product at that size."""
    from workloads import f32_to_bf16_bits
    d, N = 128, 1024
    print(f"case rising maxima: step={step} causal={causal} d={d} N={N}", flush=True)
    rng = np.random.default_rng(int(step) + 2 * causal)
    u = np.zeros(d, np.float32)
    u[:16] = 1.0
    level = (np.arange(N) // 160).astype(np.float32) * step
    kf = rng.standard_normal((1, N, d), dtype=np.float32) + level[None, :, None] * u
    qf = rng.standard_normal((1, N, d), dtype=np.float32) + 1.5 * u
    qb, kb = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
    desc = H.desc_of(1, 1, d, N, N, causal)
    got = H.row_lse(desc, H.dev_bf16(qb), H.dev_bf16(kb)).cpu().numpy()
    want = oracle.row_lse(qb, kb, causal=causal)
    raw = float(np.max(np.abs(qf)) * np.max(np.abs(kf)) * 16 + 2 * d)
    tol = 1e-4 + d * 2.0 ** -24 * raw / math.sqrt(d)
    assert np.all(np.isfinite(got))
    H.assert_abs(got, want, tol, "row_lse with rising maxima")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_pipeline(case):
    name, hq, hkv, d, N, Nq, causal, avg = case
    _pipeline(name, hq, hkv, d, N, Nq, causal, avg, seed=zlib.crc32(name.encode()) % 1000)


def test_config0_tiny_full_parity():
    from workloads import get_config, make_config_inputs
    cfg = get_config(0)
    x = make_config_inputs(cfg)
    _pipeline("config0", cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries,
              True, cfg.avg_bits, seed=None, x=x, n_fid=cfg.fidelity_rows)


MAXCASES = [
    # name, H_q, H_kv, d, N, Nq, D_h, causal
    ("max_g7_d128", 14, 2, 128, 600, 600, 256, True),
    ("max_g2_d64_q_lt_n", 4, 2, 64, 300, 200, 96, True),
    ("max_g1_d128_noncausal", 2, 2, 128, 129, 64, 40, False),
]


@pytest.mark.parametrize("case", MAXCASES, ids=[c[0] for c in MAXCASES])
def test_max_scores_and_topk(case):
    name, hq, hkv, d, N, Nq, Dh, causal = case
    print(f"case {name}", flush=True)
    x = make_inputs(hq, hkv, d, N, Nq, seed=77, hidden_dim=Dh)
    desc = H.desc_of(hq, hkv, d, N, Nq, causal)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    lse_t = H.row_lse(desc, q, k)
    lse_r = oracle.row_lse(x["q"], x["k"], causal=causal)
    s_g = H.score_max(desc, q, k, lse_t, H.dev_bf16(x["hidden"]), H.dev_bf16(x["w_o"]), v).cpu().numpy()
    s_r = oracle.token_scores_max(x["q"], x["k"], lse_r, x["hidden"], x["w_o"], x["v"], causal=causal)
    H.assert_rel(s_g, s_r, 1e-3, what="KVzip+ scores")
    s32 = s_r.astype(np.float32)
    for frac in (0.25, 0.0, 1.0, 0.5):
        b_g, res, st = H.allocate(desc, kvc.ALLOC_TOPK, H.dev_f32(s32), keep_fraction=frac, keep_bits=16)
        b_r = oracle.topk_keep(s32, frac, 16)
        np.testing.assert_array_equal(b_g.cpu().numpy(), b_r)
        assert res["used"] == int(b_r.astype(np.int64).sum()) * d
    cache, st = H.pack(desc, k, v, H.dev_u8(b_r), H.dev_u8(np.full((hkv, d), 16, np.uint8)))
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], b_r, np.full((hkv, d), 16, np.uint8)))


UNCHUNKED = [
    # name, mode, H_q, H_kv, d, N, Nq, causal, D_h
    ("sum_g16_d128_n2304", "sum", 128, 8, 128, 2304, 2304, True, 0),
    ("sum_g4_d64_q_lt_n", "sum", 128, 32, 64, 2500, 2100, True, 0),
    ("sum_g8_d128_noncausal", "sum", 128, 16, 128, 2600, 2304, False, 0),
    ("max_g4_d64_n2048", "max", 128, 32, 64, 2048, 2048, True, 512),
]


@pytest.mark.parametrize("case", UNCHUNKED, ids=[c[0] for c in UNCHUNKED])
def test_scorer_one_chunk_per_item(case):
    """The scorer's launch shape for layers with at least 1024 (query head, 256-row tile) items:
    each item takes its whole key range as one chunk, pass 1 writes the row LSE directly, and the
    column reduction adds one partial per row tile (9 here, with a ragged last tile when Nq is not
    a multiple of 256).  The full-size workloads take this path; here every row LSE and every
    score column of every head is compared with the oracle."""
    from tests import oracle_blocks as OB
    name, mode, hq, hkv, d, N, Nq, causal, Dh = case
    assert -(-Nq // 256) * hq >= 1024
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} N={N} Nq={Nq} causal={causal} mode={mode}", flush=True)
    x = make_inputs(hq, hkv, d, N, Nq, seed=zlib.crc32(name.encode()) % 1000, hidden_dim=Dh)
    desc = H.desc_of(hq, hkv, d, N, Nq, causal)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    lse_t = H.row_lse(desc, q, k)
    lse_r = OB.head_lse(x["q"], x["k"], list(range(hq)), causal=causal)
    H.assert_abs(lse_t.cpu().numpy(), lse_r, 1e-4, "row_lse")
    G = hq // hkv
    if mode == "sum":
        s_g = H.score_sum(desc, q, k, lse_t).cpu().numpy()
        s_r = np.stack([OB.group_scores_sum(x["q"], x["k"], lse_r[g * G:(g + 1) * G], g, causal=causal)
                        for g in range(hkv)])
        np.testing.assert_allclose(s_g.astype(np.float64).sum(axis=1), G * Nq, rtol=2e-5)
    else:
        s_g = H.score_max(desc, q, k, lse_t, H.dev_bf16(x["hidden"]), H.dev_bf16(x["w_o"]), v).cpu().numpy()
        s_r = np.stack([OB.group_scores_max(x["q"], x["k"], lse_r[g * G:(g + 1) * G], x["hidden"], x["w_o"],
                                            x["v"], g, causal=causal) for g in range(hkv)])
    H.assert_rel(s_g, s_r, 1e-3, what=f"token scores ({mode})")


def test_kvsculpt_pilot_flow():
    """KVSculpt's adaptive budget (KVSculpt summary, §2) as one flow through the C ABI: a pilot at a
    uniform budget (every KV head allocated alone at the same average, one-head descriptors), pack,
    compressed and full attends on the last rows, per-head loss terms, budgets in proportion to
    sqrt(pilot MSE), then every head allocated again alone at its own budget.  Each decision is
    compared with the oracle's same step on identical inputs: widths, budgets and packed bytes bit
    for bit, attends within their derived bounds, loss terms at rel 1e-10."""
    hq, hkv, d, N, Nq, nf, a0 = 8, 2, 128, 1024, 1024, 64, 3.0   # N d = 2^17: budgets map to exact averages
    print(f"case pilot flow: H_q={hq} H_kv={hkv} d={d} N={N} fidelity rows={nf} pilot avg={a0}", flush=True)
    G = hq // hkv
    x = make_inputs(hq, hkv, d, N, Nq, seed=808, k_outliers=True)
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    w32 = H.score_sum(desc, q, k, H.row_lse(desc, q, k)).cpu().numpy()
    wc32 = H.channel_weights(desc, q, k).cpu().numpy()
    one = H.desc_of(G, 1, d, N, Nq, True)

    def allocate_heads(avgs):
        bv = np.zeros((hkv, N), np.uint8)
        bk = np.zeros((hkv, d), np.uint8)
        for g in range(hkv):
            bvg, res, st = H.allocate(one, kvc.ALLOC_V_TOKENS, H.dev_f32(w32[g:g + 1]), avgs[g])
            assert st == 0
            bv_r, info = oracle.allocate_v_tokens(w32[g:g + 1], avgs[g], d)
            np.testing.assert_array_equal(bvg.cpu().numpy(), bv_r)
            assert res["used"] == info["used"] and res["budget"] == info["budget"]
            bkg, resk, st = H.allocate(one, kvc.ALLOC_K_CHANNELS, H.dev_f32(wc32[g:g + 1]), avgs[g],
                                       bits_v=H.dev_u8(bv_r))
            bk_r, infok = oracle.allocate_k_channels(wc32[g:g + 1], bv_r, avgs[g])
            np.testing.assert_array_equal(bkg.cpu().numpy(), bk_r)
            bv[g], bk[g] = bv_r[0], bk_r[0]
        return bv, bk

    qf = np.ascontiguousarray(x["q"][:, Nq - nf:, :])
    desc_f = H.desc_of(hq, hkv, d, N, nf, True)
    c16, st = H.pack(desc, k, v, H.dev_u8(np.full((hkv, N), 16, np.uint8)), H.dev_u8(np.full((hkv, d), 16, np.uint8)))
    y_g, l_g, st2 = H.attend(desc_f, H.dev_bf16(qf), c16)
    assert st == 0 and st2 == 0

    # pilot: every head at the same average
    bv, bk = allocate_heads([a0] * hkv)
    cache, st = H.pack(desc, k, v, H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], bv, bk))
    yh_g, lh_g, st = H.attend(desc_f, H.dev_bf16(qf), cache)
    assert st == 0
    yh_r, lh_r = oracle.compressed_attend(qf, x["k"], x["v"], bv, bk)
    ty, tl = H.attend_tols(qf, [x["k"]], [x["v"]], lh_r)
    H.assert_abs(yh_g.cpu().numpy(), yh_r, ty, "pilot attend output")
    H.assert_abs(lh_g.cpu().numpy(), lh_r, tl, "pilot attend lse")
    terms = torch.empty(hq, 2, dtype=torch.float64, device=H.DEV)
    kvc.kvc_fidelity_terms(desc_f, yh_g, lh_g, y_g, l_g, terms)
    t_g = terms.cpu().numpy()
    np.testing.assert_allclose(t_g, oracle.fidelity_terms_per_head(yh_g.cpu().numpy(), y_g.cpu().numpy(),
                                                                   lh_g.cpu().numpy(), l_g.cpu().numpy()),
                               rtol=1e-10, atol=0)
    # the pilot MSE of a KV head: output error over its query heads' rows and channels
    mse = t_g[:, 0].reshape(hkv, G).sum(axis=1) / (G * nf * d)
    total = int(a0 * hkv * N * d)
    budgets = kvc.kvc_pilot_budgets(mse, total)
    np.testing.assert_array_equal(budgets, oracle.pilot_budgets(mse, total))
    assert int(budgets.sum()) == total
    # the same decision from the oracle's own attend moves each budget by no more than the change
    # of its share, times the total, plus one unit of rounding
    y_r, l_r = oracle.full_attend(qf, x["k"], x["v"])
    mse_r = oracle.fidelity_terms_per_head(yh_r, y_r, lh_r, l_r)[:, 0].reshape(hkv, G).sum(axis=1) / (G * nf * d)
    share, share_r = np.sqrt(mse) / np.sqrt(mse).sum(), np.sqrt(mse_r) / np.sqrt(mse_r).sum()
    assert np.abs(oracle.pilot_budgets(mse_r, total) - budgets).max() <= total * np.abs(share - share_r).max() + 1
    print(f"pilot MSE per KV head {mse.tolist()}, budgets {budgets.tolist()} bits", flush=True)

    # final allocation: each head alone at its own budget (budget / (N d) is exact, so B = budget)
    avgs = [float(b) / (N * d) for b in budgets]
    bv2, bk2 = allocate_heads(avgs)
    used = [int((bv2[g].astype(np.int64)).sum()) * d for g in range(hkv)]
    assert all(u <= int(b) for u, b in zip(used, budgets))
    cache2, st = H.pack(desc, k, v, H.dev_u8(bv2), H.dev_u8(bk2))
    assert st == 0
    H.compare_packed(cache2.to_numpy(), oracle.pack_cache(x["k"], x["v"], bv2, bk2))


def test_allocation_ties_zeros_and_extremes():
    print("case allocation edge cases", flush=True)
    hkv, N, d = 3, 2000, 64
    desc = H.desc_of(hkv, hkv, d, N, N, True)
    rng = np.random.default_rng(5)
    w = rng.integers(0, 6, (hkv, N)).astype(np.float32) * np.float32(0.125)   # many ties, zeros
    for avg in (0.0, 0.3, 1.0, 2.0, 3.0, 4.0, 7.5, 16.0, 20.0):
        b_g, res, st = H.allocate(desc, kvc.ALLOC_V_TOKENS, H.dev_f32(w), avg)
        b_r, info = oracle.allocate_v_tokens(w, avg, d)
        np.testing.assert_array_equal(b_g.cpu().numpy(), b_r, err_msg=f"avg {avg}")
        assert res["lam"] == info["lam"] and res["used"] == info["used"]
        assert res["budget"] == info["budget"]
    sigma = rng.uniform(0.5, 2.0, (hkv, N)).astype(np.float32)
    b_g, res, st = H.allocate(desc, kvc.ALLOC_V_TOKENS, H.dev_f32(w), 2.5, sigma=H.dev_f32(sigma))
    b_r, info = oracle.allocate_v_tokens(w, 2.5, d, sigma=sigma)
    np.testing.assert_array_equal(b_g.cpu().numpy(), b_r)
    # K stage where one head keeps nothing
    bv = rng.choice(np.array([0, 2, 4, 8, 16], np.uint8), (hkv, N))
    bv[1] = 0
    wc = rng.exponential(1.0, (hkv, d)).astype(np.float32)
    b_g, res, st = H.allocate(desc, kvc.ALLOC_K_CHANNELS, H.dev_f32(wc), 3.0, bits_v=H.dev_u8(bv))
    b_r, info = oracle.allocate_k_channels(wc, bv, 3.0)
    np.testing.assert_array_equal(b_g.cpu().numpy(), b_r)
    assert res["lam"] == info["lam"] and res["used"] == info["used"]


def test_bad_width_sets_device_status():
    print("case bad width status", flush=True)
    x = make_inputs(2, 1, 64, 100, 100, seed=3)
    desc = H.desc_of(2, 1, 64, 100, 100, True)
    bv = np.full((1, 100), 4, np.uint8)
    bv[0, 7] = 3
    bk = np.full((1, 64), 8, np.uint8)
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(x["v"]), H.dev_u8(bv), H.dev_u8(bk))
    assert st & kvc.DEV_BAD_WIDTH
    bv[0, 7] = 4
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(x["v"]), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    wc = np.ones((1, 64), np.float32)
    bv[0, 9] = 5
    _, _, st = H.allocate(desc, kvc.ALLOC_K_CHANNELS, H.dev_f32(wc), 2.0, bits_v=H.dev_u8(bv))
    assert st & kvc.DEV_BAD_WIDTH


@pytest.mark.parametrize("rows", [1, 40], ids=["decode_path", "matrix_core_path"])
def test_attend_reports_a_cache_that_does_not_match(rows):
    """A packed cache whose header does not match the call's descriptor is refused on the device
    (KVC_DEV_BAD_CACHE; the kernels read nothing past the header), on both attend paths, and the
    next call with a matching cache and the same workspace clears the status word."""
    print(f"case bad cache status, {rows} rows per query head", flush=True)
    hq, hkv, d, N = 4, 2, 64, 300
    x = make_inputs(hq, hkv, d, N, N, seed=77)
    desc = H.desc_of(hq, hkv, d, N, N, True)
    bv = np.full((hkv, N), 4, np.uint8)
    bk = np.full((hkv, d), 4, np.uint8)
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(x["v"]), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    desc_f = H.desc_of(hq, hkv, d, N, rows, True)
    qf = H.dev_bf16(np.ascontiguousarray(x["q"][:, N - rows:, :]))
    ws = kvc.workspace(kvc.OP_COMPRESSED_ATTEND, desc_f, 0, H.DEV)
    out = torch.empty(hq, rows, d, dtype=torch.float32, device=H.DEV)
    lse = torch.empty(hq, rows, dtype=torch.float32, device=H.DEV)
    hdr = cache.buffers["header"]
    good = hdr[16:24].clone()                       # global header word 2: N
    hdr[16:24] = torch.from_numpy(np.array([N + 1], np.int64).view(np.uint8)).to(hdr.device)
    kvc.kvc_compressed_attend(desc_f, qf, cache, out, lse, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == kvc.DEV_BAD_CACHE
    hdr[16:24] = good
    kvc.kvc_compressed_attend(desc_f, qf, cache, out, lse, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == 0
    out_r, lh_r = oracle.compressed_attend(np.ascontiguousarray(x["q"][:, N - rows:, :]), x["k"], x["v"], bv, bk)
    ty, tl = H.attend_tols(x["q"][:, N - rows:, :], [x["k"]], [x["v"]], lh_r)
    H.assert_abs(out.cpu().numpy(), out_r, ty, "attend output after a refused call")


def test_evict_everything_and_empty_rows():
    print("case evict everything", flush=True)
    hq, hkv, d, N, Nq = 4, 2, 128, 300, 40
    x = make_inputs(hq, hkv, d, N, Nq, seed=9)
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    k, v = H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    bv = np.zeros((hkv, N), np.uint8)
    bv[1, :5] = 8                     # head 1 keeps 5 early tokens; head 0 keeps nothing
    bk = np.full((hkv, d), 4, np.uint8)
    cache, st = H.pack(desc, k, v, H.dev_u8(bv), H.dev_u8(bk))
    H.compare_packed(cache.to_numpy(), oracle.pack_cache(x["k"], x["v"], bv, bk))
    out_g, lh_g, st = H.attend(desc, H.dev_bf16(x["q"]), cache)
    out_r, lh_r = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk)
    ty, tl = H.attend_tols(x["q"], [x["k"]], [x["v"]], lh_r)
    H.assert_abs(out_g.cpu().numpy(), out_r, ty, "out")
    H.assert_abs(lh_g.cpu().numpy(), lh_r, tl, "lse")
    assert np.isneginf(lh_g.cpu().numpy()[:2]).all()


def test_determinism_bitwise():
    print("case determinism", flush=True)
    hq, hkv, d, N, Nq = 8, 2, 128, 2048, 2048
    x = make_inputs(hq, hkv, d, N, Nq, seed=31, k_outliers=True)
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    q, k, v = H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    runs = []
    for _ in range(2):
        lse = H.row_lse(desc, q, k)
        w = H.score_sum(desc, q, k, lse)
        wc = H.channel_weights(desc, q, k)
        bv, _, _ = H.allocate(desc, kvc.ALLOC_V_TOKENS, w, 2.0)
        bk, _, _ = H.allocate(desc, kvc.ALLOC_K_CHANNELS, wc, 2.0, bits_v=bv)
        cache, _ = H.pack(desc, k, v, bv, bk)
        runs.append((lse.cpu().numpy(), w.cpu().numpy(), wc.cpu().numpy(), bv.cpu().numpy(),
                     bk.cpu().numpy(), cache.to_numpy()))
    a, b = runs
    for i in range(5):
        assert a[i].tobytes() == b[i].tobytes()
    H.compare_packed(a[5], b[5])
    # the whole GPU pipeline vs the oracle pipeline: report width mismatches, each must sit
    # at a key within tolerance of lambda*
    w_r = oracle.token_scores_sum(x["q"], x["k"], oracle.row_lse(x["q"], x["k"]))
    bv_r, info = oracle.allocate_v_tokens(w_r.astype(np.float32), 2.0, d)
    mism = np.argwhere(a[3] != bv_r)
    print(f"end-to-end V widths differing from the oracle pipeline: {len(mism)} of {bv_r.size}")
    lam = info["lam"]
    for g, t in mism:
        ks = oracle.step_keys(np.array([w_r[g, t]], np.float32), np.array([d]))[0]
        assert np.min(np.abs(ks - lam)) <= 2e-3 * lam


@pytest.mark.gpu
@pytest.mark.parametrize("bvv,bkk", [(16, 16), (16, 8), (8, 16), (4, 4), (2, 2)])
def test_attend_group_aligned_uniform_widths(bvv, bkk):
    """Every K group full (N a multiple of 32, nothing evicted): the causal mask must act inside
    full groups too, at every width."""
    hq, hkv, d, N, Nq, nf = 4, 1, 128, 64, 64, 64
    x = make_inputs(hq, hkv, d, N, Nq, seed=5)
    desc = H.desc_of(hq, hkv, d, N, Nq, True)
    k, v = H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    bv = np.full((hkv, N), bvv, np.uint8)
    bk = np.full((hkv, d), bkk, np.uint8)
    cache, st = H.pack(desc, k, v, H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    qf = np.ascontiguousarray(x["q"][:, Nq - nf:, :])
    y_g, l_g, st2 = H.attend(H.desc_of(hq, hkv, d, N, nf, True), H.dev_bf16(qf), cache)
    assert st2 == 0
    y_r, l_r = oracle.compressed_attend(qf, x["k"], x["v"], bv, bk)
    ty, tl = H.attend_tols(qf, [x["k"]], [x["v"]], l_r)
    H.assert_abs(y_g.cpu().numpy(), y_r, ty, "attend output")
    H.assert_abs(l_g.cpu().numpy(), l_r, tl, "attend lse")


KEEP_CASES = [
    # name, H_kv, N, threshold (None: the head-0 median score), window, keep_bits
    ("ragged_median_w128", 3, 1000, None, 128, 16),
    ("ragged_inf_window_only", 3, 1000, float("inf"), 128, 16),
    ("ragged_neg_inf_all", 2, 777, float("-inf"), 0, 8),
    ("window_past_n", 2, 100, 5.0, 1000, 4),
    ("no_window_bits2", 4, 4096 + 17, 0.25, 0, 2),
    ("large_8x131072", 8, 131072, None, 128, 16),
]


@pytest.mark.parametrize("case", KEEP_CASES, ids=[c[0] for c in KEEP_CASES])
def test_keep_threshold(case):
    """Threshold-and-window keep against the oracle, bit-exact, with planted NaN scores and
    scores equal to the threshold, rows both 16-byte aligned and not."""
    name, hkv, n, thr, window, kb = case
    print(f"case keep_threshold {name}: H_kv={hkv} N={n}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    s = rng.standard_normal((hkv, n)).astype(np.float32)
    if thr is None:
        thr = float(np.median(s[0]))
    if np.isfinite(thr):
        s.flat[rng.choice(s.size, 5, replace=False)] = np.float32(thr)    # ties at the threshold
    s.flat[rng.choice(s.size, 3, replace=False)] = np.nan
    desc = H.desc_of(hkv, hkv, 64, n, 1, True)
    bits = torch.full((hkv, n), 255, dtype=torch.uint8, device=H.DEV)
    kept = torch.full((hkv,), -1, dtype=torch.int64, device=H.DEV)
    kvc.kvc_keep_threshold(desc, H.dev_f32(s), thr, bits, window=window, keep_bits=kb, kept=kept)
    torch.cuda.synchronize()
    want = oracle.threshold_keep(s, thr, window, keep_bits=kb)
    np.testing.assert_array_equal(bits.cpu().numpy(), want)
    np.testing.assert_array_equal(kept.cpu().numpy(), (want > 0).sum(axis=1))
    # without the count buffer the widths are the same
    bits2 = torch.zeros((hkv, n), dtype=torch.uint8, device=H.DEV)
    kvc.kvc_keep_threshold(desc, H.dev_f32(s), thr, bits2, window=window, keep_bits=kb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits2.cpu().numpy(), want)


DECODE_CASES = [
    # name, H_q, H_kv, d, N, rows per query head, causal
    ("dec_g4_d128_n3000_r1", 8, 2, 128, 3000, 1, True),
    ("dec_g7_d128_n1000_r2", 7, 1, 128, 1000, 2, True),
    ("dec_g8_d64_n777_r2", 8, 1, 64, 777, 2, True),
    ("dec_g1_d64_n64_r1", 1, 1, 64, 64, 1, False),
    ("dec_g2_d128_n513_noncausal", 4, 2, 128, 513, 1, False),
    ("dec_g3_d128_n2049_r1", 6, 2, 128, 2049, 1, True),
]


def _random_widths(rng, hkv, n, d):
    bv = rng.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(hkv, n), p=[0.3, 0.2, 0.2, 0.2, 0.1])
    bk = rng.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(hkv, d), p=[0.1, 0.3, 0.3, 0.2, 0.1])
    return bv.astype(np.uint8), bk.astype(np.uint8)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_attend_decode_rows(case):
    """Decode-shaped attend (G * rows <= 16 query rows per KV head: the VALU path) against the
    oracle, on random widths with evictions, then on the all-16 cache against full attention."""
    name, hq, hkv, d, N, rows, causal = case
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} N={N} rows={rows} causal={causal}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    x = make_inputs(hq, hkv, d, N, N, seed=zlib.crc32(name.encode()) % 1000, k_outliers=True)
    bv, bk = _random_widths(rng, hkv, N, d)
    desc = H.desc_of(hq, hkv, d, N, N, causal)
    k, v = H.dev_bf16(x["k"]), H.dev_bf16(x["v"])
    cache, st = H.pack(desc, k, v, H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    qf_bits = np.ascontiguousarray(x["q"][:, N - rows:, :])
    desc_f = H.desc_of(hq, hkv, d, N, rows, causal)
    out_g, lh_g, st = H.attend(desc_f, H.dev_bf16(qf_bits), cache)
    assert st == 0
    out_r, lh_r = oracle.compressed_attend(qf_bits, x["k"], x["v"], bv, bk, causal=causal)
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [x["v"]], lh_r)
    H.assert_abs(out_g.cpu().numpy(), out_r, ty, "decode attend output")
    H.assert_abs(lh_g.cpu().numpy(), lh_r, tl, "decode attend lse")
    cache16, st = H.pack(desc, k, v, H.dev_u8(np.full((hkv, N), 16, np.uint8)),
                         H.dev_u8(np.full((hkv, d), 16, np.uint8)))
    y_g, l_g, st2 = H.attend(desc_f, H.dev_bf16(qf_bits), cache16)
    assert st == 0 and st2 == 0
    y_r, l_r = oracle.full_attend(qf_bits, x["k"], x["v"], causal=causal)
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [x["v"]], l_r)
    H.assert_abs(y_g.cpu().numpy(), y_r, ty, "decode attend output, all-16 cache")
    H.assert_abs(l_g.cpu().numpy(), l_r, tl, "decode attend lse, all-16 cache")


def test_attend_decode_row_that_sees_nothing():
    """Two rows per query head, only the last token retained: the first row (one position
    earlier) sees no retained token (output 0, LSE -inf); the second sees exactly one."""
    hq, hkv, d, N, rows = 4, 1, 128, 300, 2
    print("case decode row that sees nothing", flush=True)
    x = make_inputs(hq, hkv, d, N, N, seed=77)
    bv = np.zeros((hkv, N), np.uint8)
    bv[:, N - 1] = 8
    bk = np.full((hkv, d), 4, np.uint8)
    desc = H.desc_of(hq, hkv, d, N, N, True)
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(x["v"]), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    qf_bits = np.ascontiguousarray(x["q"][:, N - rows:, :])
    out_g, lh_g, st = H.attend(H.desc_of(hq, hkv, d, N, rows, True), H.dev_bf16(qf_bits), cache)
    assert st == 0
    out_r, lh_r = oracle.compressed_attend(qf_bits, x["k"], x["v"], bv, bk, causal=True)
    og, lg = out_g.cpu().numpy(), lh_g.cpu().numpy()
    assert np.all(og[:, 0, :] == 0.0) and np.all(np.isneginf(lg[:, 0]))
    assert np.all(np.isneginf(lh_r[:, 0]))
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [x["v"]], lh_r)
    H.assert_abs(og, out_r, ty, "decode attend output")
    H.assert_abs(lg[:, 1], lh_r[:, 1], tl, "decode attend lse")


RANGE_CASES = [
    # name, H_q, H_kv, d, N, rows per query head, V scale
    ("range_mfma_large", 8, 2, 128, 700, 64, 1e5),
    ("range_mfma_tiny", 8, 2, 128, 700, 64, 1e-6),
    ("range_mfma_d64_huge", 4, 1, 64, 300, 40, 3e30),
    ("range_decode_large", 8, 2, 128, 700, 1, 1e5),
    ("range_decode_tiny", 8, 2, 128, 700, 1, 1e-6),
]


@pytest.mark.parametrize("case", RANGE_CASES, ids=[c[0] for c in RANGE_CASES])
def test_attend_value_range(case):
    """Values far outside fp16's range (|V| up to ~5e5 and ~1e31) and far below its normal range
    (|V| ~ 1e-6), in the 16-bit zone and the quantised zones (random widths), on both attend paths:
    the output stays within the operand-precision bound relative to max|V|."""
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits
    name, hq, hkv, d, N, rows, vs = case
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} N={N} rows={rows} V scale={vs}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    x = make_inputs(hq, hkv, d, N, N, seed=zlib.crc32(name.encode()) % 1000)
    v_bits = f32_to_bf16_bits((bf16_bits_to_f32(x["v"]) * np.float32(vs)).astype(np.float32))
    bv, bk = _random_widths(rng, hkv, N, d)
    bv[:, -1] = 16                                   # the last row always sees a 16-bit token
    desc = H.desc_of(hq, hkv, d, N, N, True)
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(v_bits), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    qf_bits = np.ascontiguousarray(x["q"][:, N - rows:, :])
    out_g, lh_g, st = H.attend(H.desc_of(hq, hkv, d, N, rows, True), H.dev_bf16(qf_bits), cache)
    assert st == 0
    out_r, lh_r = oracle.compressed_attend(qf_bits, x["k"], v_bits, bv, bk)
    og = out_g.cpu().numpy()
    assert np.isfinite(og).all()
    ty, tl = H.attend_tols(qf_bits, [x["k"]], [v_bits], lh_r, capped=False)
    H.assert_abs(og, out_r, ty, "attend output, scaled V")
    H.assert_abs(lh_g.cpu().numpy(), lh_r, tl, "attend lse, scaled V")
    # the outputs are not flushed: a typical row has |Y| of the order of the V scale
    assert np.abs(out_r).max() > 0.05 * vs


APPEND_CASES = [
    # name, H_q, H_kv, d, N (packed), n_new, rows per query head, causal
    ("app_dec_g4_d128", 8, 2, 128, 1500, 37, 1, True),
    ("app_dec_g8_d64_r2", 8, 1, 64, 700, 130, 2, True),
    ("app_mfma_g4_d128_r64", 8, 2, 128, 1200, 100, 64, True),
    ("app_mfma_rows_before_buffer", 4, 1, 128, 900, 20, 48, True),
    ("app_dec_noncausal", 4, 2, 128, 600, 50, 1, False),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_attend_with_append_buffer(case):
    """Packed cache + raw bf16 buffer of new tokens against the oracle, on the decode path
    (few rows) and the matrix-core path (many rows, some of them before the buffer)."""
    name, hq, hkv, d, N, n_new, rows, causal = case
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} N={N} n_new={n_new} rows={rows} causal={causal}", flush=True)
    seed = zlib.crc32(name.encode())
    rng = np.random.default_rng(seed)
    x = make_inputs(hq, hkv, d, N + n_new, N + n_new, seed=seed % 1000, k_outliers=True)
    k, v = np.ascontiguousarray(x["k"][:, :N]), np.ascontiguousarray(x["v"][:, :N])
    kn, vn = np.ascontiguousarray(x["k"][:, N:]), np.ascontiguousarray(x["v"][:, N:])
    bv, bk = _random_widths(rng, hkv, N, d)
    desc = H.desc_of(hq, hkv, d, N, N, causal)
    cache, st = H.pack(desc, H.dev_bf16(k), H.dev_bf16(v), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    qf_bits = np.ascontiguousarray(x["q"][:, N + n_new - rows:, :])
    desc_f = H.desc_of(hq, hkv, d, N, rows, causal)
    out = torch.empty(hq, rows, d, dtype=torch.float32, device=H.DEV)
    lse = torch.empty(hq, rows, dtype=torch.float32, device=H.DEV)
    ws = kvc.workspace(kvc.OP_COMPRESSED_ATTEND, desc_f, 0, H.DEV)
    kvc.kvc_compressed_attend_append(desc_f, H.dev_bf16(qf_bits), cache, H.dev_bf16(kn), H.dev_bf16(vn),
                                     out, lse, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == 0
    out_r, lh_r = oracle.compressed_attend_append(qf_bits, k, v, bv, bk, kn, vn, causal=causal)
    ty, tl = H.attend_tols(qf_bits, [k, kn], [v, vn], lh_r)
    H.assert_abs(out.cpu().numpy(), out_r, ty, "append attend output")
    H.assert_abs(lse.cpu().numpy(), lh_r, tl, "append attend lse")
    # no new tokens: the same call is the packed cache alone
    kvc.kvc_compressed_attend_append(desc_f, H.dev_bf16(qf_bits), cache, None, None, out, lse, ws)
    torch.cuda.synchronize()
    out0, l0 = oracle.compressed_attend(qf_bits, k, v, bv, bk, causal=causal)
    ty, tl = H.attend_tols(qf_bits, [k], [v], l0)
    H.assert_abs(out.cpu().numpy(), out0, ty, "attend output, empty buffer")
    H.assert_abs(lse.cpu().numpy(), l0, tl, "attend lse, empty buffer")


FID_CASES = [
    # name, H_q, Nq, d
    ("fid_one_row_d128", 4, 1, 128),
    ("fid_ragged_d64", 6, 1001, 64),
    ("fid_many_rows_d128", 32, 2048, 128),
    ("fid_short_d64", 2, 3, 64),
]


@pytest.mark.parametrize("case", FID_CASES, ids=[c[0] for c in FID_CASES])
def test_fidelity_terms(case):
    """Per-head output and LSE error sums against the oracle on the same float32 arrays, with
    rows that see nothing in both attends (0), in one of them (+inf) and equal finite LSEs."""
    name, hq, nq, d = case
    print(f"case {name}: H_q={hq} Nq={nq} d={d}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    y = rng.normal(0.0, 1.0, (hq, nq, d)).astype(np.float32)
    y_hat = (y + rng.normal(0.0, 0.05, y.shape)).astype(np.float32)
    lse = rng.normal(5.0, 2.0, (hq, nq)).astype(np.float32)
    lse_hat = (lse + rng.normal(0.0, 0.01, lse.shape)).astype(np.float32)
    lse_hat[0, 0] = lse[0, 0]                               # equal: adds 0
    if nq > 1:
        lse[1 % hq, 1] = lse_hat[1 % hq, 1] = -np.inf       # sees nothing in both: adds 0
        y[1 % hq, 1] = y_hat[1 % hq, 1] = 0.0
    if hq > 2:
        lse_hat[2, nq - 1] = -np.inf                        # sees nothing only after compression
    desc = H.desc_of(hq, hq, d, nq, nq, True)
    terms = torch.empty(hq, 2, dtype=torch.float64, device=H.DEV)
    kvc.kvc_fidelity_terms(desc, H.dev_f32(y_hat), H.dev_f32(lse_hat), H.dev_f32(y), H.dev_f32(lse), terms)
    got = terms.cpu().numpy()
    want = oracle.fidelity_terms_per_head(y_hat, y, lse_hat, lse)
    fin = np.isfinite(want)
    np.testing.assert_array_equal(np.isfinite(got), fin)
    np.testing.assert_array_equal(got[~fin], want[~fin])
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-10, atol=0)
    # fixed summation order: a second call gives the same bits
    again = torch.empty_like(terms)
    kvc.kvc_fidelity_terms(desc, H.dev_f32(y_hat), H.dev_f32(lse_hat), H.dev_f32(y), H.dev_f32(lse), again)
    assert torch.equal(terms, again)


def _check_ridge(name, x, v_r, y, nc, lam, causal, got):
    """V from the GPU against the oracle's exact solve, within the elementwise bounds derived from
    the GPU's operand precisions (tests/ridge_bounds.py); prints the measured error and residual
    relative to their bounds."""
    from tests.ridge_bounds import ridge_error_bounds
    for g, b in enumerate(ridge_error_bounds(x["q"], x["k"], v_r, y, nc, lam, causal, got)):
        vmax = np.abs(b["exact"]).max()
        print(f"ridge {name} head {g}: cond(M) {b['cond']:.3g}; max|dV|/max|V| {b['err'].max() / vmax:.3g} "
              f"(bound {b['err_bound'].max() / vmax:.3g}); worst error / its bound {(b['err'] / b['err_bound']).max():.3g}; "
              f"worst residual / its bound {(b['res'] / b['res_bound']).max():.3g}", flush=True)
        assert (b["res"] <= b["res_bound"]).all(), "residual outside its derived bound"
        assert (b["err"] <= b["err_bound"]).all(), "V outside its derived bound"
        # The derived bounds are worst cases (d roundings per logit, absolute values through
        # M^-1); the measured errors sit far inside them, at most 6.5e-7 of max|V| over every
        # case, the benchmark shape included.  A regression guard at about 15 times that:
        assert b["err"].max() <= 1e-5 * vmax, "V error far above every measured one"


RIDGE_CASES = [
    # name, H_q, H_kv, d, n_c, m, Nq, causal, lambda
    ("ridge_d64_small", 4, 2, 64, 40, 24, 100, False, 0.1),
    ("ridge_d128_ragged_causal", 8, 2, 128, 130, 70, 200, True, 0.01),
    ("ridge_d128_one_block_no_zone", 2, 1, 128, 64, 0, 64, False, 1.0),
    ("ridge_d128_five_blocks", 6, 2, 128, 300, 100, 128, False, 0.05),
    ("ridge_g1_d64_tiny_lambda", 1, 1, 64, 33, 7, 90, False, 1e-4),
]


@pytest.mark.parametrize("case", RIDGE_CASES, ids=[c[0] for c in RIDGE_CASES])
def test_ridge_value_fit(case):
    """KVSculpt's value solve against the oracle.  The GPU's V solves exactly a system whose float32
    weights and target carry bounded elementwise perturbations, so the residual of the oracle's
    (M, B) at the GPU's V and the error of V itself have elementwise bounds derived from those
    precisions (tests/ridge_bounds.py)."""
    name, hq, hkv, d, nc, m, nq, causal, lam = case
    print(f"case {name}: H_q={hq} H_kv={hkv} d={d} n_c={nc} m={m} Nq={nq} causal={causal} lambda={lam}", flush=True)
    seed = zlib.crc32(name.encode()) % 1000
    x = make_inputs(hq, hkv, d, nc + m, nq, seed=seed)
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((hq, nq, d)).astype(np.float32)
    v_r = np.ascontiguousarray(x["v"][:, nc:])
    desc = H.desc_of(hq, hkv, d, nc + m, nq, causal)
    ws = kvc.workspace(kvc.OP_RIDGE_FIT, desc, nc, H.DEV)
    v_c = torch.empty(hkv, nc, d, dtype=torch.float32, device=H.DEV)
    kvc.kvc_ridge_value_fit(desc, nc, H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(v_r) if m else None,
                            H.dev_f32(y), lam, v_c, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == 0
    got = v_c.cpu().numpy().astype(np.float64)
    _check_ridge(name, x, v_r, y, nc, lam, causal, got)
    # fixed summation order: a second call gives the same bits
    v2 = torch.empty_like(v_c)
    kvc.kvc_ridge_value_fit(desc, nc, H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), H.dev_bf16(v_r) if m else None,
                            H.dev_f32(y), lam, v2, ws)
    torch.cuda.synchronize()
    assert torch.equal(v_c, v2)


def test_ridge_single_key_closed_form():
    """One compressed key and no retained zone: every weight is 1, so V_c = sum(Y rows) / (R + lambda)."""
    hq, hkv, d, lam = 4, 1, 128, 3.0
    print(f"case ridge_single_key: H_q={hq} d={d} lambda={lam}", flush=True)
    x = make_inputs(hq, hkv, d, 1, 1, seed=3)
    y = np.random.default_rng(5).standard_normal((hq, 1, d)).astype(np.float32)
    desc = H.desc_of(hq, hkv, d, 1, 1, False)
    ws = kvc.workspace(kvc.OP_RIDGE_FIT, desc, 1, H.DEV)
    v_c = torch.empty(hkv, 1, d, dtype=torch.float32, device=H.DEV)
    kvc.kvc_ridge_value_fit(desc, 1, H.dev_bf16(x["q"]), H.dev_bf16(x["k"]), None, H.dev_f32(y), lam, v_c, ws)
    torch.cuda.synchronize()
    assert kvc.kvc_get_device_status(ws) == 0
    want = y.astype(np.float64).reshape(-1, d).sum(axis=0) / (hq + lam)
    np.testing.assert_allclose(v_c.cpu().numpy()[0, 0], want, rtol=1e-5, atol=1e-6)


ALLROW_CASES = [
    # name, H_q, H_kv, d, N, Nq, causal
    ("allrows_causal_d128", 8, 2, 128, 777, 777, True),
    ("allrows_causal_d64", 4, 1, 64, 1000, 1000, True),
    ("rows_noncausal_d128", 4, 2, 128, 650, 97, False),
    # more than 24 row tiles per KV head (decoded-record launches), future rows that see every
    # key, and a grid of 6 (split, head) units padded to 8
    ("rows_noncausal_many_d128", 8, 2, 128, 700, 300, False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", ALLROW_CASES, ids=[c[0] for c in ALLROW_CASES])
def test_attend_every_row_mixed_widths(case):
    """The matrix-core attend on every query row of a causal layer (row blocks whose last row
    comes before a key split's groups stop early, and splits of one or a few groups), with each
    token's V width and each channel's K width drawn independently from {0, 2, 4, 8, 16}, so
    the lanes of one wave decode different widths side by side.  The layers with more than 24
    row tiles per KV head take the decode-once launches, the others the one-pass kernel."""
    name, hq, hkv, d, N, Nq, causal = case
    print(f"case {name}", flush=True)
    x = make_inputs(hq, hkv, d, N, Nq, seed=zlib.crc32(name.encode()) % 1000)
    rng = np.random.default_rng(11)
    widths = np.array([0, 2, 4, 8, 16], np.uint8)
    bv = widths[rng.integers(0, 5, size=(hkv, N))]
    bv[:, 0] = 4                                   # every row sees at least one token
    bk = widths[rng.integers(0, 5, size=(hkv, d))]
    desc = H.desc_of(hq, hkv, d, N, Nq, causal)
    cache, st = H.pack(desc, H.dev_bf16(x["k"]), H.dev_bf16(x["v"]), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    y_g, l_g, st2 = H.attend(desc, H.dev_bf16(x["q"]), cache)
    assert st2 == 0
    y_r, l_r = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk, causal=causal)
    ty, tl = H.attend_tols(x["q"], [x["k"]], [x["v"]], l_r)
    H.assert_abs(y_g.cpu().numpy(), y_r, ty, "attend output")
    H.assert_abs(l_g.cpu().numpy(), l_r, tl, "attend lse")


def _bf16_bits(vals):
    """bf16 bit patterns of float32 values that bf16 holds exactly."""
    a = np.asarray(vals, dtype=np.float32).view(np.uint32)
    assert not (a & 0xFFFF).any()
    return (a >> 16).astype(np.uint16)


# group patterns of 32 values: constant (scale 0: every code 0); a subnormal range of one bf16 ulp
# (the float32 scale is subnormal and 1/scale overflows, so every value takes the float64 decision);
# values on or next to half-integer code boundaries (round half to even, and the float64 decision
# near a boundary)
_TIE = [0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.5]
EDGE_PATTERNS = {
    "constant": _bf16_bits(np.full(32, 1.5)),
    "subnormal_range": _bf16_bits(np.tile(np.array([0.0, 2.0 ** -133], np.float32), 16)),
    "ties": _bf16_bits(np.tile(np.array(_TIE, np.float32), 4)),
    "ties_wide": _bf16_bits(np.tile(np.array([0.0, 0.5, 7.5, 14.5, 15.0, 100.5, 127.5, 255.0], np.float32), 4)),
}


@pytest.mark.parametrize("d", [128, 64])
def test_pack_edge_groups(d):
    """Quantize/pack of groups that take the quantiser's special paths, at every width and on
    both axes: V groups along the channels of a token, K groups along the tokens of a channel.
    Every packed buffer must match the oracle byte for byte."""
    hq, hkv, N = 4, 2, 256
    print(f"case pack_edge_d{d}", flush=True)
    x = make_inputs(hq, hkv, d, N, N, seed=77 + d)
    k, v = x["k"].copy(), x["v"].copy()
    pats = list(EDGE_PATTERNS.values())
    # V: token t's channel groups take the patterns in turn (the rest of the token stays random)
    for g in range(hkv):
        for t in range(0, 96):
            for j in range(d // 32):
                p = pats[(t + j) % len(pats)]
                if (t + j) % 5 != 4:
                    v[g, t, 32 * j:32 * (j + 1)] = p
    # K: channel c's first three token groups take the patterns in turn
    for g in range(hkv):
        for c in range(d):
            for grp in range(3):
                p = pats[(c + grp) % len(pats)]
                if (c + grp) % 5 != 4:
                    k[g, 32 * grp:32 * (grp + 1), c] = p
    widths = np.array([2, 4, 8, 16, 0], np.uint8)
    bv = np.stack([widths[(np.arange(N) + g) % 5] for g in range(hkv)])
    bv[:, :96] = np.array([2, 4, 8], np.uint8)[np.arange(96) % 3]     # planted tokens: quantised widths
    bk = np.stack([widths[(np.arange(d) + 2 * g) % 5] for g in range(hkv)])
    desc = H.desc_of(hq, hkv, d, N, N, True)
    cache, st = H.pack(desc, H.dev_bf16(k), H.dev_bf16(v), H.dev_u8(bv), H.dev_u8(bk))
    assert st == 0
    ref = oracle.pack_cache(k, v, bv, bk)
    H.compare_packed(cache.to_numpy(), ref)
