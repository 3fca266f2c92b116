"""Helpers for the GPU parity tests: run each C-ABI call on device tensors and bring the
results back as numpy.  Every computation here happens in libkvc's kernels."""

import numpy as np
import torch

import kv_cache_compression_pass_amd as kvc

DEV = "cuda:0"


def dev_bf16(bits):
    return kvc.bf16_tensor(bits, DEV)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def desc_of(hq, hkv, d, N, Nq, causal=True, scale=0.0):
    return kvc.make_desc(hq, hkv, d, N, Nq, causal, scale)


def row_lse(desc, q, k):
    lse = torch.empty(desc.n_q_heads, desc.n_queries, dtype=torch.float32, device=DEV)
    kvc.kvc_row_lse(desc, q, k, lse, kvc.workspace(kvc.OP_ROW_LSE, desc, 0, DEV))
    torch.cuda.synchronize()
    return lse


def score_sum(desc, q, k, lse):
    ws = kvc.workspace(kvc.OP_SCORE_TOKENS, desc, kvc.SCORE_SUM, DEV)
    out = torch.empty(desc.n_kv_heads, desc.n_keys, dtype=torch.float32, device=DEV)
    kvc.kvc_score_tokens(desc, kvc.SCORE_SUM, q, k, lse, out, ws)
    torch.cuda.synchronize()
    return out


def score_max(desc, q, k, lse, hidden, w_o, v):
    ws = kvc.workspace(kvc.OP_SCORE_TOKENS, desc, kvc.SCORE_MAX, DEV)
    out = torch.empty(desc.n_kv_heads, desc.n_keys, dtype=torch.float32, device=DEV)
    kvc.kvc_score_tokens(desc, kvc.SCORE_MAX, q, k, lse, out, ws, hidden=hidden, w_o=w_o, v=v,
                         hidden_dim=hidden.shape[-1])
    torch.cuda.synchronize()
    return out


def channel_weights(desc, q, k):
    ws = kvc.workspace(kvc.OP_CHANNEL_WEIGHTS, desc, 0, DEV)
    out = torch.empty(desc.n_kv_heads, desc.head_dim, dtype=torch.float32, device=DEV)
    kvc.kvc_channel_weights(desc, q, k, out, ws)
    torch.cuda.synchronize()
    return out


def allocate(desc, stage, weight, avg=0.0, bits_v=None, sigma=None, keep_fraction=0.0,
             keep_bits=16):
    ws = kvc.workspace(kvc.OP_ALLOCATE_BITS, desc, stage, DEV)
    out = torch.empty(weight.shape, dtype=torch.uint8, device=DEV)
    res = kvc.alloc_result_buffer(DEV)
    kvc.kvc_allocate_bits(desc, stage, weight, out, ws, sigma=sigma, bits_v=bits_v, avg_bits=avg,
                          keep_fraction=keep_fraction, keep_bits=keep_bits, result=res)
    torch.cuda.synchronize()
    status = kvc.kvc_get_device_status(ws)
    return out, kvc.decode_alloc_result(res), status


def pack(desc, k, v, bits_v, bits_k):
    ws = kvc.workspace(kvc.OP_QUANTIZE_PACK, desc, 0, DEV)
    cache = kvc.PackedCache(desc, DEV)
    kvc.kvc_quantize_pack(desc, k, v, bits_v, bits_k, cache, ws)
    torch.cuda.synchronize()
    return cache, kvc.kvc_get_device_status(ws)


def attend(desc_f, q_f, cache):
    ws = kvc.workspace(kvc.OP_COMPRESSED_ATTEND, desc_f, 0, DEV)
    out = torch.empty(desc_f.n_q_heads, desc_f.n_queries, desc_f.head_dim, dtype=torch.float32,
                      device=DEV)
    lse = torch.empty(desc_f.n_q_heads, desc_f.n_queries, dtype=torch.float32, device=DEV)
    kvc.kvc_compressed_attend(desc_f, q_f, cache, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse, kvc.kvc_get_device_status(ws)


def rel_ok(got, want, rel, floor=1e-30):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return np.abs(got - want) <= rel * np.abs(want) + floor


def assert_rel(got, want, rel, floor=1e-30, what=""):
    ok = rel_ok(got, want, rel, floor)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        g = np.asarray(got)
        w = np.asarray(want)
        detail = "; ".join(f"{tuple(i)}: got {g[tuple(i)]!r} want {w[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside rel {rel}: {detail}")


def assert_abs(got, want, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(want)
    diff = np.where(both_inf, 0.0, np.abs(got - want))
    bad = ~(diff <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = "; ".join(f"{tuple(i)}: got {got[tuple(i)]!r} want {want[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside abs {tol}: {detail}")


def compare_packed(gpu, ref):
    """Bit-exact comparison of every packed buffer (trimmed to the used lengths)."""
    for name in ("header", "v_idx", "v_words", "v_par", "k_keep", "k_vloc", "k_words", "k_par",
                 "k_width"):
        g = np.asarray(gpu[name])
        r = np.asarray(ref[name])
        assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
        if g.dtype.kind == "f":
            eq = g.view(np.uint32) == r.astype(g.dtype).view(np.uint32)
        else:
            eq = g == r.astype(g.dtype)
        if not np.all(eq):
            bad = np.argwhere(~eq)[:5]
            raise AssertionError(f"{name}: {int((~eq).sum())} mismatches, first at {bad.tolist()}")


def attend_tols(q_bits, k_bits_list, v_bits_list, lse_ref, scale=None, capped=True):
    """Bounds on |Y_hat - Y_ref| and |l_hat - l_ref| for the attend calls: the stated bars
    (2e-2 and 1e-3 abs), tightened to what the arithmetic allows for the test's own inputs.

    Logits: the keys enter the products as bf16 hi + lo (exact to 2^-17 relative) and the d
    products are summed in fp32 (at most d 2^-24 relative to sum |q_c k_c|), and sum |q_c k_c|
    <= ||q|| ||k_hat|| with |k_hat_c| <= max_t |k_tc| (a dequantised value stays inside its
    group's range), so dl = (2^-17 + d 2^-24) max||q|| kcap scale bounds a logit's error and,
    the LSE being a smooth maximum, the LSE's; the base-2 to natural conversion adds a few
    float32 roundings of |l|.  Outputs: V_hat and the probabilities enter the matrix products
    as fp16 (2^-11 relative each; the probabilities of a row sum to 1 and |V_hat| <= max|V|),
    one more such term covers the fp32 sums, and a logit error dl moves each probability by at
    most a factor e^dl, i.e. the output by about 2 dl max|V|."""
    from workloads import bf16_bits_to_f32
    q = bf16_bits_to_f32(np.asarray(q_bits)).astype(np.float64)
    d = q.shape[-1]
    s = scale if scale else 1.0 / np.sqrt(d)
    qn = float(np.sqrt((q * q).sum(-1)).max()) if q.size else 0.0
    kcap = 0.0
    for kb in k_bits_list:
        k = bf16_bits_to_f32(np.asarray(kb)).astype(np.float64)
        if k.size:
            kcap = max(kcap, float(np.sqrt((np.abs(k).max(axis=-2) ** 2).sum(-1)).max()))
    vmax = 0.0
    for vb in v_bits_list:
        v = np.asarray(vb)
        if v.size:
            vmax = max(vmax, float(np.abs(bf16_bits_to_f32(v)).max()))
    dl = (2.0 ** -17 + d * 2.0 ** -24) * qn * kcap * s
    lr = np.asarray(lse_ref, dtype=np.float64)
    lmax = float(np.abs(lr[np.isfinite(lr)]).max()) if np.isfinite(lr).any() else 0.0
    ty = (3 * 2.0 ** -11 + 2 * dl) * vmax
    tl = dl + 4 * 2.0 ** -24 * lmax + 1e-6
    if not capped:
        # values of any magnitude: the output bound scales with max|V| (floor included)
        return ty + 1e-6 * vmax, tl
    # never looser than the stated bars (output 2e-2 abs, LSE 1e-3 abs)
    return min(ty + 1e-5, 2e-2), min(tl, 1e-3)
