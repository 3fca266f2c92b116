"""Pins of the oracle's compressed-cache attention (CPU only).

* 16-bit widths with no eviction reproduce full attention exactly (and full attention is
  itself pinned to torch's SDPA in test_oracle_attention).
* Eviction only (every kept unit at 16 bits): exp(l_hat - l) = 1 - sum of the evicted
  visible probabilities, and Y_hat = (Y - sum_evicted a_t v_t) / (1 - sum_evicted a_t),
  with the probabilities computed here by an explicit softmax.
* V-only quantisation: every output moves by at most the largest half step s/2, because
  attention output is a convex combination of the value rows.
* A row whose visible tokens are all evicted gets l_hat = -inf and Y_hat = 0.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import make_inputs, bf16_bits_to_f32


def _f64(b):
    return bf16_bits_to_f32(b).astype(np.float64)


@pytest.mark.parametrize("causal", [True, False])
def test_all_sixteen_no_eviction_is_full_attention(causal):
    hq, hkv, d, N, Nq = 4, 2, 64, 45, 20
    x = make_inputs(hq, hkv, d, N, Nq, seed=21)
    bv = np.full((hkv, N), 16, np.uint8)
    bk = np.full((hkv, d), 16, np.uint8)
    y, l = oracle.full_attend(x["q"], x["k"], x["v"], causal=causal)
    yh, lh = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk, causal=causal)
    assert np.array_equal(y, yh) and np.array_equal(l, lh)
    assert oracle.fidelity_terms(yh, y, lh, l) == (0.0, 0.0)
    np.testing.assert_allclose(l, oracle.row_lse(x["q"], x["k"], causal=causal), rtol=0, atol=1e-12)


def test_eviction_only_identities():
    hq, hkv, d, N, Nq = 4, 2, 32, 30, 10
    x = make_inputs(hq, hkv, d, N, Nq, seed=22)
    rng = np.random.default_rng(3)
    bv = np.where(rng.random((hkv, N)) < 0.4, 0, 16).astype(np.uint8)
    bv[:, N - Nq:] = 16                      # keep the diagonal so no row is empty
    bk = np.full((hkv, d), 16, np.uint8)
    y, l = oracle.full_attend(x["q"], x["k"], x["v"])
    yh, lh = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk)
    Q, K, V = _f64(x["q"]), _f64(x["k"]), _f64(x["v"])
    G = hq // hkv
    for h in range(hq):
        g = h // G
        for i in range(Nq):
            vis = np.arange(N - Nq + i + 1)
            logit = (Q[h, i] @ K[g, vis].T) / math.sqrt(d)
            a = np.exp(logit - logit.max())
            a /= a.sum()
            ev = bv[g, vis] == 0
            mass = a[ev].sum()
            assert math.exp(lh[h, i] - l[h, i]) == pytest.approx(1.0 - mass, rel=1e-12)
            want = (y[h, i] - (a[ev, None] * V[g, vis[ev]]).sum(axis=0)) / (1.0 - mass)
            np.testing.assert_allclose(yh[h, i], want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_value_only_quantization_bound(b):
    hq, hkv, d, N, Nq = 2, 1, 64, 40, 16
    x = make_inputs(hq, hkv, d, N, Nq, seed=23)
    bv = np.full((hkv, N), b, np.uint8)
    bk = np.full((hkv, d), 16, np.uint8)
    y, l = oracle.full_attend(x["q"], x["k"], x["v"])
    yh, lh = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk)
    np.testing.assert_array_equal(l, lh)             # K untouched: same logits
    V = _f64(x["v"])[0].reshape(N, d // 32, 32)
    half_step = ((V.max(axis=2) - V.min(axis=2)) / (2 ** b - 1)).max() / 2
    assert np.abs(yh - y).max() <= half_step * (1 + 1e-6)


def test_empty_row_gives_minus_inf_and_zero():
    hq, hkv, d, N, Nq = 1, 1, 32, 12, 12
    x = make_inputs(hq, hkv, d, N, Nq, seed=24)
    bv = np.full((hkv, N), 16, np.uint8)
    bv[0, :3] = 0                             # rows 0..2 see only tokens 0..2
    bk = np.full((hkv, d), 16, np.uint8)
    yh, lh = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk)
    assert np.all(np.isneginf(lh[0, :3])) and np.all(yh[0, :3] == 0)
    assert np.all(np.isfinite(lh[0, 3:]))


def test_key_channel_width_zero_drops_the_channel():
    hq, hkv, d, N, Nq = 2, 1, 32, 16, 16
    x = make_inputs(hq, hkv, d, N, Nq, seed=25)
    bv = np.full((hkv, N), 16, np.uint8)
    bk = np.full((hkv, d), 16, np.uint8)
    bk[0, 5] = 0
    yh, lh = oracle.compressed_attend(x["q"], x["k"], x["v"], bv, bk)
    Q = _f64(x["q"]).copy()
    Q[:, :, 5] = 0.0                          # zeroing k's channel == zeroing q's channel
    y2, l2 = oracle.full_attend(Q, x["k"], x["v"])
    np.testing.assert_allclose(yh, y2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lh, l2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_append_buffer_all_sixteen_is_full_attention(causal):
    """An all-16, no-eviction cache followed by the append buffer is full attention over the
    concatenated raw keys and values (rows are the last Nq of the N + n_new positions)."""
    hq, hkv, d, N, n_new, Nq = 4, 2, 64, 40, 7, 5
    x = make_inputs(hq, hkv, d, N + n_new, N + n_new, seed=31)
    k, v = x["k"][:, :N], x["v"][:, :N]
    kn, vn = x["k"][:, N:], x["v"][:, N:]
    q = x["q"][:, -Nq:]
    bv = np.full((hkv, N), 16, np.uint8)
    bk = np.full((hkv, d), 16, np.uint8)
    y, l = oracle.compressed_attend_append(q, k, v, bv, bk, kn, vn, causal=causal)
    yr, lr = oracle.full_attend(q, x["k"], x["v"], causal=causal)
    np.testing.assert_allclose(y, yr, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lr, rtol=0, atol=1e-12)


def test_append_buffer_is_the_lse_merge_of_the_two_zones():
    """For a decode row (it sees every cached and every new token) the result is the
    log-sum-exp merge of attention over the compressed cache alone and over the buffer
    alone: l = logaddexp(l1, l2), Y = e^(l1 - l) Y1 + e^(l2 - l) Y2."""
    hq, hkv, d, N, n_new = 6, 2, 32, 70, 9
    x = make_inputs(hq, hkv, d, N + n_new, N + n_new, seed=32)
    rng = np.random.default_rng(3)
    bv = rng.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(hkv, N)).astype(np.uint8)
    bk = rng.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(hkv, d)).astype(np.uint8)
    k, v, kn, vn = x["k"][:, :N], x["v"][:, :N], x["k"][:, N:], x["v"][:, N:]
    q = x["q"][:, -1:]
    y, l = oracle.compressed_attend_append(q, k, v, bv, bk, kn, vn, causal=True)
    y1, l1 = oracle.compressed_attend(q, k, v, bv, bk, causal=False)
    y2, l2 = oracle.full_attend(q, kn, vn, causal=False)
    lm = np.logaddexp(l1, l2)
    ym = np.exp(l1 - lm)[..., None] * y1 + np.exp(l2 - lm)[..., None] * y2
    np.testing.assert_allclose(l, lm, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y, ym, rtol=0, atol=1e-12)


def test_append_buffer_empty_is_the_cache_alone():
    hq, hkv, d, N, Nq = 4, 1, 32, 50, 3
    x = make_inputs(hq, hkv, d, N, N, seed=33)
    bv = np.full((hkv, N), 4, np.uint8)
    bv[:, ::3] = 0
    bk = np.full((hkv, d), 8, np.uint8)
    q = x["q"][:, -Nq:]
    empty = np.zeros((hkv, 0, d), np.uint16)
    y, l = oracle.compressed_attend_append(q, x["k"], x["v"], bv, bk, empty, empty, causal=True)
    yc, lc = oracle.compressed_attend(q, x["k"], x["v"], bv, bk, causal=True)
    assert np.array_equal(y, yc) and np.array_equal(l, lc)


def test_fidelity_terms_per_head_closed_forms():
    rng = np.random.default_rng(4)
    hq, nq, d = 3, 5, 8
    y = rng.standard_normal((hq, nq, d))
    l = rng.standard_normal((hq, nq))
    c = np.array([0.5, -2.0, 0.0])
    yh = y + c[:, None, None]                                     # a constant offset per head
    lh = l + np.array([1.0, 0.0, 3.0])[:, None]
    t = oracle.fidelity_terms_per_head(yh, y, lh, l)
    np.testing.assert_allclose(t[:, 0], nq * d * c ** 2, rtol=1e-12)
    np.testing.assert_allclose(t[:, 1], nq * np.array([1.0, 0.0, 9.0]), rtol=1e-12)
    tot = oracle.fidelity_terms(yh, y, lh, l)
    assert t[:, 0].sum() == pytest.approx(tot[0], rel=1e-12) and t[:, 1].sum() == pytest.approx(tot[1], rel=1e-12)
    # rows empty in both caches add 0; empty in one only adds +inf
    l2, lh2 = l.copy(), lh.copy()
    l2[0, 1] = lh2[0, 1] = -np.inf
    assert np.isfinite(oracle.fidelity_terms_per_head(yh, y, lh2, l2)[0, 1])
    lh2[1, 2] = -np.inf
    assert np.isinf(oracle.fidelity_terms_per_head(yh, y, lh2, l2)[1, 1])
