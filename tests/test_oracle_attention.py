"""Pins of the oracle's attention-derived quantities (CPU only).

Each check reaches the value by a route other than the oracle's own code: explicit Python
loops into scipy's logsumexp, torch's scaled_dot_product_attention in float64, the
total-variation definition of the RDKV token weight, the spectral norm of the rank-1 logit
change behind the RDKV channel weight, and brute-force loops for the KVzip+ score.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from workloads import make_inputs, bf16_bits_to_f32

CASES = [
    # H_q, H_kv, d, N, Nq, causal
    (1, 1, 8, 9, 9, True),
    (4, 2, 8, 13, 7, True),
    (3, 1, 16, 10, 4, False),
    (6, 3, 8, 17, 17, True),
]


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _visible(N, Nq, i, t, causal):
    return (not causal) or t <= N - Nq + i


@pytest.mark.parametrize("hq,hkv,d,N,Nq,causal", CASES)
def test_row_lse_matches_scipy_logsumexp(hq, hkv, d, N, Nq, causal):
    x = make_inputs(hq, hkv, d, N, Nq, seed=11)
    Q, K = _f64(x["q"]), _f64(x["k"])
    G = hq // hkv
    s = 1.0 / math.sqrt(d)
    got = oracle.row_lse(x["q"], x["k"], causal=causal)
    for h in range(hq):
        for i in range(Nq):
            logits = [s * sum(Q[h, i, c] * K[h // G, t, c] for c in range(d))
                      for t in range(N) if _visible(N, Nq, i, t, causal)]
            assert got[h, i] == pytest.approx(logsumexp(logits), rel=0, abs=1e-12)


@pytest.mark.parametrize("hq,hkv,d,N,Nq,causal", CASES)
def test_full_attention_matches_torch_sdpa(hq, hkv, d, N, Nq, causal):
    x = make_inputs(hq, hkv, d, N, Nq, seed=12)
    y, _ = oracle.full_attend(x["q"], x["k"], x["v"], causal=causal)
    G = hq // hkv
    q = torch.from_numpy(_f64(x["q"]))
    k = torch.from_numpy(_f64(x["k"])).repeat_interleave(G, dim=0)
    v = torch.from_numpy(_f64(x["v"])).repeat_interleave(G, dim=0)
    mask = torch.ones(Nq, N, dtype=torch.bool)
    if causal:
        pos = torch.arange(N - Nq, N)
        mask = torch.arange(N)[None, :] <= pos[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,d,N,Nq,causal", CASES)
def test_token_weights_sum_to_query_rows(hq, hkv, d, N, Nq, causal):
    """Each attention row sums to 1, so sum_t w[g,t] = G * Nq for every KV head."""
    x = make_inputs(hq, hkv, d, N, Nq, seed=13)
    lse = oracle.row_lse(x["q"], x["k"], causal=causal)
    w = oracle.token_scores_sum(x["q"], x["k"], lse, causal=causal)
    np.testing.assert_allclose(w.sum(axis=1), (hq // hkv) * Nq, rtol=1e-13)
    assert (w >= 0).all()


def test_token_weight_is_total_variation_of_evicting_the_token():
    """RDKV token weight: total-variation distance of each attention row after evicting t
    (and renormalising), summed over rows and the group's query heads."""
    hq, hkv, d, N, Nq = 4, 2, 8, 11, 6          # every row sees >= 6 keys
    x = make_inputs(hq, hkv, d, N, Nq, seed=14)
    Q, K = _f64(x["q"]), _f64(x["k"])
    G = hq // hkv
    s = 1.0 / math.sqrt(d)
    lse = oracle.row_lse(x["q"], x["k"])
    w = oracle.token_scores_sum(x["q"], x["k"], lse)
    for g in range(hkv):
        for t in range(N):
            tv_total = 0.0
            for h in range(g * G, (g + 1) * G):
                for i in range(Nq):
                    vis = [u for u in range(N) if u <= N - Nq + i]
                    e = {u: math.exp(s * float(Q[h, i] @ K[g, u])) for u in vis}
                    z = sum(e.values())
                    a = {u: e[u] / z for u in vis}
                    rest = [u for u in vis if u != t]
                    z2 = sum(e[u] for u in rest)
                    a2 = {u: (e[u] / z2 if u != t else 0.0) for u in vis}
                    tv_total += 0.5 * sum(abs(a[u] - a2[u]) for u in vis)
            assert w[g, t] == pytest.approx(tv_total, rel=1e-12, abs=1e-15)


def test_channel_weight_is_spectral_norm_of_zeroing_deviation():
    """RDKV channel weight: spectral norm of the logit change from zeroing channel c."""
    hq, hkv, d, N, Nq = 4, 2, 8, 12, 12
    x = make_inputs(hq, hkv, d, N, Nq, seed=15)
    Q, K = _f64(x["q"]), _f64(x["k"])
    G = hq // hkv
    s = 1.0 / math.sqrt(d)
    wc = oracle.channel_weights(x["q"], x["k"])
    for g in range(hkv):
        Qg = Q[g * G:(g + 1) * G].reshape(-1, d)
        for c in range(d):
            full = s * Qg @ K[g].T
            Qz, Kz = Qg.copy(), K[g].copy()
            Qz[:, c] = 0.0
            Kz[:, c] = 0.0
            dev = full - s * Qz @ Kz.T
            assert wc[g, c] == pytest.approx(np.linalg.norm(dev, 2), rel=1e-12)


def _brute_max_scores(Q, K, V, Hd, W, N, Nq, G, causal):
    hq, _, d = Q.shape
    hkv = K.shape[0]
    s = 1.0 / math.sqrt(d)
    hn = [math.sqrt(sum(float(c) ** 2 for c in Hd[j])) for j in range(Nq)]
    out = np.zeros((hkv, N))
    for g in range(hkv):
        for t in range(N):
            best = 0.0
            for h in range(g * G, (g + 1) * G):
                Wh = W[:, h * d:(h + 1) * d]
                won = math.sqrt(sum(float(sum(Wh[r, c] * V[g, t, c] for c in range(d))) ** 2
                                    for r in range(W.shape[0])))
                num = 0.0
                for j in range(Nq):
                    vis = [u for u in range(N) if _visible(N, Nq, j, u, causal)]
                    if t not in vis:
                        continue
                    e = [math.exp(s * float(Q[h, j] @ K[g, u])) for u in vis]
                    a = math.exp(s * float(Q[h, j] @ K[g, t])) / sum(e)
                    num = max(num, a * hn[j])
                best = max(best, num / won)
            out[g, t] = best
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_max_scores_brute_force(causal):
    hq, hkv, d, N, Nq, Dh = 4, 2, 8, 9, 5, 12
    x = make_inputs(hq, hkv, d, N, Nq, seed=16, hidden_dim=Dh)
    lse = oracle.row_lse(x["q"], x["k"], causal=causal)
    got = oracle.token_scores_max(x["q"], x["k"], lse, x["hidden"], x["w_o"], x["v"], causal=causal)
    ref = _brute_max_scores(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), _f64(x["hidden"]),
                            _f64(x["w_o"]), N, Nq, hq // hkv, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-12)


def test_max_scores_scale_laws():
    """Scaling W_O by alpha divides s+ by alpha; scaling the hidden states multiplies it."""
    hq, hkv, d, N, Nq, Dh = 4, 2, 16, 20, 20, 24
    x = make_inputs(hq, hkv, d, N, Nq, seed=17, hidden_dim=Dh)
    q, k, v = _f64(x["q"]), _f64(x["k"]), _f64(x["v"])
    hid, wo = _f64(x["hidden"]), _f64(x["w_o"])
    lse = oracle.row_lse(q, k)
    base = oracle.token_scores_max(q, k, lse, hid, wo, v)
    np.testing.assert_allclose(oracle.token_scores_max(q, k, lse, hid, 3.0 * wo, v), base / 3.0,
                               rtol=1e-13)
    np.testing.assert_allclose(oracle.token_scores_max(q, k, lse, 0.5 * hid, wo, v), base * 0.5,
                               rtol=1e-13)


def test_scale_argument_is_used():
    x = make_inputs(2, 1, 8, 10, 10, seed=18)
    a = oracle.row_lse(x["q"], x["k"], scale=0.25)
    q2 = _f64(x["q"]) * (0.25 * math.sqrt(8))         # fold the scale into q
    b = oracle.row_lse(q2, x["k"])
    np.testing.assert_allclose(a, b, rtol=1e-13)
