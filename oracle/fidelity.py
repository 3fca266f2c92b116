"""Attention over the compressed cache, and the fidelity terms against the full cache.

Test infrastructure only (see the package docstring).

KVSculpt summary, §2 (loss): a compressed cache is judged by the squared Frobenius error of
the attention output, ||Y_hat - Y||_F^2, and of the row log-sum-exp, ||l_hat - l||_F^2.
RDKV summary, §2.3: decode attention runs straight over the packed zones with the
dequantisation fused in.  Here the definition is written out plainly: dequantise the
retained units to float64 (x_hat = zero + scale * code; a channel of width 0 is 0; width 16
is the bf16 value itself) and run masked softmax attention over the retained tokens only.
"""

import numpy as np

from .common import as_f64, default_scale, query_positions
from .quantize import quantize_group


def dequantized_head(k_head, v_head, bits_v_head, bits_k_head, group_size=32):
    """Dequantised K_hat, V_hat (float64) of one KV head's retained tokens.

    Returns (tokens int64 [R], k_hat [R][d], v_hat [R][d]).
    """
    if group_size != 32:
        raise ValueError("group size 32 only")
    bv = np.asarray(bits_v_head)
    bk = np.asarray(bits_k_head)
    kept = np.nonzero(bv > 0)[0]
    K = as_f64(k_head)[kept]
    V = as_f64(v_head)[kept]
    R, d = K.shape
    v_hat = np.zeros((R, d))
    bvk = bv[kept]
    for b in (2, 4, 8, 16):                 # every 32-channel group of every token at width b
        rows = np.nonzero(bvk == b)[0]
        if rows.size == 0:
            continue
        x = V[rows].reshape(-1, 32)
        if b == 16:
            v_hat[rows] = x.reshape(rows.size, d)
        else:
            codes, s, z = quantize_group(x, b)
            xh = z.astype(np.float64)[:, None] + s.astype(np.float64)[:, None] * codes
            v_hat[rows] = xh.reshape(rows.size, d)
    k_hat = np.zeros((R, d))
    nfull = R // 32
    for c in range(d):                      # 32 consecutive retained tokens per group
        b = int(bk[c])
        if b == 0:
            continue
        if b == 16:
            k_hat[:, c] = K[:, c]
            continue
        for j0, x in ((0, K[:32 * nfull, c].reshape(nfull, 32)), (32 * nfull, K[32 * nfull:, c][None, :])):
            if x.size == 0:
                continue
            codes, s, z = quantize_group(x, b)
            xh = z.astype(np.float64)[:, None] + s.astype(np.float64)[:, None] * codes
            k_hat[j0:j0 + xh.size, c] = xh.reshape(-1)
    return kept, k_hat, v_hat


def attend(q, heads, n_keys, scale=None, causal=True):
    """Masked softmax attention of Q over per-KV-head (tokens, K, V) lists.

    q: [H_q][Nq][d]; heads: list over KV heads of (token positions, K [R][d], V [R][d]).
    Query row i sits at position N - Nq + i and sees token t iff t <= that position.
    Returns (out [H_q][Nq][d], lse [H_q][Nq]); a row with no visible token gets
    lse = -inf and out = 0.
    """
    Q = as_f64(q)
    hq, nq, d = Q.shape
    hkv = len(heads)
    G = hq // hkv
    sc = default_scale(d, scale)
    pos = query_positions(n_keys, nq)
    out = np.zeros((hq, nq, d))
    lse = np.full((hq, nq), -np.inf)
    for h in range(hq):
        toks, Kh, Vh = heads[h // G]
        if len(toks) == 0:
            continue
        S = sc * (Q[h] @ Kh.T)                                  # [Nq][R]
        if causal:
            S[np.asarray(toks)[None, :] > pos[:, None]] = -np.inf
        m = S.max(axis=1)
        ok = np.isfinite(m)
        P = np.zeros_like(S)
        P[ok] = np.exp(S[ok] - m[ok, None])
        den = P.sum(axis=1)
        lse[h, ok] = m[ok] + np.log(den[ok])
        out[h, ok] = (P[ok] @ Vh) / den[ok, None]
    return out, lse


def full_attend(q, k, v, scale=None, causal=True):
    """Attention over the whole uncompressed cache (every token, exact bf16 K and V)."""
    K, V = as_f64(k), as_f64(v)
    hkv, n, d = K.shape
    heads = [(np.arange(n), K[g], V[g]) for g in range(hkv)]
    return attend(q, heads, n, scale, causal)


def compressed_attend(q, k, v, bits_v, bits_k, scale=None, causal=True, group_size=32):
    """Attention over the compressed cache defined by the widths bits_v, bits_k."""
    K = np.asarray(k)
    hkv, n, d = K.shape
    heads = [dequantized_head(K[g], np.asarray(v)[g], np.asarray(bits_v)[g],
                              np.asarray(bits_k)[g], group_size) for g in range(hkv)]
    return attend(q, heads, n, scale, causal)


def compressed_attend_append(q, k, v, bits_v, bits_k, k_new, v_new, scale=None, causal=True, group_size=32):
    """Attention over the compressed cache followed by an uncompressed append buffer.

    RDKV summary, §2.3: decode reads the packed width zones of the compressed cache, and the
    tokens generated since compression sit beside them in full precision; attention spans
    both.  Here that is written out plainly: the retained, dequantised tokens of the cache
    (positions < N) and the new tokens k_new, v_new [H_kv][n_new][d] at positions N .. N+n_new-1
    form one token list per KV head, and the query rows are the last Nq positions of the
    N + n_new.  Reading: the buffer holds the raw bf16 values (no quantisation), and the rows'
    positions count the new tokens.
    """
    K = np.asarray(k)
    hkv, n, d = K.shape
    kn, vn = as_f64(k_new), as_f64(v_new)
    n_new = kn.shape[1]
    heads = []
    for g in range(hkv):
        toks, kh, vh = dequantized_head(K[g], np.asarray(v)[g], np.asarray(bits_v)[g],
                                        np.asarray(bits_k)[g], group_size)
        heads.append((np.concatenate([toks, n + np.arange(n_new)]),
                      np.concatenate([kh, kn[g]]), np.concatenate([vh, vn[g]])))
    return attend(q, heads, n + n_new, scale, causal)


def fidelity_terms(y_hat, y, lse_hat, lse):
    """(||Y_hat - Y||_F^2, ||l_hat - l||_F^2), the two terms of KVSculpt's loss (§2)."""
    dy = np.asarray(y_hat, dtype=np.float64) - np.asarray(y, dtype=np.float64)
    dl = np.asarray(lse_hat, dtype=np.float64) - np.asarray(lse, dtype=np.float64)
    return float((dy * dy).sum()), float((dl * dl).sum())


def fidelity_terms_per_head(y_hat, y, lse_hat, lse):
    """Per query head h: (sum over rows and channels of (Y_hat - Y)^2, sum over rows of
    (l_hat - l)^2), the two terms of KVSculpt's loss (§2) split by head.  Reading: a row with
    no visible token in both caches (l_hat = l = -inf, outputs 0) contributes 0 to the LSE
    term; one empty and one not contributes +inf.
    """
    dy = np.asarray(y_hat, dtype=np.float64) - np.asarray(y, dtype=np.float64)
    lh = np.asarray(lse_hat, dtype=np.float64)
    lr = np.asarray(lse, dtype=np.float64)
    hq = dy.shape[0]
    out = np.zeros((hq, 2))
    for h in range(hq):
        out[h, 0] = float((dy[h] * dy[h]).sum())
        acc = 0.0
        for a, b in zip(lh[h].ravel(), lr[h].ravel()):
            if a == b:                       # equal values, both -inf included
                continue
            acc += (a - b) ** 2
        out[h, 1] = acc
    return out
