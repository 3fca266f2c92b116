"""Attention-derived quantities: row log-sum-exp, token scores, channel weights.

Test infrastructure only (see the package docstring).

Shapes: Q [H_q][Nq][d], K and V [H_kv][N][d], hidden [Nq][D_h], W_O [D_h][H_q*d].
Query head h reads KV head g(h) = h // G with G = H_q / H_kv (consecutive grouping).
"""

import numpy as np

from .common import as_f64, default_scale, visible_mask

_ROWS = 512   # query rows per logits chunk (memory only; no effect on the arithmetic order of a row)


def _logits(q_rows, k_head, scale, vis):
    """s * q k^T for a block of rows, -inf where the key is not visible."""
    s = scale * (q_rows @ k_head.T)
    s[~vis] = -np.inf
    return s


def _row_logsumexp(s):
    """ln sum_t exp(s_t) per row; -inf for a row with no visible key."""
    m = s.max(axis=1)
    out = np.full(s.shape[0], -np.inf)
    ok = np.isfinite(m)
    if ok.any():
        mm = m[ok]
        out[ok] = mm + np.log(np.exp(s[ok] - mm[:, None]).sum(axis=1))
    return out


def row_lse(q, k, scale=None, causal=True):
    """Row log-sum-exp of the scaled, causally masked logits, per query head and row.

    l_{h,i} = ln sum_{t <= p_i} exp(s q_{h,i} . k_{g(h),t}), natural log, scale included.
    This is the "attention mass" whose match KVSculpt adds to its loss (KVSculpt summary,
    §2, LSE term) and the normaliser of the attention probabilities a_{tau,t} that RDKV's
    token weight sums (RDKV summary, §2.1).
    """
    Q, K = as_f64(q), as_f64(k)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    sc = default_scale(d, scale)
    out = np.empty((hq, nq))
    for h in range(hq):
        kh = K[h // G]
        for r0 in range(0, nq, _ROWS):
            r1 = min(nq, r0 + _ROWS)
            vis = visible_mask(n, nq, r0, r1, causal)
            out[h, r0:r1] = _row_logsumexp(_logits(Q[h, r0:r1], kh, sc, vis))
    return out


def _probabilities(Q, K, lse, h, G, r0, r1, sc, causal):
    n = K.shape[1]
    nq = Q.shape[1]
    vis = visible_mask(n, nq, r0, r1, causal)
    s = _logits(Q[h, r0:r1], K[h // G], sc, vis)
    return np.exp(s - lse[h, r0:r1, None])          # masked entries: exp(-inf) = 0


def token_scores_sum(q, k, lse, scale=None, causal=True):
    """RDKV token distortion weight, summed over the query heads of each KV group.

    w[g,t] = sum_{h: g(h)=g} sum_{i: p_i >= t} a_{h,i,t},  a = exp(s q.k - l).
    RDKV summary, §2.1: the weight of a V token is the total attention it receives over all
    query positions.  Under GQA the pages give a single-head formula; the group's query heads
    are summed (the reading taken for the grouped layouts).
    """
    Q, K = as_f64(q), as_f64(k)
    L = np.asarray(lse, dtype=np.float64)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    sc = default_scale(d, scale)
    w = np.zeros((hkv, n))
    for h in range(hq):
        for r0 in range(0, nq, _ROWS):
            r1 = min(nq, r0 + _ROWS)
            w[h // G] += _probabilities(Q, K, L, h, G, r0, r1, sc, causal).sum(axis=0)
    return w


def hidden_row_norms(hidden):
    """||h_j||_2 of every query row's hidden state (KVzap summary, §2.1)."""
    H = as_f64(hidden)
    return np.sqrt((H * H).sum(axis=1))


def value_out_norms(w_o, v, n_q_heads, tokens=None):
    """||W_O^{(h)} v_{g(h),t}||_2 for every query head h and token t (or a token subset).

    W_O is the output projection stored as a Linear weight [D_h][H_q*d]; head h's slice is its
    d input columns [h*d, (h+1)*d).  The product is formed directly, as the definition reads
    (KVzap summary, §2.1: the value vector's contribution to the residual stream).
    """
    W = as_f64(w_o)
    V = as_f64(v)
    hkv, n, d = V.shape
    G = n_q_heads // hkv
    idx = np.arange(n) if tokens is None else np.asarray(tokens)
    out = np.empty((n_q_heads, len(idx)))
    for h in range(n_q_heads):
        Wh = W[:, h * d:(h + 1) * d]                   # [D_h][d]
        U = V[h // G][idx] @ Wh.T                      # [tokens][D_h]
        out[h] = np.sqrt((U * U).sum(axis=1))
    return out


def token_scores_max(q, k, lse, hidden, w_o, v, scale=None, causal=True, tokens=None):
    """KVzip+ score, maximised over the query heads of each KV group.

    s+[g,t] = max_{h: g(h)=g} ( max_{j: p_j >= t} a_{h,j,t} * ||h_j|| ) / ||W_O^{(h)} v_{g,t}||.
    KVzap summary, §2.1 (the score: the largest attention a token receives over the prompt,
    normalised by its value's output-projection norm relative to the hidden-state norm) and
    §2.2 (one score per KV head).  The j range is the visible query rows (self included);
    the group reduction is a max.  A zero value norm gives +inf (0 if the numerator is 0).
    ``tokens`` restricts the output to those columns (same values, fewer columns computed).
    """
    Q, K = as_f64(q), as_f64(k)
    L = np.asarray(lse, dtype=np.float64)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    sc = default_scale(d, scale)
    cols = np.arange(n) if tokens is None else np.asarray(tokens)
    hn = hidden_row_norms(hidden)
    won = value_out_norms(w_o, v, hq, cols)
    num = np.zeros((hq, cols.size))
    for h in range(hq):
        for r0 in range(0, nq, _ROWS):
            r1 = min(nq, r0 + _ROWS)
            a = _probabilities(Q, K, L, h, G, r0, r1, sc, causal)[:, cols]
            num[h] = np.maximum(num[h], (a * hn[r0:r1, None]).max(axis=0))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = num / won
    ratio[(num == 0) & (won == 0)] = 0.0
    return ratio.reshape(hkv, G, cols.size).max(axis=1)


def channel_weights(q, k, scale=None):
    """RDKV K-channel distortion weight w_c[g,c] = s ||Q_g[:,c]||_2 ||K_g[:,c]||_2.

    RDKV summary, §2.1: the spectral norm of the logit change caused by zeroing channel c,
    which is the product of the channel's query and key column norms scaled by 1/sqrt(d).
    Q_g stacks all rows of all query heads of group g; K_g is the whole cache of head g
    (computed once on the full uncompressed cache, RDKV summary §2.2 stage 1).
    """
    Q, K = as_f64(q), as_f64(k)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    sc = default_scale(d, scale)
    out = np.empty((hkv, d))
    for g in range(hkv):
        Qg = Q[g * G:(g + 1) * G].reshape(-1, d)
        out[g] = sc * np.sqrt((Qg * Qg).sum(axis=0)) * np.sqrt((K[g] * K[g]).sum(axis=0))
    return out
