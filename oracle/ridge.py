"""KVSculpt's value solve: with the compressed keys fixed, the values that best reproduce the
full-cache attention output, in closed form (ridge least squares).

Test infrastructure only (see the package docstring).

KVSculpt summary, §2 (alternating optimisation, value step; §4 uses the same fit after a
selection, "Select+Fit").  The compressed cache is n_c free pairs (K_c, V_c) followed by the m
most recent tokens kept as they are (K_r, V_r).  With the keys fixed, the attention weights
A = softmax(s Q [K_c; K_r]^T) do not depend on the values, so the output
Y_hat = A_c V_c + A_r V_r is linear in V_c, and the V_c that minimises
||Y_hat - Y||_F^2 + lam ||V_c||_F^2 solves the normal equations

    (A_c^T A_c + lam I) V_c = A_c^T (Y - A_r V_r).

Readings (the page gives the method, not these details): the G query heads of a KV head share
its V_c, so their rows are stacked into one least-squares problem; lam is absolute (added to
the diagonal); the query rows follow the layer convention (bottom-right causal alignment over
the n_c + m keys, or no mask).
"""

import numpy as np

from .common import as_f64, default_scale, visible_mask


def _weights(q_head, k_head, scale, vis):
    """Softmax attention weights of one query head over one KV head's keys (0 where masked)."""
    s = scale * (q_head @ k_head.T)
    s[~vis] = -np.inf
    m = s.max(axis=1, keepdims=True)
    ok = np.isfinite(m[:, 0])
    a = np.zeros_like(s)
    e = np.exp(s[ok] - m[ok])
    a[ok] = e / e.sum(axis=1, keepdims=True)
    return a


def ridge_system(q, k, v_r, y, n_compressed, scale=None, causal=False):
    """Per KV head g: (A_c, A_r, T) with the rows of the group's G query heads stacked in head
    order: the attention weights on the n_c compressed keys [R][n_c] and on the m retained keys
    [R][m], and the target the compressed part must reproduce, T = Y - A_r V_r [R][d].

    q: bf16 bits [H_q][Nq][d]; k: bf16 bits [H_kv][n_c + m][d] (compressed keys first);
    v_r: bf16 bits [H_kv][m][d] (ignored when m = 0); y: [H_q][Nq][d] target outputs.
    """
    Q, K = as_f64(q), as_f64(k)
    Y = np.asarray(y, dtype=np.float64)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    nc = int(n_compressed)
    if not 1 <= nc <= n:
        raise ValueError("need 1 <= n_compressed <= n_keys")
    m = n - nc
    Vr = as_f64(v_r) if m > 0 else np.zeros((hkv, 0, d))
    sc = default_scale(d, scale)
    vis = visible_mask(n, nq, 0, nq, causal)
    out = []
    for g in range(hkv):
        Ac, Ar, T = [], [], []
        for h in range(g * G, (g + 1) * G):
            a = _weights(Q[h], K[g], sc, vis)
            Ac.append(a[:, :nc])
            Ar.append(a[:, nc:])
            T.append(Y[h] - a[:, nc:] @ Vr[g])
        out.append((np.vstack(Ac), np.vstack(Ar), np.vstack(T)))
    return out


def ridge_normal_equations(q, k, v_r, y, n_compressed, lam, scale=None, causal=False):
    """Per KV head g: (M_g, B_g) with M = A_c^T A_c + lam I [n_c][n_c] and
    B = A_c^T (Y - A_r V_r) [n_c][d], from the stacked system of ridge_system.
    """
    Ms, Bs = [], []
    for Ac, _, T in ridge_system(q, k, v_r, y, n_compressed, scale, causal):
        Ms.append(Ac.T @ Ac + float(lam) * np.eye(Ac.shape[1]))
        Bs.append(Ac.T @ T)
    return Ms, Bs


def ridge_value_fit(q, k, v_r, y, n_compressed, lam, scale=None, causal=False):
    """V_c [H_kv][n_c][d] (float64) solving each head's normal equations (see the module
    docstring); the solve is numpy's LU solve of the symmetric system."""
    Ms, Bs = ridge_normal_equations(q, k, v_r, y, n_compressed, lam, scale, causal)
    return np.stack([np.linalg.solve(M, B) for M, B in zip(Ms, Bs)])
