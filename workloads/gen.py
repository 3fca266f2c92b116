"""Seeded input generation.

Recipe (identical for every consumer):

* ``numpy.random.default_rng(seed)`` (PCG64); for the named configs ``seed = 1234 + index``.
* Draw order: Q, K, V, then the outlier channel choice, then hidden states, then W_O.
* Each tensor is ``standard_normal(dtype=float32)``, transformed in float32, then rounded to
  bfloat16 with round-to-nearest-even and stored as ``uint16`` bit patterns.

All arrays are plain numpy ``uint16`` (bf16 bits) in the layouts the library uses:
Q ``[H_q][Nq][d]``, K and V ``[H_kv][N][d]``, hidden ``[Nq][D_h]``, W_O ``[D_h][H_q*d]``.
"""

import numpy as np

from .configs import WorkloadConfig, get_config


def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    src = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(src.size, dtype=np.uint16)
    for p in range(0, src.size, chunk):
        u = src[p:p + chunk].view(np.uint32).copy()
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u >>= np.uint32(16)
        out[p:p + chunk] = u
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng, shape, scale=1.0, chunk=1 << 24):
    """standard_normal float32 -> optional scale in float32 -> bf16 bits, drawn in chunks."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    pos = 0
    while pos < total:
        n = min(chunk, total - pos)
        x = rng.standard_normal(n, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[pos:pos + n] = f32_to_bf16_bits(x)
        pos += n
    return out.reshape(shape)


def make_inputs(n_q_heads, n_kv_heads, head_dim, n_keys, n_queries, seed,
                k_outliers=False, k_drift=False, hidden_dim=0, with_v=True):
    """Draw one layer's tensors.  Returns a dict of uint16 (bf16 bit) arrays.

    ``k_outliers``: per KV head, 4 distinct channels (``rng.choice(d, 4, replace=False)``,
    drawn after V) are multiplied by 10 in float32 before the bf16 rounding.
    ``k_drift``: ``0.5*sin(t/1000)`` (float32) is added to channels ``c < d/2`` of every KV
    head, ``t`` the 0-based key position.
    ``hidden_dim > 0``: also draws hidden ``[Nq][D_h] ~ N(0,1)`` and
    ``W_O [D_h][H_q*d] ~ N(0,1)/sqrt(D_h)`` (standard deviation ``1/sqrt(D_h)``).
    """
    rng = np.random.default_rng(seed)
    d = head_dim
    q = _normal_bf16(rng, (n_q_heads, n_queries, d))
    # K is drawn in float32 first because outliers / drift are applied before rounding.
    k32 = rng.standard_normal((n_kv_heads, n_keys, d), dtype=np.float32)
    v = _normal_bf16(rng, (n_kv_heads, n_keys, d)) if with_v else None
    outlier_channels = None
    if k_outliers:
        outlier_channels = np.stack([rng.choice(d, 4, replace=False) for _ in range(n_kv_heads)])
        for g in range(n_kv_heads):
            k32[g][:, outlier_channels[g]] *= np.float32(10.0)
    if k_drift:
        t = np.arange(n_keys, dtype=np.float32)
        drift = (np.float32(0.5) * np.sin(t / np.float32(1000.0))).astype(np.float32)
        k32[:, :, : d // 2] += drift[None, :, None]
    k = f32_to_bf16_bits(k32).reshape(k32.shape)
    del k32
    out = {"q": q, "k": k, "v": v, "outlier_channels": outlier_channels}
    if hidden_dim > 0:
        out["hidden"] = _normal_bf16(rng, (n_queries, hidden_dim))
        out["w_o"] = _normal_bf16(rng, (hidden_dim, n_q_heads * d),
                                  scale=float(1.0 / np.sqrt(np.float32(hidden_dim))))
    return out


def make_config_inputs(cfg, seed=None):
    """Inputs for one of the five named workloads (``cfg`` an index or a WorkloadConfig)."""
    if not isinstance(cfg, WorkloadConfig):
        cfg = get_config(int(cfg))
    if seed is None:
        seed = 1234 + cfg.index
    return make_inputs(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_keys, cfg.n_queries,
                       seed, k_outliers=cfg.k_outliers, k_drift=cfg.k_drift,
                       hidden_dim=cfg.hidden_dim)
