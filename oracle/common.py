"""Input widening and the query-position convention shared by the oracle's modules.

Test infrastructure only (see the package docstring).
"""

import numpy as np


def as_f64(x):
    """bf16 bit patterns (uint16) -> float64 exactly; any other array -> float64 as is."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def query_positions(n_keys, n_queries):
    """Position of query row i: the rows are the LAST n_queries positions of the sequence.

    The pages do not say how a block of queries shorter than the cache lines up with it;
    the reading taken is bottom-right alignment, p_i = N - Nq + i (parity unpinned).
    """
    return n_keys - n_queries + np.arange(n_queries, dtype=np.int64)


def default_scale(head_dim, scale=None):
    """Softmax scale: 1/sqrt(d) (float64) unless the caller fixes one."""
    if scale is None or scale == 0:
        return 1.0 / np.sqrt(float(head_dim))
    return float(np.float32(scale))


def visible_mask(n_keys, n_queries, row0, row1, causal):
    """Boolean [row1-row0][N]: True where query row i may attend key t (t <= p_i)."""
    if not causal:
        return np.ones((row1 - row0, n_keys), dtype=bool)
    pos = query_positions(n_keys, n_queries)[row0:row1]
    return np.arange(n_keys)[None, :] <= pos[:, None]
