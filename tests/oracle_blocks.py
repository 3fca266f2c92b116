"""The oracle's attention quantities evaluated on blocks of query rows, side by side in threads.

Row i of a causal layer depends only on q_i and the keys up to its position p_i = N - Nq + i,
so a block of rows [r0, r1) with the keys cut at N - Nq + r1 is itself a layer whose last rows
are exactly those rows (the bottom-right alignment puts them back at their own positions).
The token scores are sums (SUM) or maxima (MAX) over rows, so the blocks' contributions are
combined in the same way, in float64, in a fixed order.  Every value still comes from the
oracle's own functions; this only lets numpy's kernels, which release the interpreter lock,
run on several cores, so whole KV heads of the full-size workloads finish in seconds.  The BLAS
library runs one thread per call meanwhile: the blocks are the parallelism, and nested BLAS
threads would oversubscribe the cores many times over.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle

_WORKERS = min(16, os.cpu_count() or 1)


def _key_end(n_keys, n_queries, r1, causal):
    return n_keys - n_queries + r1 if causal else n_keys


def _blocks(n_queries, rows):
    return [(r0, min(n_queries, r0 + rows)) for r0 in range(0, n_queries, rows)]


def head_lse(q, k, heads, causal=True, rows=256):
    """oracle.row_lse for the query heads `heads` (their KV head from the GQA grouping)."""
    hq, nq, _ = q.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    jobs = [(h, r0, r1) for h in heads for r0, r1 in _blocks(nq, rows)]

    def run(job):
        h, r0, r1 = job
        ke = _key_end(n, nq, r1, causal)
        return oracle.row_lse(q[h:h + 1, r0:r1], k[h // G:h // G + 1, :ke], causal=causal)[0]

    out = np.empty((len(heads), nq))
    pos = {h: j for j, h in enumerate(heads)}
    with threadpool_limits(limits=1), ThreadPoolExecutor(_WORKERS) as ex:
        for (h, r0, r1), l in zip(jobs, ex.map(run, jobs)):
            out[pos[h], r0:r1] = l
    return out


def group_scores_sum(q, k, lse_heads, g, causal=True, rows=256):
    """oracle.token_scores_sum of KV head g: lse_heads holds the LSE rows of its G query heads."""
    hq, nq, _ = q.shape
    hkv, n, _ = k.shape
    G = hq // hkv
    jobs = [(j, r0, r1) for j in range(G) for r0, r1 in _blocks(nq, rows)]

    def run(job):
        j, r0, r1 = job
        h = g * G + j
        ke = _key_end(n, nq, r1, causal)
        return oracle.token_scores_sum(q[h:h + 1, r0:r1], k[g:g + 1, :ke], lse_heads[j:j + 1, r0:r1],
                                       causal=causal)[0]

    w = np.zeros(n)
    with threadpool_limits(limits=1), ThreadPoolExecutor(_WORKERS) as ex:
        for part in ex.map(run, jobs):
            w[:part.size] += part
    return w


def group_scores_max(q, k, lse_heads, hidden, w_o, v, g, causal=True):
    """oracle.token_scores_max of KV head g, one query head per job (its W_O columns only), then
    the maximum over the group's heads, as the grouped score takes it."""
    hq, nq, d = q.shape
    hkv, n, _ = k.shape
    G = hq // hkv

    def run(j):
        h = g * G + j
        return oracle.token_scores_max(q[h:h + 1], k[g:g + 1], lse_heads[j:j + 1], hidden,
                                       np.ascontiguousarray(w_o[:, h * d:(h + 1) * d]), v[g:g + 1],
                                       causal=causal)[0]

    with threadpool_limits(limits=1), ThreadPoolExecutor(_WORKERS) as ex:
        parts = list(ex.map(run, range(G)))
    return np.max(np.stack(parts), axis=0)
