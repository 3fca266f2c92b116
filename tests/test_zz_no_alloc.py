"""The allocation-free row LSE (kvc_row_lse_noalloc) against the row LSE with a workspace
(kvc_row_lse): the same kernels, so the results are bitwise equal, on two calls in a row, the
second on a smaller layer than the first (the static scratch keeps the first call's partials).
Both layers split their keys into chunks, so the scratch is used.  The smaller layer is also
checked against the oracle at the row LSE bar (1e-4 abs)."""

import numpy as np
import pytest
import torch

import kv_cache_compression_pass_amd as kvc
import oracle
from workloads import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(hq, hkv, d, N, Nq, causal, seed):
    print(f"case row_lse_noalloc: H_q={hq} H_kv={hkv} d={d} N={N} Nq={Nq} causal={causal}", flush=True)
    x = make_inputs(hq, hkv, d, N, Nq, seed=seed)
    desc = kvc.make_desc(hq, hkv, d, N, Nq, causal)
    ws_bytes = kvc.kvc_workspace_size(kvc.OP_ROW_LSE, desc, 0)
    assert 256 < ws_bytes <= 16 << 20
    q, k = kvc.bf16_tensor(x["q"], DEV), kvc.bf16_tensor(x["k"], DEV)
    want = torch.empty(hq, Nq, dtype=torch.float32, device=DEV)
    kvc.kvc_row_lse(desc, q, k, want, kvc.workspace(kvc.OP_ROW_LSE, desc, 0, DEV))
    got = torch.full((hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    kvc.kvc_row_lse_noalloc(desc, q, k, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    return x, got.cpu().numpy()


def test_row_lse_noalloc_two_calls_smaller_second():
    assert torch.cuda.is_available()
    kvc.load()
    # 1: the decode-shaped layer of the 128k workload at a quarter of the keys (chunked keys)
    _run(32, 8, 128, 32768, 512, True, seed=11)
    # 2: a smaller, ragged layer right after it, on the same scratch
    x, got = _run(6, 2, 64, 3001, 300, True, seed=12)
    want = oracle.row_lse(x["q"], x["k"])
    assert np.abs(got - want).max() <= 1e-4
