"""The row-block evaluation of the oracle (tests/oracle_blocks.py), used by the full-size GPU
parity tests, equals the oracle's own whole-layer evaluation on small layers: row LSE, SUM and
MAX scores, causal with Nq < N and not causal, with blocks smaller than the layer."""

import numpy as np
import pytest

import oracle
from tests import oracle_blocks as OB
from workloads import make_inputs


@pytest.mark.parametrize("causal,N,Nq", [(True, 300, 300), (True, 301, 170), (False, 200, 150)])
def test_blocks_match_whole_layer(causal, N, Nq):
    hq, hkv, d = 6, 2, 64
    x = make_inputs(hq, hkv, d, N, Nq, seed=N + Nq, hidden_dim=40)
    lse = oracle.row_lse(x["q"], x["k"], causal=causal)
    lse_b = OB.head_lse(x["q"], x["k"], list(range(hq)), causal=causal, rows=64)
    np.testing.assert_allclose(lse_b, lse, rtol=0, atol=1e-12)
    w = oracle.token_scores_sum(x["q"], x["k"], lse, causal=causal)
    s = oracle.token_scores_max(x["q"], x["k"], lse, x["hidden"], x["w_o"], x["v"], causal=causal)
    G = hq // hkv
    for g in range(hkv):
        wb = OB.group_scores_sum(x["q"], x["k"], lse[g * G:(g + 1) * G], g, causal=causal, rows=64)
        np.testing.assert_allclose(wb, w[g], rtol=1e-12, atol=1e-300)
        sb = OB.group_scores_max(x["q"], x["k"], lse[g * G:(g + 1) * G], x["hidden"], x["w_o"], x["v"], g,
                                 causal=causal)
        np.testing.assert_allclose(sb, s[g], rtol=1e-12, atol=0)
