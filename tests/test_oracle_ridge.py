"""Pins of the ridge value fit (KVSculpt summary, §2 value step): the oracle against things
other than itself.

* exact recovery: targets made by torch's scaled_dot_product_attention (float64) over
  [K_c; K_r], [V_c*; V_r] are fitted back to V_c* at lam = 0;
* first-order optimality: the gradient (torch autograd through scaled_dot_product_attention)
  of ||Y_hat(V) - Y||^2 + lam ||V||^2 vanishes at the fitted V, with G > 1 query heads per
  KV head, causal and not, with and without a retained zone;
* the same solution from numpy's least squares on the augmented system [A_c; sqrt(lam) I];
* a closed form: one compressed key and no retained zone give every weight 1, so
  V_c = (sum of the target rows) / (R + lam).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs


def _case(hq, hkv, d, nc, m, nq, seed):
    x = make_inputs(hq, hkv, d, nc + m, nq, seed=seed)
    return x["q"], x["k"], x["v"]


def _sdpa_out(q, k, v, causal, scale=None):
    """Attention outputs [H_q][Nq][d] by torch (float64), bottom-right causal alignment."""
    Q = torch.from_numpy(oracle.as_f64(q))
    K = torch.from_numpy(oracle.as_f64(k)) if isinstance(k, np.ndarray) else k
    V = v
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    mask = None
    if causal:
        mask = torch.arange(n)[None, :] <= (n - nq + torch.arange(nq))[:, None]
    outs = [torch.nn.functional.scaled_dot_product_attention(Q[h][None], K[h // G][None], V[h // G][None],
                                                             attn_mask=mask, scale=sc)[0] for h in range(hq)]
    return torch.stack(outs)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [0, 24])
def test_exact_recovery_at_zero_lambda(causal, m):
    hq, hkv, d, nc, nq = 4, 2, 32, 20, 48
    q, k, v = _case(hq, hkv, d, nc, m, nq, seed=7 + m)
    V = torch.from_numpy(oracle.as_f64(v))
    y = _sdpa_out(q, k, V, causal).numpy()
    got = oracle.ridge_value_fit(q, k, v[:, nc:], y, nc, 0.0, causal=causal)
    np.testing.assert_allclose(got, oracle.as_f64(v[:, :nc]), rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m,lam", [(0, 0.5), (16, 0.05), (16, 3.0)])
def test_gradient_vanishes_at_the_fit(causal, m, lam):
    hq, hkv, d, nc, nq = 6, 2, 32, 12, 40
    q, k, v = _case(hq, hkv, d, nc, m, nq, seed=11)
    rng = np.random.default_rng(3)
    y = rng.standard_normal((hq, nq, d))                    # any target, not reachable exactly
    fit = oracle.ridge_value_fit(q, k, v[:, nc:], y, nc, lam, causal=causal)
    Vc = torch.tensor(fit, requires_grad=True)
    Vr = torch.from_numpy(oracle.as_f64(v[:, nc:]))
    Y = torch.from_numpy(y)

    def objective(vc):
        full = torch.cat([vc, Vr], dim=1)
        return ((_sdpa_out(q, k, full, causal) - Y) ** 2).sum() + lam * (vc ** 2).sum()

    f = objective(Vc)
    f.backward()
    g = Vc.grad.numpy()
    assert np.abs(g).max() < 1e-9 * max(1.0, float(f.detach()))
    # convex: any step away costs more
    with torch.no_grad():
        for s in (1e-3, 1e-1):
            step = torch.from_numpy(rng.standard_normal(fit.shape)) * s
            assert objective(Vc + step) > f


@pytest.mark.parametrize("m", [0, 10])
def test_matches_augmented_least_squares(m):
    hq, hkv, d, nc, nq = 2, 1, 16, 9, 30
    lam = 0.7
    q, k, v = _case(hq, hkv, d, nc, m, nq, seed=5)
    y = np.random.default_rng(9).standard_normal((hq, nq, d))
    fit = oracle.ridge_value_fit(q, k, v[:, nc:], y, nc, lam)
    # A from torch's softmax, independent of the oracle's weights
    Q = torch.from_numpy(oracle.as_f64(q))
    K = torch.from_numpy(oracle.as_f64(k))[0]
    A = torch.softmax((Q @ K.T) / np.sqrt(d), dim=-1).numpy().reshape(hq * nq, nc + m)
    Vr = oracle.as_f64(v[0, nc:])
    T = y.reshape(hq * nq, d) - A[:, nc:] @ Vr
    Aug = np.vstack([A[:, :nc], np.sqrt(lam) * np.eye(nc)])
    rhs = np.vstack([T, np.zeros((nc, d))])
    ls = np.linalg.lstsq(Aug, rhs, rcond=None)[0]
    np.testing.assert_allclose(fit[0], ls, rtol=0, atol=1e-10)


def test_single_compressed_key_closed_form():
    hq, hkv, d, nq = 3, 1, 16, 7
    q, k, v = _case(hq, hkv, d, 1, 0, nq, seed=2)
    y = np.random.default_rng(4).standard_normal((hq, nq, d))
    for lam in (0.0, 2.5):
        fit = oracle.ridge_value_fit(q, k, None, y, 1, lam)
        want = y.reshape(-1, d).sum(axis=0) / (hq * nq + lam)
        np.testing.assert_allclose(fit[0, 0], want, rtol=1e-13, atol=1e-15)


def test_rejects_bad_sizes():
    q, k, v = _case(2, 1, 16, 4, 0, 5, seed=1)
    with pytest.raises(ValueError):
        oracle.ridge_value_fit(q, k, None, np.zeros((2, 5, 16)), 0, 1.0)
    with pytest.raises(ValueError):
        oracle.ridge_value_fit(q, k, None, np.zeros((2, 5, 16)), 5, 1.0)
