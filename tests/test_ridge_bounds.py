"""The ridge error bounds (tests/ridge_bounds.py) hold for a solve whose weights and target carry
perturbations of exactly the modelled sizes, and are not vacuous: a perturbation 4x larger than
modelled, in the direction that moves V most, breaks the residual bound."""

import numpy as np

import oracle
from tests.ridge_bounds import ridge_error_bounds
from workloads import bf16_bits_to_f32, make_inputs


def _perturbed_solve(x, y, nc, lam, causal, scale_eps, rng):
    q, k = x["q"], x["k"]
    v_r = np.ascontiguousarray(x["v"][:, nc:])
    d = q.shape[-1]
    G = q.shape[0] // k.shape[0]
    s = 1.0 / np.sqrt(d)
    Q = bf16_bits_to_f32(q).astype(np.float64)
    K = bf16_bits_to_f32(k).astype(np.float64)
    Vr = bf16_bits_to_f32(v_r).astype(np.float64)
    out = []
    for g, (Ac, Ar, T) in enumerate(oracle.ridge_system(q, k, v_r, y, nc, causal=causal)):
        Qg = Q[g * G:(g + 1) * G].reshape(-1, d)
        A = np.hstack([Ac, Ar])
        dx = d * 2.0 ** -24 * s * (np.abs(Qg) @ np.abs(K[g]).T)
        dl = np.where(A > 0, dx, 0.0).max(axis=1) + 2.0 ** -20
        eps = scale_eps * (dx + dl[:, None] + 2.0 ** -21)
        Ap = A * (1 + eps * rng.choice([-1.0, 1.0], A.shape))
        Acp, Arp = Ap[:, :nc], Ap[:, nc:]
        Yg = np.asarray(y, dtype=np.float64)[g * G:(g + 1) * G].reshape(-1, d)
        Tp = Yg - Arp @ Vr[g]
        out.append(np.linalg.solve(Acp.T @ Acp + lam * np.eye(nc), Acp.T @ Tp))
    return np.stack(out)


def test_bounds_hold_at_the_modelled_perturbation():
    rng = np.random.default_rng(3)
    for causal, (hq, hkv, d, nc, m, nq, lam) in ((False, (4, 2, 64, 40, 24, 100, 0.1)),
                                                  (True, (6, 2, 128, 70, 30, 128, 0.01))):
        x = make_inputs(hq, hkv, d, nc + m, nq, seed=nc + m)
        y = rng.standard_normal((hq, nq, d)).astype(np.float32)
        v_gpu = _perturbed_solve(x, y, nc, lam, causal, 1.0, rng)
        for b in ridge_error_bounds(x["q"], x["k"], np.ascontiguousarray(x["v"][:, nc:]), y, nc, lam, causal,
                                    v_gpu):
            assert (b["res"] <= b["res_bound"]).all()
            assert (b["err"] <= b["err_bound"]).all()


def test_bounds_are_not_vacuous():
    rng = np.random.default_rng(4)
    hq, hkv, d, nc, m, nq, lam = 4, 1, 64, 30, 10, 80, 1e-3
    x = make_inputs(hq, hkv, d, nc + m, nq, seed=99)
    y = rng.standard_normal((hq, nq, d)).astype(np.float32)
    v_exact = oracle.ridge_value_fit(x["q"], x["k"], x["v"][:, nc:], y, nc, lam)
    b = ridge_error_bounds(x["q"], x["k"], np.ascontiguousarray(x["v"][:, nc:]), y, nc, lam, False, v_exact)[0]
    # the exact solution sits inside, and a V moved by 4x the error bound along one entry is outside
    assert (b["err"] <= b["err_bound"]).all()
    i, j = np.unravel_index(np.argmax(b["err_bound"]), b["err_bound"].shape)
    v_off = v_exact.copy()
    v_off[0, i, j] += 4 * b["err_bound"][i, j] + 1e-12
    b2 = ridge_error_bounds(x["q"], x["k"], np.ascontiguousarray(x["v"][:, nc:]), y, nc, lam, False, v_off)[0]
    assert not (b2["err"] <= b2["err_bound"]).all()
