"""Error bounds for the ridge value fit computed on the GPU, derived from its operand precisions.

The GPU forms the attention weights A in float32 (bf16 matrix-core logits with float32 sums, the
row LSE from the scorer's pass 1, one hardware exp2), the target T = Y - A_r V_r in float32 (the
weights as a bf16 hi + lo pair, to 2^-17, against the exact bf16 V_r), and then solves
(A_c^T A_c + lam I) V = A_c^T T in float64 from those float32 values (every product exact, sums
and the Cholesky solve in float64).  So its V solves exactly a system whose weights and target
are perturbed elementwise:
  |dA_rt| <= eps_rt A_rt,  eps_rt = dx_rt + dl_r + 2^-21,
  dx_rt = d 2^-24 s sum_c |q_rc k_tc|   (float32 sum of d exact products, the logit's error),
  dl_r = max_t dx_rt + 2^-20           (the LSE: a smooth maximum of the logits, plus its sums),
  |dT| <= |dA_r| |V_r| + (2^-17 + m 2^-24) |A_r| |V_r| + 2^-24 (|Y| + |A_r| |V_r|).
The residual of the exact system at the GPU's V is then bounded elementwise,
  |M V - B| <= (2 |dA_c|^T |A_c| + |dA_c|^T |dA_c|) |V| + |dA_c|^T |T| + (|A_c| + |dA_c|)^T |dT|,
and V - V_exact = M^-1 (M V - B), so |V - V_exact| <= |M^-1| times that bound.  Conditioning enters
only through |M^-1| itself, not through cond(M) times a norm.
"""

import numpy as np

import oracle
from workloads import bf16_bits_to_f32


def _f64(bits):
    return bf16_bits_to_f32(np.asarray(bits)).astype(np.float64)


def ridge_error_bounds(q, k, v_r, y, nc, lam, causal, v_gpu, scale=None):
    """Per KV head: dict with the exact solution, the measured error and residual, and their
    elementwise bounds (arrays [n_c][d])."""
    Q, K = _f64(q), _f64(k)
    hq, nq, d = Q.shape
    hkv, n, _ = K.shape
    G = hq // hkv
    m = n - nc
    s = float(scale) if scale else 1.0 / np.sqrt(d)
    Vr = _f64(v_r) if m > 0 else np.zeros((hkv, 0, d))
    Y = np.asarray(y, dtype=np.float64)
    u = 2.0 ** -24
    out = []
    for g, (Ac, Ar, T) in enumerate(oracle.ridge_system(q, k, v_r, y, nc, scale, causal)):
        Qg = Q[g * G:(g + 1) * G].reshape(-1, d)
        A = np.hstack([Ac, Ar])
        dx = d * u * s * (np.abs(Qg) @ np.abs(K[g]).T)
        vis = A > 0
        dl = np.where(vis, dx, 0.0).max(axis=1) + 2.0 ** -20
        eps = dx + dl[:, None] + 2.0 ** -21
        dA = eps * A
        dAc, dAr = dA[:, :nc], dA[:, nc:]
        Yg = Y[g * G:(g + 1) * G].reshape(-1, d)
        ArVr = np.abs(Ar) @ np.abs(Vr[g])
        dT = dAr @ np.abs(Vr[g]) + (2.0 ** -17 + m * u) * ArVr + u * (np.abs(Yg) + ArVr)
        M = Ac.T @ Ac + float(lam) * np.eye(nc)
        B = Ac.T @ T
        V = np.asarray(v_gpu[g], dtype=np.float64)
        res_bound = ((2 * dAc.T @ np.abs(Ac) + dAc.T @ dAc) @ np.abs(V) + dAc.T @ np.abs(T)
                     + (np.abs(Ac) + dAc).T @ dT)
        res_bound += 4 * n * 2.0 ** -53 * (np.abs(M) @ np.abs(V) + np.abs(B))   # the float64 solve
        exact = np.linalg.solve(M, B)
        err_bound = np.abs(np.linalg.inv(M)) @ res_bound
        out.append({"exact": exact, "err": np.abs(V - exact), "err_bound": err_bound,
                    "res": np.abs(M @ V - B), "res_bound": res_bound, "cond": np.linalg.cond(M)})
    return out
