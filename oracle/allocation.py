"""Rate-distortion bit allocation over the widths {0, 2, 4, 8, 16}, top-k keep, and the
threshold-and-window keep.

Test infrastructure only (see the package docstring).

RDKV summary, §2.1: minimise sum_u w_u sigma_u 2^{-b_u} subject to a total bit budget B.
RDKV summary, §2.2: solve it by reverse water-filling (a Lagrangian relaxation) over the
hardware widths {0,2,4,8,16} -- a multiple-choice knapsack -- first over V tokens (width 0
evicts the token), then over K channels counting only the tokens kept by the first stage.

Readings where the pages are silent (all parity unpinned; they are conventions):
* sigma_u = 1 unless the caller supplies it (sigma is never defined on the page);
* the rate of a unit is its width times its size in elements (d for a V token, the number
  of retained tokens of its head for a K channel); B = floor(avg_bits * elements covered);
* one multiplier lambda per call (per layer and stage), shared by all KV heads;
* units whose cost is not > 0, or whose size is 0, keep width 0;
* the steps tied exactly at lambda* are granted in ascending unit index while they fit, and
  granting stops at the first one that does not fit.
"""

import math
from fractions import Fraction

import numpy as np

LEVELS = (0, 2, 4, 8, 16)


def step_ratios():
    """Distortion decrease per bit of each step between consecutive widths, as exact fractions.

    theta_k = (2^-b_k - 2^-b_{k+1}) / (b_{k+1} - b_k).  They strictly decrease, so every width
    is on the lower convex hull and the per-unit optimum at a given lambda is a prefix of steps.
    Returns [(numerator, denominator)] in lowest terms.
    """
    out = []
    for b0, b1 in zip(LEVELS[:-1], LEVELS[1:]):
        th = (Fraction(1, 2 ** b0) - Fraction(1, 2 ** b1)) / (b1 - b0)
        out.append((th.numerator, th.denominator))
    return out


def stage_costs(weight, sigma=None):
    """c_u = w_u * sigma_u rounded once to float32 (sigma = 1 gives c_u = w_u)."""
    w = np.asarray(weight, dtype=np.float32).ravel()
    if sigma is None:
        return w.copy()
    return (w * np.asarray(sigma, dtype=np.float32).ravel()).astype(np.float32)


def step_keys(cost32, size):
    """Lagrangian key of step k of unit u: (c_u * num_k) / (size_u * den_k), float64.

    The numerator (24-bit cost times a small integer) and the denominator (an integer below
    2^53) are exact; the single division is IEEE-rounded.  Units with cost <= 0 (or NaN) or
    size 0 get key 0 for every step, and keys equal to 0 are never taken.
    """
    c = np.asarray(cost32, dtype=np.float32).astype(np.float64)
    s = np.asarray(size, dtype=np.int64)
    keys = np.zeros((c.size, len(LEVELS) - 1))
    ok = (c > 0) & (s > 0)
    for kk, (num, den) in enumerate(step_ratios()):
        keys[ok, kk] = (c[ok] * float(num)) / (s[ok].astype(np.float64) * float(den))
    return keys


def lagrangian_allocate(cost32, size, budget):
    """Reverse water-filling with a deterministic tie rule.

    Rate at multiplier lam: R(lam) = sum of size_u * (b_{k+1} - b_k) over the steps whose key
    exceeds lam.  lam* is the smallest value in {keys} U {0} with R(lam*) <= budget.  All steps
    with key > lam* are taken; then the steps with key == lam* (at most one per unit) in
    ascending unit index while the cumulative rate stays within budget, stopping at the first
    that does not fit.
    Returns (bits uint8[U], lam*, used_bits, distortion = sum c_u 2^-b_u).
    """
    c = np.asarray(cost32, dtype=np.float32)
    s = np.asarray(size, dtype=np.int64)
    U = c.size
    B = int(budget)
    keys = step_keys(c, s)
    inc = s[:, None] * np.diff(np.array(LEVELS, dtype=np.int64))[None, :]

    def rate(lam):
        return int(inc[keys > lam].sum())

    if rate(0.0) <= B:
        lam = 0.0
    else:
        cand = np.unique(keys[keys > 0])       # ascending; rate() is non-increasing in lam
        lo, hi = 0, cand.size - 1               # rate(cand[-1]) == 0 <= B
        while lo < hi:
            mid = (lo + hi) // 2
            if rate(cand[mid]) <= B:
                hi = mid
            else:
                lo = mid + 1
        lam = float(cand[lo])

    taken = keys > lam
    nsteps = taken.sum(axis=1)
    used = rate(lam)
    if lam > 0:
        nxt = np.minimum(nsteps, len(LEVELS) - 2)
        tied = (nsteps < len(LEVELS) - 1) & (keys[np.arange(U), nxt] == lam)
        for u in np.nonzero(tied)[0]:           # ascending unit index
            k = nsteps[u]
            if used + int(inc[u, k]) > B:
                break
            used += int(inc[u, k])
            nsteps[u] += 1
    bits = np.array(LEVELS, dtype=np.uint8)[nsteps]
    dist = float((c.astype(np.float64) * np.exp2(-bits.astype(np.float64))).sum())
    return bits, lam, used, dist


def retained_counts(bits_v):
    """R_g = number of tokens of head g with a V width > 0 (kept by the token stage)."""
    return (np.asarray(bits_v) > 0).sum(axis=1).astype(np.int64)


def allocate_v_tokens(w_t, avg_bits, head_dim, sigma=None):
    """Stage 2: one unit per (KV head, token), size d; B = floor(avg * H_kv * N * d)."""
    w = np.asarray(w_t)
    hkv, n = w.shape
    E = hkv * n * head_dim
    B = math.floor(float(avg_bits) * E)
    bits, lam, used, dist = lagrangian_allocate(stage_costs(w, sigma),
                                                np.full(hkv * n, head_dim, dtype=np.int64), B)
    return bits.reshape(hkv, n), dict(lam=lam, budget=B, used=used, distortion=dist)


def allocate_k_channels(w_c, bits_v, avg_bits, sigma=None):
    """Stage 3: one unit per (KV head, channel), size R_g; B = floor(avg * d * sum_g R_g)."""
    w = np.asarray(w_c)
    hkv, d = w.shape
    R = retained_counts(bits_v)
    E = d * int(R.sum())
    B = math.floor(float(avg_bits) * E)
    size = np.repeat(R, d)
    bits, lam, used, dist = lagrangian_allocate(stage_costs(w, sigma), size, B)
    return bits.reshape(hkv, d), dict(lam=lam, budget=B, used=used, distortion=dist)


def topk_keep(scores, keep_fraction, keep_bits=16):
    """Fixed-budget keep per KV head (the KVzip policy the KVzap summary contrasts, §2.3).

    Keep the floor(rho * N) highest scores of each head at width keep_bits; order by score
    descending, ties to the lower token index; every other token gets width 0.
    """
    s = np.asarray(scores, dtype=np.float32)
    hkv, n = s.shape
    kkeep = math.floor(float(keep_fraction) * n)
    bits = np.zeros((hkv, n), dtype=np.uint8)
    for g in range(hkv):
        order = sorted(range(n), key=lambda t: (-float(s[g, t]), t))
        bits[g, order[:kkeep]] = keep_bits
    return bits


def threshold_keep(scores, threshold, window=128, keep_bits=16):
    """Adaptive keep per KV head (KVzap summary, §2.3: thresholding and the sliding window).

    Token t of head g keeps width keep_bits when its score is at or above the threshold, or
    when it is one of the head's last `window` tokens (t >= N - window); every other token
    gets width 0.  Scores and threshold are compared as float32.

    Readings: the pages threshold predicted log-scores against tau, and log is increasing,
    so the threshold here is on the score's own scale (a caller holding tau passes exp(tau)
    rounded to float32); a score equal to the threshold is kept (only scores below it are
    dropped); a NaN score is never at or above the threshold.
    """
    s = np.asarray(scores, dtype=np.float32)
    if s.ndim != 2:
        raise ValueError("scores must be [H_kv, N]")
    thr = np.float32(threshold)
    hkv, n = s.shape
    in_window = np.arange(n) >= n - int(window)
    with np.errstate(invalid="ignore"):
        keep = (s >= thr) | in_window[None, :]
    return np.where(keep, np.uint8(keep_bits), np.uint8(0)).astype(np.uint8)


def pilot_budgets(mse, total, floor_each=0):
    """KVSculpt summary, §2 (adaptive budget): after a pilot run at a uniform budget, give
    each head a share of the total budget in proportion to the square root of its pilot MSE.

    Readings: every head first gets floor_each; the rest, R = total - n * floor_each, is split
    as R * sqrt(mse_i) / sum_j sqrt(mse_j), rounded down, and the units left over go one each
    to the largest fractional parts (ties to the lower index).  If every MSE is 0, the shares
    are equal.  Shares are computed in float64.  Should rounding ever make the floors add up to
    more than R, the excess is taken back one unit each from the smallest fractional parts among
    heads that still hold a unit (ties to the higher index).
    """
    m = np.asarray(mse, dtype=np.float64).ravel()
    n = m.size
    if n < 1:
        raise ValueError("no heads")
    if not np.all(np.isfinite(m)) or np.any(m < 0):
        raise ValueError("MSE values must be finite and >= 0")
    if int(floor_each) < 0 or int(total) < 0:
        raise ValueError("total and floor_each must be >= 0")
    rest = int(total) - n * int(floor_each)
    if rest < 0:
        raise ValueError("total is below n * floor_each")
    r = np.sqrt(m)
    tot = 0.0
    for x in r:                              # left to right
        tot += float(x)
    share = np.full(n, rest / n) if tot == 0.0 else rest * (r / tot)
    base = np.floor(share).astype(np.int64)
    left = rest - int(base.sum())
    frac = share - base
    if left >= 0:
        order = sorted(range(n), key=lambda i: (-frac[i], i))
        for i in order[:left]:
            base[i] += 1
    else:
        order = sorted((i for i in range(n) if base[i] > 0), key=lambda i: (frac[i], -i))
        for i in order[:-left]:
            base[i] -= 1
    return base + int(floor_each)
