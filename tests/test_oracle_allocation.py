"""Pins of the oracle's bit allocation and top-k keep (CPU only).

The Lagrangian allocation is checked against exhaustive enumeration of the multiple-choice
knapsack on tiny problems (exact optimum at its own rate, and within the Lagrangian dual
bound at the requested budget), against the hand-derived examples in
``golden/allocation_uniform_example.txt``, and against feasibility and monotonicity.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

LEVELS = (0, 2, 4, 8, 16)


def _read_rows(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_step_ratios_match_hand_derivation(golden_dir):
    rows = _read_rows(os.path.join(golden_dir, "step_ratios.txt"))
    want = [(int(r[2]), int(r[3])) for r in rows]
    assert oracle.step_ratios() == want


def test_uniform_worked_examples(golden_dir):
    for r in _read_rows(os.path.join(golden_dir, "allocation_uniform_example.txt")):
        avg, B = float(r[0]), int(r[1])
        lam = Fraction(int(r[2]), int(r[3]))
        used, D = int(r[4]), float(r[5])
        bits_want = [int(b) for b in r[6:]]
        cost = np.ones(8, dtype=np.float32)
        size = np.ones(8, dtype=np.int64)
        assert math.floor(avg * 8) == B
        bits, got_lam, got_used, got_D = oracle.lagrangian_allocate(cost, size, B)
        assert got_lam == float(lam)
        assert got_used == used
        assert got_D == D
        assert bits.tolist() == bits_want


def _enumerate(cost, size, budget):
    """min sum c 2^-b subject to sum size*b <= budget, by exhaustive enumeration."""
    best = math.inf
    for combo in itertools.product(LEVELS, repeat=len(cost)):
        r = sum(int(s) * b for s, b in zip(size, combo))
        if r <= budget:
            best = min(best, sum(float(c) * 2.0 ** -b for c, b in zip(cost, combo)))
    return best


@pytest.mark.parametrize("seed", range(12))
def test_lagrangian_is_optimal_at_its_rate_and_within_dual_gap(seed):
    rng = np.random.default_rng(seed)
    U = int(rng.integers(2, 7))
    cost = rng.exponential(1.0, U).astype(np.float32)
    if seed % 3 == 0:
        cost[rng.integers(0, U)] = cost[0]              # force equal costs (ties)
    size = rng.integers(1, 5, U).astype(np.int64)
    B = int(rng.integers(0, 16 * int(size.sum()) + 1))
    bits, lam, used, D = oracle.lagrangian_allocate(cost, size, B)
    assert set(bits.tolist()) <= set(LEVELS)
    assert used == int((size * bits.astype(np.int64)).sum()) <= B
    assert D == pytest.approx(float((cost.astype(np.float64) * 2.0 ** -bits.astype(np.float64)).sum()),
                              rel=1e-15)
    # exactly optimal for the rate it used
    assert D == pytest.approx(_enumerate(cost, size, used), rel=1e-12, abs=1e-300)
    # Lagrangian dual bound at the requested budget
    opt_B = _enumerate(cost, size, B)
    assert opt_B <= D * (1 + 1e-12)
    assert opt_B >= D - lam * (B - used) - 1e-12 * D


def test_monotone_in_cost_at_equal_size():
    rng = np.random.default_rng(5)
    cost = rng.exponential(1.0, 400).astype(np.float32)
    size = np.full(400, 64, dtype=np.int64)
    for avg in (0.5, 1.0, 2.5, 3.0, 7.0):
        B = math.floor(avg * 400 * 64)
        bits, *_ = oracle.lagrangian_allocate(cost, size, B)
        order = np.argsort(cost, kind="stable")
        b_sorted = bits[order].astype(int)
        c_sorted = cost[order]
        for i in range(len(order) - 1):
            if c_sorted[i] < c_sorted[i + 1]:
                assert b_sorted[i] <= b_sorted[i + 1]


def test_budget_extremes_and_zero_costs():
    cost = np.array([0.0, 1.0, 2.0, 0.5, 0.0], dtype=np.float32)
    size = np.array([3, 3, 1, 2, 0], dtype=np.int64)
    bits, lam, used, D = oracle.lagrangian_allocate(cost, size, 0)
    assert bits.tolist() == [0] * 5 and used == 0 and D == pytest.approx(3.5)
    bits, lam, used, D = oracle.lagrangian_allocate(cost, size, 10 ** 6)
    assert bits.tolist() == [0, 16, 16, 16, 0] and lam == 0.0
    assert used == 16 * (3 + 1 + 2)


def test_stage_wrappers_budget_and_sizes():
    rng = np.random.default_rng(9)
    w_t = rng.exponential(1.0, (3, 50))
    bits_v, info = oracle.allocate_v_tokens(w_t, 2.5, 64)
    assert info["budget"] == math.floor(2.5 * 3 * 50 * 64)
    assert info["used"] == int(bits_v.astype(np.int64).sum()) * 64 <= info["budget"]
    w_c = rng.exponential(1.0, (3, 64))
    bits_k, info_k = oracle.allocate_k_channels(w_c, bits_v, 2.5)
    R = (bits_v > 0).sum(axis=1)
    assert info_k["budget"] == math.floor(2.5 * 64 * int(R.sum()))
    assert info_k["used"] == int((bits_k.astype(np.int64) * R[:, None]).sum()) <= info_k["budget"]


def test_sigma_multiplies_cost():
    w = np.array([1.0, 2.0, 4.0], dtype=np.float32)
    sigma = np.array([4.0, 2.0, 1.0], dtype=np.float32)
    c = oracle.stage_costs(w, sigma)
    assert c.tolist() == [4.0, 4.0, 4.0]
    bits, *_ = oracle.lagrangian_allocate(c, np.ones(3, dtype=np.int64), 6)
    assert bits.tolist() == [2, 2, 2]


@pytest.mark.parametrize("seed", range(4))
def test_topk_keep_properties(seed):
    rng = np.random.default_rng(seed)
    n = 97
    s = rng.integers(0, 12, (3, n)).astype(np.float32)      # many equal scores
    bits = oracle.topk_keep(s, 0.25)
    k = math.floor(0.25 * n)
    for g in range(3):
        kept = np.nonzero(bits[g] == 16)[0]
        drop = np.nonzero(bits[g] == 0)[0]
        assert kept.size == k and kept.size + drop.size == n
        assert s[g, kept].min() >= s[g, drop].max()
        thr = s[g, kept].min()
        eq_kept = kept[s[g, kept] == thr]
        eq_drop = drop[s[g, drop] == thr]
        if eq_kept.size and eq_drop.size:
            assert eq_kept.max() < eq_drop.min()


def test_threshold_keep_worked_examples(golden_dir):
    path = os.path.join(golden_dir, "threshold_keep_example.txt")
    with open(path) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for r in rows:
        head, sc, want = (part.split() for part in r.split("|"))
        thr, win = float(head[0]), int(head[1])
        s = np.array([[float(x) for x in sc]], dtype=np.float32)
        got = oracle.threshold_keep(s, thr, win)
        assert got.tolist() == [[int(x) for x in want]]


def test_threshold_keep_extremes_and_nan():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((3, 300)).astype(np.float32)
    n = s.shape[1]
    # threshold +inf: exactly the window; -inf: everything
    only_win = oracle.threshold_keep(s, np.inf, 128)
    assert (only_win[:, : n - 128] == 0).all() and (only_win[:, n - 128:] == 16).all()
    assert (oracle.threshold_keep(s, -np.inf, 0) == 16).all()
    # a NaN score is dropped outside the window and kept inside it
    s2 = s.copy()
    s2[0, 5] = np.nan
    s2[0, n - 1] = np.nan
    b = oracle.threshold_keep(s2, -np.inf, 1)
    assert b[0, 5] == 0 and b[0, n - 1] == 16
    # keep_bits is the width of every kept token
    assert set(np.unique(oracle.threshold_keep(s, 0.0, 10, keep_bits=8))) <= {0, 8}


@pytest.mark.parametrize("seed", range(3))
def test_threshold_keep_matches_topk_at_the_kth_score(seed):
    """With distinct scores, no window and the threshold at each head's k-th largest score,
    the threshold rule keeps exactly the k highest scores: the sort-based top-k keep."""
    rng = np.random.default_rng(100 + seed)
    n = 211
    s = rng.permutation(np.arange(3 * n, dtype=np.float32)).reshape(3, n) * np.float32(0.37)
    k = math.floor(0.3 * n)
    want = oracle.topk_keep(s, 0.3)
    for g in range(3):
        thr = np.sort(s[g])[::-1][k - 1]
        got = oracle.threshold_keep(s[g : g + 1], thr, 0)
        assert got[0].tolist() == want[g].tolist()


def test_threshold_keep_monotone_in_threshold_and_window():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((2, 500)).astype(np.float32)
    prev = None
    for thr in (-1.0, -0.2, 0.0, 0.7, 2.0):
        b = oracle.threshold_keep(s, thr, 64)
        if prev is not None:
            assert ((b > 0) <= (prev > 0)).all()     # a higher threshold never keeps more
        prev = b
    small = oracle.threshold_keep(s, 1.0, 16)
    large = oracle.threshold_keep(s, 1.0, 200)
    assert ((small > 0) <= (large > 0)).all()


def test_pilot_budget_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "pilot_budget_example.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 4
    for r in rows:
        head, mse, want = (part.split() for part in r.split("|"))
        got = oracle.pilot_budgets([float(x) for x in mse], int(head[0]), int(head[1]))
        assert got.tolist() == [int(x) for x in want]


@pytest.mark.parametrize("seed", range(4))
def test_pilot_budget_properties(seed):
    rng = np.random.default_rng(seed)
    n = 9
    mse = rng.random(n) ** 3
    total = 1000 + seed
    b = oracle.pilot_budgets(mse, total)
    assert int(b.sum()) == total                                  # the whole budget, no more
    share = total * np.sqrt(mse) / np.sqrt(mse).sum()
    assert np.all(np.abs(b - share) < 1.0)                        # within one unit of the exact share
    order = np.argsort(mse)
    assert np.all(np.diff(b[order]) >= 0)                         # more pilot error, no smaller budget
    assert b.tolist() == oracle.pilot_budgets(mse * 37.0, total).tolist()   # only ratios matter
    bf = oracle.pilot_budgets(mse, total, floor_each=50)
    assert bf.min() >= 50 and int(bf.sum()) == total
