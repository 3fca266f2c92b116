"""kvc_pilot_budgets (a host function of the library, KVSculpt summary §2 adaptive budget)
against the oracle, bit for bit: the hand-derived golden rows, random pilot MSEs of every scale,
zero heads, floors, and the all-zero equal split.  The call touches no device, so it runs here."""

import os

import numpy as np
import pytest

import oracle
from kv_cache_compression_pass_amd import _lib as C
from kv_cache_compression_pass_amd.api import kvc_pilot_budgets


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(C.LIB_PATH):
        pytest.fail("libkvc.so is not built (run __graft_entry__.build())")


def test_golden_rows(golden_dir):
    with open(os.path.join(golden_dir, "pilot_budget_example.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for ln in rows:
        head, mse, want = (p.split() for p in ln.split("|"))
        got = kvc_pilot_budgets([float(x) for x in mse], int(head[0]), int(head[1]))
        assert got.tolist() == [int(x) for x in want]


@pytest.mark.parametrize("seed", range(12))
def test_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        n = int(rng.integers(1, 65))
        kind = int(rng.integers(0, 5))
        if kind == 0:
            mse = rng.random(n)
        elif kind == 1:
            mse = np.exp(rng.normal(0.0, 12.0, n))              # many decades apart
        elif kind == 2:
            mse = rng.integers(0, 4, n).astype(np.float64) ** 2  # exact roots, ties, zeros
        elif kind == 3:
            mse = np.zeros(n)
        else:
            mse = rng.random(n) * (rng.random(n) < 0.3)         # mostly zero heads
        floor_each = int(rng.integers(0, 20))
        total = n * floor_each + int(rng.integers(0, 1 << int(rng.integers(1, 40))))
        want = oracle.pilot_budgets(mse, total, floor_each)
        got = kvc_pilot_budgets(mse, total, floor_each)
        assert got.tolist() == want.tolist(), (n, kind, total, floor_each)
        assert int(got.sum()) == total


def test_single_head_and_zero_rest():
    assert kvc_pilot_budgets([3.0], 17).tolist() == [17]
    assert kvc_pilot_budgets([0.0], 17).tolist() == [17]
    assert kvc_pilot_budgets([1.0, 9.0], 8, 4).tolist() == [4, 4]
    assert kvc_pilot_budgets([1.0, 9.0], 0).tolist() == [0, 0]
