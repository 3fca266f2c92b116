"""The pack kernels decide a code from v = (x - z) * (1 / s) evaluated in float32 and fall back to
the defining float64 division only where v lies within 2^(b-21) of a half-integer.  This checks
that argument on the CPU: numpy's float32 operations round like the kernel's (no fused
multiply-add), so outside the band the float32 decision must equal the float64 one, at every
width and over value scales from 1e-3 to 1e4."""

import numpy as np
import pytest


def _bf16(x):
    u = x.astype(np.float32).view(np.uint32)
    u = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return u.view(np.float32)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_float32_decision_outside_the_band(b):
    rng = np.random.default_rng(b)
    maxc = (1 << b) - 1
    band = np.float32(2.0 ** (b - 21))
    near_total = 0
    for scale in (1e-3, 1.0, 30.0, 1e4):
        x = _bf16(rng.standard_normal((20000, 32)).astype(np.float32) * np.float32(scale))
        mn, mx = x.min(1), x.max(1)
        s = ((mx.astype(np.float64) - mn.astype(np.float64)) / maxc).astype(np.float32)
        ok = s != 0
        rs = (np.float32(1) / s[ok]).astype(np.float32)
        v32 = ((x[ok] - mn[ok, None]).astype(np.float32) * rs[:, None]).astype(np.float32)
        r32 = np.rint(v32)
        v64 = (x[ok].astype(np.float64) - mn[ok, None].astype(np.float64)) / s[ok, None].astype(np.float64)
        r64 = np.clip(np.rint(v64), 0, maxc)
        near = np.abs(v32 - r32) > np.float32(0.5) - band
        assert not np.any((r32 != r64) & ~near)
        assert r32.max() <= maxc and r32.min() >= 0          # no clamp needed on the fast path
        near_total += int(near.sum())
    assert near_total > 0                                     # the fallback is exercised (exact ties)
