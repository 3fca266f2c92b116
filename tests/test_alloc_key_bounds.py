"""The allocator's float32 bounds on its float64 step keys (alloc.hip, key_bounds): the multi-block
select skips a unit's exact keys when their float32 estimates, widened to float64 bit patterns, lie
more than 2^33 patterns away from the range in question.  This emulates the estimate step by step in
float32 (the kernels round every operation as written, no contraction) and checks that the exact key's
pattern stays within 2^32 of it, half the margin, over costs across the whole float32 range and the unit
sizes of both stages."""

import numpy as np

THETA_NUM = np.array([3, 3, 15, 255], dtype=np.float64)
THETA_DEN = np.array([8, 32, 1024, 524288], dtype=np.float64)
THETA_F = (THETA_NUM / THETA_DEN).astype(np.float32)


def exact_patterns(c, s):
    """float64 step keys (c * num) / (s * den) as the kernels form them, as bit patterns."""
    k = (c.astype(np.float64)[:, None] * THETA_NUM) / (s.astype(np.float64)[:, None] * THETA_DEN)
    return k.view(np.uint64)


def estimate_patterns(c, s):
    """The float32 estimates widened to float64 patterns; mask of normal estimates."""
    inv = (np.float32(1.0) / s.astype(np.float32)).astype(np.float32)
    kf = ((c[:, None] * THETA_F[None, :]).astype(np.float32) * inv[:, None]).astype(np.float32)
    b = kf.view(np.uint32).astype(np.uint64)
    e = b >> np.uint64(23)
    ok = (e > 0) & (e < 255)
    pat = ((e + np.uint64(896)) << np.uint64(52)) | ((b & np.uint64(0x7FFFFF)) << np.uint64(29))
    return pat, ok


def test_float32_key_estimates_stay_within_half_the_margin():
    rng = np.random.default_rng(11)
    n = 400_000
    c = np.exp2(rng.uniform(-120, 120, n)).astype(np.float32)
    c[:1000] = np.float32(1.0)                                   # exact powers of two
    c[1000:2000] = np.nextafter(np.float32(2.0), np.float32(0)) # just below a binade edge
    s = np.where(rng.random(n) < 0.5, 128, rng.integers(1, 1 << 29, n)).astype(np.int64)
    s[:500] = 64
    exact = exact_patterns(c, s)
    est, ok = estimate_patterns(c, s)
    mid = (c > 2.0 ** -60) & (c < 2.0 ** 60)
    assert ok[mid].all()                         # ordinary weights always get a usable estimate
    diff = np.where(ok, np.abs(exact.astype(np.int64) - est.astype(np.int64)), 0)
    assert diff.max() <= 2 ** 32, hex(int(diff.max()))


def test_estimates_order_like_the_keys():
    """Positive doubles order like their patterns, so an interval of patterns bounds the key: a
    planted pair of costs one float32 step apart keeps its order in both forms."""
    c = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0))], dtype=np.float32)
    s = np.array([128, 128], dtype=np.int64)
    exact = exact_patterns(c, s)
    assert np.all(exact[1] > exact[0])
