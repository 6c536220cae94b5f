"""Facts about the level tables that the HIP kernels rely on, checked on the
tables of the reading (generated here and by the oracle), on the CPU.

1. The kernels skip the clamp of v to [-1, 1]: just above +1 the rounding-up
   threshold P of the last interval already exceeds every d + 0.5 (d < 2^16),
   and just below -1 it is negative, so codes cannot change.
2. The interval search looks up a bucket of v keyed by the sign, the exponent
   and 7 mantissa bits of |v| (all |v| < 2^-9 share one bucket): each bucket
   holds at most one level boundary.
"""
import numpy as np
import pytest

from oracle import pyoracle as po


def f32(x):
    return np.float32(x)


@pytest.mark.parametrize("q", [2, 4, 8])
def test_no_clamp_needed_at_the_ends(q):
    L, W = po.levels(q)
    Q = 1 << q
    one = f32(1.0)
    v = one
    for _ in range(4):   # 1 and the next three floats above it
        P = f32(f32(v - L[Q - 2]) * W[Q - 2])
        assert P > f32(65535.5), (q, v, P)
        v = np.nextafter(v, f32(2.0))
    v = f32(-1.0)
    for _ in range(4):
        v = np.nextafter(v, f32(-2.0))
        P = f32(f32(v - L[0]) * W[0])
        assert P < 0
    # |v| overshoots 1 by at most a few ulps: |y| <= sigma and v = y * fl(1/sigma)
    rng = np.random.default_rng(q)
    sig = rng.uniform(1e-30, 1e30, 200000).astype(np.float32)
    inv = (f32(1.0) / sig).astype(np.float32)
    v = (sig * inv).astype(np.float32)
    assert np.all(v <= np.nextafter(np.nextafter(one, f32(2)), f32(2)))


@pytest.mark.parametrize("q", [4, 8])
def test_buckets_hold_at_most_one_boundary(q):
    L, _ = po.levels(q)
    base, kmax = 0x3B00, 0x3F80 - 0x3B00
    keys = np.arange(kmax + 1, dtype=np.uint32)
    lo = ((keys + base) << 16).view(np.float32).copy()
    lo[0] = 0.0
    hi = ((keys + 1 + base) << 16).view(np.float32).copy()
    hi[kmax] = 1.0
    Lp = L.astype(np.float64)
    # v >= 0 in [lo, hi): levels strictly inside (lo, hi)
    inside = ((Lp[None, :] > lo[:, None]) & (Lp[None, :] < hi[:, None])).sum(1)
    assert inside.max() <= 1
    # v < 0 in (-hi, -lo]
    inside = ((Lp[None, :] > -hi[:, None]) & (Lp[None, :] <= -lo[:, None])).sum(1)
    assert inside.max() <= 1
    # the smallest positive level is above the shared bucket of tiny |v|
    assert L[(1 << q) // 2] > np.float32(2.0 ** -9) * np.float32(1 + 2.0 ** -7) or q == 4
