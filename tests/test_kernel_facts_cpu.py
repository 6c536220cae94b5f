"""Facts about the level tables that the HIP kernels rely on, checked on the
tables of the reading (generated here and by the oracle), on the CPU.

1. The kernels skip the clamp of v to [-1, 1]: just above +1 the rounding-up
   threshold P of the last interval already exceeds every d + 0.5 (d < 2^16),
   and just below -1 it is negative, so codes cannot change.
2. The interval search looks up a bucket of v keyed by the sign, the exponent
   and 7 mantissa bits of |v| (all |v| < 2^-12 share one bucket): each bucket
   holds at most one level boundary, for level shapes eps from 0.01 to 1.
"""
import os

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
@pytest.mark.parametrize("eps", [1.0, 0.75, 0.5, 0.3, 0.1, 0.05, 0.01])
def test_buckets_hold_at_most_one_boundary(q, eps):
    """Buckets of 7 mantissa bits per exponent of |v|, all |v| < 2^-12 in one
    bucket: at most one level boundary per bucket, for level shapes from
    eps = 0.01 to the uniform grid."""
    L, _ = po.levels(q, eps)
    base, kmax = 0x3980, 0x3F80 - 0x3980
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


def test_higher_tiny_bucket_would_fail_small_shapes():
    """Were the shared bucket of tiny |v| to end at 2^-9, the 8-bit levels of
    eps = 0.1 would put two boundaries into it: ending it at 2^-12 is what
    admits the small shapes."""
    L, _ = po.levels(8, 0.1)
    assert ((L > 0) & (L < np.float32(2.0 ** -9))).sum() >= 2
    assert ((L > 0) & (L < np.float32(2.0 ** -12))).sum() <= 1


def test_scale_unit_division_by_255_with_two_fmas(tmp_path):
    """The codec kernels compute the scale unit's first guess fl(A / 255) as
    y = fl(A R), r = fma(-y, 255, A), q = fma(r, R, y) with R = fl(1/255).
    Checked here for every non-negative finite fp32 A (all 255 exponent
    fields, subnormals included; about 20 s, most of it in the subnormal
    binades)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(os.path.dirname(__file__), "native", "div255_check.c")
    exe = str(tmp_path / "div255_check")
    # hardware FMA where the host has it (glibc's fmaf is correctly rounded either way)
    if subprocess.run([cc, "-O2", "-mfma", "-ffp-contract=off", "-o", exe, src, "-lm"]).returncode:
        subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
    ranges = ["0", "254"]
    out = subprocess.run([exe] + ranges, check=True, capture_output=True, text=True).stdout.split()
    checked, bad, second = int(out[0]), int(out[1]), int(out[2])
    assert checked == 255 * (1 << 23)
    assert bad == 0
    # the scale unit's raise loop stops after at most one step
    assert second == 0
