"""Facts about the level tables that the HIP kernels rely on, checked on the
tables of the reading (generated here and by the oracle), on the CPU.

1. The kernels skip the clamp of v to [-1, 1]: just above +1 the rounding-up
   threshold P of the last interval already exceeds every d + 0.5 (d < 2^16),
   and just below -1 it is negative, so codes cannot change.
2. The interval search looks up a linear bucket of v, NB/2 + rne(v M) with
   M = NB/2 - 1 (NB = 1024 buckets for 16 levels, 8192 for 256), computed as
   the bits of one FMA on the subnormal grid, clamped to [0, 1]:
   fl(fma(v, M 2^-149, (NB/2) 2^-149)).  That identity holds for every fp32
   v in [-1, 1] and 1024 ulps beyond, and NaN lands in bucket 0 (tests/
   native/bucket_check.c); the interior levels fall in strictly increasing
   buckets for level shapes eps from 0.0274 to 1 (the plan refuses smaller
   eps), so each bucket holds at most one level boundary.
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


def _buckets(v, q):
    NB = 1024 if q == 4 else 8192
    return NB // 2 + np.rint(v.astype(np.float64) * (NB // 2 - 1)).astype(np.int64)


@pytest.mark.parametrize("q", [4, 8])
@pytest.mark.parametrize("eps", [1.0, 0.75, 0.5, 0.3, 0.1, 0.05, 0.03, 0.0274])
def test_buckets_hold_at_most_one_boundary(q, eps):
    """The interior levels L[1..2^q-2] of the oracle's table fall in strictly
    increasing linear buckets, all inside the table, for level shapes from
    eps = 0.0274 to the uniform grid."""
    L, _ = po.levels(q, eps)
    b = _buckets(L[1:-1], q)
    assert np.all(np.diff(b) > 0)
    assert b.min() >= 0 and b.max() < (1024 if q == 4 else 8192)


def test_small_level_shapes_are_refused():
    """Below eps = 0.0273 the two central 8-bit levels share a bucket: the
    library refuses such a shape (the plan option returns DQ_EINVAL)."""
    import ctypes as C
    from compressed_hop_gradient_amd import dq
    L, _ = po.levels(8, 0.027)
    b = _buckets(L[1:-1], 8)
    assert np.any(np.diff(b) == 0)
    lib = dq.lib()
    h = C.c_void_p()
    assert lib.dq_plan_create(256 * 4, 1, dq.RING, C.c_float(5.0), C.byref(h)) == dq.DQ_OK
    assert lib.dq_plan_set_f64(h, dq.OPT_EPS, C.c_double(0.027)) == dq.DQ_EINVAL
    assert lib.dq_plan_set_f64(h, dq.OPT_EPS, C.c_double(0.0274)) == dq.DQ_OK
    lib.dq_plan_destroy(h)


def test_linear_bucket_is_one_subnormal_fma(tmp_path):
    """The kernels' bucket, the bits of fl(fma(v, M 2^-149, (NB/2) 2^-149))
    clamped to [0, 1] (the FMA's output modifier; NaN gives +0), equals
    NB/2 + rne(v M), stays inside the table and never decreases, for v from
    -(1 + 1024 ulp) to 1 + 1024 ulp (both table sizes; the encoder's |v| is
    at most 1 + 2^-22): every fp32 v with |v| >= 2^-14 and every 64th bit
    pattern below, where the key is NB/2.  Every NaN lands in bucket 0."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(os.path.dirname(__file__), "native", "bucket_check.c")
    exe = str(tmp_path / "bucket_check")
    if subprocess.run([cc, "-O2", "-fopenmp", "-mfma", "-ffp-contract=off", "-o", exe, src, "-lm"]).returncode:
        subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    checked, bad, dec, outside, nan_ok = (int(x) for x in out)
    b14, top = 0x38800000, 0x3F800000 + 1024
    assert checked == 2 * (top - b14 + 1) + 2 * ((b14 + 63) // 64)
    assert bad == 0 and dec == 0 and outside == 0 and nan_ok == 1


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
