"""Facts about the hardware that the codec kernels rely on, checked on the GPU
through the library's own device functions.

The codecs compute v = y * fl(1/sigma) with one Newton step on the hardware
reciprocal where sigma lies in [2^-126, 2^126), and with the IEEE division
elsewhere.  Bit-exact parity with the oracle needs that reciprocal to be the
correctly rounded quotient: checked here for every fp32 bit pattern.  The
rounding decision uses the hardware's round-half-up conversion, checked the
same way."""
import pytest
import torch

from compressed_hop_gradient_amd import dq

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_reciprocal_is_correctly_rounded_for_every_float():
    _need_gpu()
    # all 2^32 bit patterns in two halves (the count argument is 32-bit)
    bad = dq.check_reciprocal(0, 1 << 31) + dq.check_reciprocal(1 << 31, 1 << 31)
    assert bad == 0


def test_reciprocal_fast_range_edges():
    _need_gpu()
    lo, hi = 0x00800000, 0x7E800000          # 2^-126 .. 2^126: the Newton-step range
    assert dq.check_reciprocal(lo - 4096, 8192) == 0
    assert dq.check_reciprocal(hi - 4096, 8192) == 0


def test_round_half_up_is_exact_for_every_float():
    """The codec's rounding decision d + 0.5 <= P is evaluated as
    d < floor(P + 0.5) with the hardware's round-half-up conversion: it must
    equal the exact floor(x + 0.5) for every fp32 bit pattern (saturated
    beyond the int32 range; NaN saturates by its sign bit)."""
    _need_gpu()
    bad = dq.check_round_half_up(0, 1 << 31) + dq.check_round_half_up(1 << 31, 1 << 31)
    assert bad == 0
