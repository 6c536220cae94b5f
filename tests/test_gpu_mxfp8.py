"""GPU parity of the MXFP8 reference round (quality report) against the oracle."""
import numpy as np
import pytest
import torch

from compressed_hop_gradient_amd import dq, synth
from oracle import pyoracle as po

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,J,n,topo", [("tiny", 256, 4, dq.RING), ("gemma", 2051, 8, dq.BUTTERFLY),
                                           ("bert", 777, 8, dq.RING), ("bert", 300, 1, dq.RING),
                                           ("llama", 513, 16, dq.BUTTERFLY), ("large", 97, 5, dq.RING)])
def test_mxfp8_round_bit_exact(name, J, n, topo):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grads = synth.generate(name, d=256 * J, device="cuda", workers=range(n))
    p = dq.Plan(256 * J, n, topo, 5.0)
    out = p.mxfp8_allreduce(grads).cpu().numpy()
    o = po.Oracle(256 * J, n, po.BUTTERFLY if topo == dq.BUTTERFLY else po.RING, 5.0)
    ref = o.mxfp8_allreduce([synth.as_numpy(g) for g in grads])
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", [dq.MX_FP8_E4M3, dq.MX_FP6_E3M2, dq.MX_FP6_E2M3, dq.MX_FP4_E2M1])
@pytest.mark.parametrize("name,J,n,topo", [("tiny", 256, 4, dq.RING), ("gemma", 1029, 8, dq.BUTTERFLY),
                                           ("bert", 300, 1, dq.RING), ("large", 97, 5, dq.RING)])
def test_mx_formats_round_bit_exact(fmt, name, J, n, topo):
    """FP8 E4M3, FP6 E3M2 / E2M3 and FP4 E2M1 element codes in the same
    schedule: the fp32 result against the oracle, bit for bit."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grads = synth.generate(name, d=256 * J, device="cuda", workers=range(n))
    p = dq.Plan(256 * J, n, topo, 5.0)
    out = p.mx_allreduce(fmt, grads).cpu().numpy()
    o = po.Oracle(256 * J, n, po.BUTTERFLY if topo == dq.BUTTERFLY else po.RING, 5.0)
    ref = o.mx_allreduce(fmt, [synth.as_numpy(g) for g in grads])
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    if fmt == dq.MX_FP8_E4M3:
        assert np.array_equal(p.mxfp8_allreduce(grads).cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_mx_format_rejected():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p = dq.Plan(256 * 4, 2, dq.RING, 5.0)
    g = [torch.zeros(1024, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    with pytest.raises(dq.DQError):
        p.mx_allreduce(4, g)
