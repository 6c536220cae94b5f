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
