"""The seeded input generator: finite values, determinism, structure."""
import numpy as np
import pytest
import torch

from compressed_hop_gradient_amd import synth


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_finite_and_deterministic(name):
    d = 256 * 4099
    a = synth.generate(name, d=d, workers=range(2))
    b = synth.generate(name, d=d, workers=range(2))
    for x, y in zip(a, b):
        assert x.shape == (d,)
        assert torch.isfinite(x.float()).all()
        assert torch.equal(x, y)
    assert not torch.equal(a[0], a[1])          # values differ per worker
    dt = torch.float32 if synth.WORKLOADS[name].dtype == "f32" else torch.bfloat16
    assert a[0].dtype == dt


def test_structure():
    d = 256 * 8000
    g = synth.generate("large", d=d, workers=range(2))
    z0 = (g[0].view(-1, 256) == 0).all(1)
    z1 = (g[1].view(-1, 256) == 0).all(1)
    assert torch.equal(z0, z1) and 0 < int(z0.sum()) < 40    # shared 0.1% zero super-groups
    g = synth.generate("gemma", d=d, workers=range(1))[0].float()
    emb = (262_144 * d) // 1_000_000_000 * 1000
    rows = g[:emb].view(-1, 1000).abs().amax(1)
    frac_small = float((rows < 1e-6).float().mean())
    assert 0.85 < frac_small < 0.95                            # 90% near-zero embedding rows
    h = synth.as_numpy(synth.generate("bert", d=256, workers=range(1))[0])
    assert h.dtype == np.uint16
