"""Seeded synthetic gradients for the five workloads.

This module only draws inputs; it holds none of the method's arithmetic and
is shared by the tests and the benchmark.  The pages' own workloads (BERT-large,
Gemma 1B and LLaMA 1B fine-tuning) and their gradients are not available, so
these recipes stand in for them with the model sizes and with gradient norms
that are skewed across super-groups and spatially local (DynamiQ pith review,
Fig. 1 and Fig. 3 captions).

Every recipe is a function of (workload, data seed, worker).  Scales and
masks that describe the model (per block / per super-group / per embedding
row) are shared by all workers; the values themselves are drawn per worker.
Draws happen in fixed chunks of ``CHUNK`` coordinates, each with its own
seeded ``torch.Generator``, so results do not depend on memory limits.
bf16 gradients are the round-to-nearest-even bf16 of the fp32 draw.
"""
import math
from dataclasses import dataclass, field

import torch

CHUNK = 1 << 24  # coordinates per independently seeded draw


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    n: int
    topology: str          # "ring" | "butterfly"
    dtype: str             # "f32" | "bf16"
    budget: float = 5.0
    data_seed: int = 0
    rounding_seed: int = 1
    budgets: tuple = field(default=(5.0,))


WORKLOADS = {
    "tiny": Workload("tiny", 65_536, 4, "ring", "f32"),
    "bert": Workload("bert", 336_000_000, 8, "ring", "bf16"),
    "gemma": Workload("gemma", 1_000_000_000, 8, "butterfly", "bf16"),
    "llama": Workload("llama", 1_240_000_000, 16, "ring", "bf16", budgets=(3.0, 4.0, 5.0, 6.0)),
    "large": Workload("large", 4_300_000_000, 8, "ring", "bf16"),
}


def _mix(*xs):
    """splitmix64-style mixing of small integers into a 63-bit seed."""
    h = 0x9E3779B97F4A7C15
    for x in xs:
        h ^= (int(x) + 0x9E3779B97F4A7C15 + (h << 6) + (h >> 2)) & 0xFFFFFFFFFFFFFFFF
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*key))
    return g


def _student_t(nu, n, g, device):
    z = torch.randn((nu + 1, n), generator=g, device=device, dtype=torch.float32)
    chi2 = (z[1:] * z[1:]).sum(0) / nu
    return z[0] / torch.sqrt(chi2)


def _log_uniform(lo, hi, n, g, device):
    u = torch.rand(n, generator=g, device=device, dtype=torch.float32)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def _laplace(n, g, device):
    # a random sign times Exp(1) = -log(1 - U), U in [0, 1) so always finite
    e = -torch.log1p(-torch.rand(n, generator=g, device=device, dtype=torch.float32))
    sign = torch.where(torch.rand(n, generator=g, device=device) < 0.5, -1.0, 1.0)
    return sign * e


def _blocks(d, nblocks):
    return [(b * d // nblocks, (b + 1) * d // nblocks) for b in range(nblocks)]


class _Shared:
    """Per-model draws shared by every worker (scales, masks)."""

    def __init__(self, wl: Workload, d: int, device, seed: int):
        self.d = d
        self.J = d // 256
        g = _gen(device, seed, 0xC0FFEE)
        name = wl.name
        if name == "tiny":
            self.sg_scale = _log_uniform(1e-5, 1e-2, self.J, g, device)
        elif name == "bert":
            self.block_scale = _log_uniform(1e-6, 1e-3, 24, g, device)
            self.bounds = _blocks(d, 24)
        elif name == "gemma":
            rows = (262_144 * d) // 1_000_000_000
            self.emb = rows * 1000
            self.row_zero = torch.rand(rows, generator=g, device=device) < 0.9
            self.block_scale = _log_uniform(1e-6, 1e-3, 26, g, device)
            self.bounds = [(self.emb + a, self.emb + b) for a, b in _blocks(d - self.emb, 26)]
        elif name == "llama":
            self.sg_scale = torch.exp(math.log(1e-4) + 1.5 * torch.randn(self.J, generator=g, device=device))
        elif name == "large":
            self.sg_scale = _log_uniform(1e-7, 1e-2, self.J, g, device)
            self.sg_zero = torch.rand(self.J, generator=g, device=device) < 0.001
        else:
            raise ValueError(name)


def _block_scale_of(idx, bounds, scales):
    starts = torch.tensor([a for a, _ in bounds], device=idx.device, dtype=torch.int64)
    b = torch.searchsorted(starts, idx, right=True) - 1
    return scales[b.clamp(min=0)]


def _chunk_values(wl, sh, lo, hi, g, device):
    n = hi - lo
    idx = torch.arange(lo, hi, device=device, dtype=torch.int64)
    name = wl.name
    if name == "tiny":
        s = sh.sg_scale[idx // 256]
        x = torch.randn(n, generator=g, device=device) * s
        u = torch.rand(n, generator=g, device=device)
        sign = torch.where(torch.rand(n, generator=g, device=device) < 0.5, -1.0, 1.0)
        return torch.where(u < 0.01, sign * 10.0 * s, x)
    if name == "bert":
        return _block_scale_of(idx, sh.bounds, sh.block_scale) * _student_t(3, n, g, device)
    if name == "gemma":
        z = torch.randn(n, generator=g, device=device)
        lap = _laplace(n, g, device)
        in_emb = idx < sh.emb
        row = torch.clamp(idx // 1000, max=max(sh.row_zero.numel() - 1, 0))
        emb_sigma = torch.where(sh.row_zero[row], 1e-7, 1e-4) if sh.emb > 0 else torch.zeros_like(z)
        blk = _block_scale_of(idx, sh.bounds, sh.block_scale)
        return torch.where(in_emb, z * emb_sigma, lap * blk)
    if name == "llama":
        return sh.sg_scale[idx // 256] * _student_t(4, n, g, device)
    if name == "large":
        sg = idx // 256
        x = sh.sg_scale[sg] * _student_t(3, n, g, device)
        return torch.where(sh.sg_zero[sg], torch.zeros_like(x), x)
    raise ValueError(name)


def generate(name, d=None, device="cpu", seed=None, workers=None):
    """Return the list of per-worker gradients (torch tensors on ``device``).

    ``d`` overrides the coordinate count (a multiple of 256) for scaled-down
    versions of a workload with the same structure.
    """
    wl = WORKLOADS[name]
    d = wl.d if d is None else int(d)
    assert d % 256 == 0 and d > 0
    seed = wl.data_seed if seed is None else seed
    workers = range(wl.n) if workers is None else workers
    sh = _Shared(wl, d, device, seed)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    out = []
    for w in workers:
        g_out = torch.empty(d, dtype=dt, device=device)
        for c0 in range(0, d, CHUNK):
            c1 = min(d, c0 + CHUNK)
            g = _gen(device, seed, w + 1, c0 // CHUNK)
            g_out[c0:c1] = _chunk_values(wl, sh, c0, c1, g, device).to(dt)
        out.append(g_out)
    return out


def as_numpy(t):
    """Host copy: float32 stays float32, bf16 becomes its raw uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
