"""The DynamiQ DDP comm hook in a one-rank process group (RCCL backend on
cuda:0): buckets of a small model's real gradients, fp32 and bf16, against the
oracle's one-worker round on the same bytes (padded to whole super-groups, the
hook's round index), bit for bit."""
import os
import socket

import numpy as np
import pytest
import torch

from compressed_hop_gradient_amd import ddp_hook, dq
from oracle import pyoracle as po

pytestmark = pytest.mark.gpu


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _bf16_rne(x):
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = x.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.fixture(scope="module")
def group():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import torch.distributed as dist
    torch.cuda.set_device(0)
    dist.init_process_group("nccl", init_method=f"tcp://127.0.0.1:{_free_port()}", rank=0,
                            world_size=1)
    yield dist.group.WORLD
    dist.destroy_process_group()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_ddp_hook_one_rank_matches_oracle(group, dtype):
    from torch.nn.parallel import DistributedDataParallel as DDP
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(300, 257), torch.nn.GELU(),
                                torch.nn.Linear(257, 129), torch.nn.GELU(),
                                torch.nn.Linear(129, 10)).to("cuda", dtype)
    ddp = DDP(model, device_ids=[0], bucket_cap_mb=0.25)
    state = ddp_hook.DynamiQHookState(process_group=group, avg_bits=5.0)
    seen = []

    def hook(st, bucket):
        raw = bucket.buffer().detach().clone()
        e = st.entry(ddp_hook.padded_length(raw.numel()), raw.dtype, raw.device)
        rnd = e.step
        fut = ddp_hook.dynamiq_hook(st, bucket)
        seen.append((raw, bucket.buffer().detach().clone(), rnd))
        return fut

    ddp.register_comm_hook(state, hook)
    x = torch.randn(64, 300, device="cuda", dtype=dtype)
    for _ in range(3):
        ddp.zero_grad()
        ddp(x).float().square().mean().backward()
    torch.cuda.synchronize()
    # one call per bucket and step; each bucket shape's plan is made once and reused
    assert len(seen) >= 3 and len(state.entries) >= 1
    assert sum(e.step for e in state.entries.values()) == len(seen)
    assert any(raw.numel() % 256 for raw, _, _ in seen)       # a padded bucket
    for raw, got, rnd in seen:
        n = raw.numel()
        npad = ddp_hook.padded_length(n)
        if dtype == torch.float32:
            g = np.zeros(npad, np.float32)
            g[:n] = raw.cpu().numpy()
        else:
            g = np.zeros(npad, np.uint16)
            g[:n] = raw.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = po.Oracle(npad, 1, po.RING, 5.0, seed=1, rnd=rnd, rounding=po.STRATIFIED).allreduce([g])[:n]
        if dtype == torch.float32:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        else:
            assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), _bf16_rne(ref))
    # the gradients the optimiser sees are the hook's output
    p0 = next(model.parameters())
    assert p0.grad is not None and torch.isfinite(p0.grad.float()).all()
