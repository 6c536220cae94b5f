"""Host logic of the DDP comm hook (no GPU): bucket padding to whole
super-groups, and refusal of a group of more than one rank (the multi-GPU
transport is not built) in a two-rank gloo group on the CPU."""
import os
import socket

import pytest
import torch
import torch.multiprocessing as mp


def test_padded_length():
    from compressed_hop_gradient_amd.ddp_hook import padded_length
    assert [padded_length(n) for n in (1, 255, 256, 257, 512, 100000)] == [256, 256, 256, 512, 512, 100096]


def _rank(rank, port, path):
    import torch.distributed as dist
    from compressed_hop_gradient_amd import ddp_hook
    dist.init_process_group("gloo", init_method=f"tcp://127.0.0.1:{port}", rank=rank, world_size=2)
    state = ddp_hook.DynamiQHookState()
    msg = "no error"
    try:
        ddp_hook.reduce_bucket(state, torch.zeros(1000))
    except NotImplementedError as e:
        msg = str(e)
    with open(f"{path}.{rank}", "w") as f:
        f.write(msg)
    dist.barrier()
    dist.destroy_process_group()


def test_hook_refuses_more_than_one_rank(tmp_path):
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        port = s.getsockname()[1]
    mp.spawn(_rank, args=(port, str(tmp_path / "r")), nprocs=2, join=True)
    for r in range(2):
        msg = (tmp_path / f"r.{r}").read_text()
        assert "2 ranks" in msg and "single-rank" in msg
