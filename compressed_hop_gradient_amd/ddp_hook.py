"""PyTorch DDP communication hook running DynamiQ on each gradient bucket.

The pages integrate DynamiQ with PyTorch DDP (mlsanity abstract; scribe notes,
"Evaluation").  A DDP comm hook receives one flattened gradient bucket per call
and returns a future of the reduced bucket.  This hook maps a bucket to a
DynamiQ round:

  * the bucket (fp32 or bf16) is copied into a zero-padded buffer whose length
    is the next multiple of 256 (a super-group); padding super-groups are all
    zero and decode to exactly zero;
  * one plan per (padded length, dtype) is created on first use and reused on
    every later step, with its workspace, region arena and output; the plan's
    round index is the step count of that bucket, so every step draws fresh
    dithers;
  * the round's fp32 output (the sum over workers) is divided by the world
    size for ``reduce="mean"`` (what DDP's default all-reduce hook returns),
    cast to the bucket dtype (round to nearest even for bf16) and written back
    into the bucket.

The workers of the round are the ranks of the process group.  Only one rank
(one GPU) is supported here: the multi-GPU transport (point-to-point region
hand-offs and the statistics all-reduce over RCCL) is not built, and a group
of more than one rank is refused.  All work is enqueued on the current stream;
no device memory is allocated after a bucket size's first step.
"""
import torch
import torch.distributed as dist

from . import dq


def padded_length(numel):
    """The bucket length rounded up to whole super-groups of 256."""
    return max(256, (int(numel) + 255) // 256 * 256)


class DynamiQHookState:
    """Per-process hook state: options of the rounds and the plan cache."""

    def __init__(self, process_group=None, avg_bits=5.0, topology=dq.RING, seed=1,
                 rounding=dq.STRATIFIED, reduce="mean"):
        if reduce not in ("mean", "sum"):
            raise ValueError("reduce must be 'mean' or 'sum'")
        self.process_group = process_group
        self.avg_bits = float(avg_bits)
        self.topology = topology
        self.seed = seed
        self.rounding = rounding
        self.reduce = reduce
        self.entries = {}      # (padded length, dtype, device) -> _Entry

    def world_size(self):
        return dist.get_world_size(self.process_group)

    def entry(self, n, dtype, device):
        key = (n, dtype, str(device))
        e = self.entries.get(key)
        if e is None:
            e = _Entry(self, n, dtype, device)
            self.entries[key] = e
        return e


class _Entry:
    """Plan and buffers of one bucket shape, reused across steps."""

    def __init__(self, state, n, dtype, device):
        self.plan = dq.Plan(n, 1, state.topology, state.avg_bits, seed=state.seed,
                            rounding=state.rounding, device=device)
        self.grad = torch.zeros(n, dtype=dtype, device=device)
        self.arena = torch.empty(self.plan.arena_bytes(), dtype=torch.uint8, device=device)
        self.out = torch.empty(n, dtype=torch.float32, device=device)
        self.step = 0


def reduce_bucket(state, flat):
    """Run the round on one flattened gradient ``flat`` and write the result
    back in place; returns ``flat``."""
    world = state.world_size()
    if world != 1:
        raise NotImplementedError(
            f"DynamiQ DDP hook: {world} ranks; only a single-rank group is supported "
            "(the multi-GPU transport is not built)")
    if flat.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"DynamiQ DDP hook: bucket dtype {flat.dtype} (fp32 or bf16 only)")
    numel = flat.numel()
    e = state.entry(padded_length(numel), flat.dtype, flat.device)
    e.grad[:numel].copy_(flat)
    e.plan.set(dq.OPT_ROUND, e.step & 0xFFFFFFFF)
    e.step += 1
    e.plan.allreduce([e.grad], out=e.out, arena=e.arena)
    res = e.out[:numel]
    if state.reduce == "mean" and world > 1:
        res = res / world
    flat.copy_(res)
    return flat


def dynamiq_hook(state, bucket):
    """DDP comm hook: ``model.register_comm_hook(state, dynamiq_hook)``."""
    flat = reduce_bucket(state, bucket.buffer())
    fut = torch.futures.Future()
    fut.set_result(flat)
    return fut
