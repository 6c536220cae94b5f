"""Argument checks of the Python binding, on the CPU.

The C ABI takes bare pointers, so the binding rejects what the kernels could
not address safely -- tensors on another device, non-contiguous views,
buffers shorter than the schedule step reads or writes -- before any call
into the library.  The plans here have no bound workspace: a call that gets
past the binding's checks is answered by the library with DQ_EWORKSPACE,
before any launch."""
import ctypes as C
from types import SimpleNamespace

import pytest
import torch

from compressed_hop_gradient_amd import dq


def _plan(n_coords, n, topo, own=dq.OWN_PACKED):
    h = C.c_void_p()
    assert dq.lib().dq_plan_create(n_coords, n, topo, 5.0, C.byref(h)) == dq.DQ_OK
    p = dq.Plan.__new__(dq.Plan)
    p.h = h
    p.d, p.n, p.J, p.topology = n_coords, n, n_coords // 256, topo
    p.log2n = max(0, (n - 1).bit_length())
    p.own = own
    p.device = torch.device("cpu")
    p.set(dq.OPT_OWN, own)
    return p


# the null stream, passed explicitly (the default asks torch for the current
# GPU stream)
NULL_STREAM = SimpleNamespace(cuda_stream=0)


def _passes(fn, *args, **kw):
    """The binding forwarded the call: the library refused it for the
    missing workspace, not for its arguments."""
    with pytest.raises(dq.DQError) as e:
        fn(*args, stream=NULL_STREAM, **kw)
    assert e.value.status == dq.DQ_EWORKSPACE


def _region(p, m, short=0):
    return torch.zeros(p.region_bytes_max(m) - short, dtype=torch.uint8)


def test_plan_needs_gpu_workspace():
    with pytest.raises(ValueError):
        dq.Plan(256 * 4, 2, dq.RING, 5.0, device="cpu")


def test_stats_and_compress_check_the_gradient_and_region():
    p = _plan(256 * 10, 4, dq.RING)
    g = torch.zeros(p.d, dtype=torch.bfloat16)
    _passes(p.stats, 0, g)
    with pytest.raises(ValueError):
        p.stats(0, g[:-256])                                    # too short
    with pytest.raises(ValueError):
        p.stats(0, torch.zeros(2 * p.d, dtype=torch.bfloat16)[::2])   # strided view
    with pytest.raises(ValueError):
        p.stats(0, torch.zeros(p.d, dtype=torch.bfloat16, device="meta"))   # another device
    with pytest.raises(TypeError):
        p.stats(0, [0.0] * p.d)
    _passes(p.compress, 0, 0, g, _region(p, 4))                 # ring: a part of m = n
    with pytest.raises(ValueError):
        p.compress(0, 0, g, _region(p, 4, short=1))


def test_butterfly_compress_writes_a_half():
    p = _plan(256 * 64, 8, dq.BUTTERFLY)
    g = torch.zeros(p.d, dtype=torch.float32)
    assert p._m_compress() == 2
    _passes(p.compress, 0, 1, g, _region(p, 2))
    with pytest.raises(ValueError):
        p.compress(0, 1, g, _region(p, 4))                      # sized for a quarter


def test_hop_region_sizes_follow_the_schedule():
    p = _plan(256 * 64, 8, dq.BUTTERFLY)
    g = torch.zeros(p.d, dtype=torch.bfloat16)
    assert [p._m_hop(s) for s in (0, 1, 2, 3, 4)] == [None, (2, 4), (4, 8), (8, 8), None]
    # level 1: the half in, both quarters out
    _passes(p.hop, 0, 1, _region(p, 2), g, _region(p, 4), _region(p, 4))
    with pytest.raises(ValueError):
        p.hop(0, 1, _region(p, 2, short=16), g, _region(p, 4), _region(p, 4))
    with pytest.raises(ValueError):
        p.hop(0, 1, _region(p, 2), g, _region(p, 4), _region(p, 4, short=1))
    # level 2: the own packed quarter is the local operand
    _passes(p.hop, 0, 2, _region(p, 4), _region(p, 4), _region(p, 8), _region(p, 8))
    with pytest.raises(ValueError):
        p.hop(0, 2, _region(p, 4), _region(p, 8), _region(p, 8), _region(p, 8))
    # last level with the decoded sum
    out = torch.zeros(p.d, dtype=torch.float32)
    _passes(p.hop_finalize, 0, 3, _region(p, 8), _region(p, 8), _region(p, 8), out)
    with pytest.raises(ValueError):
        p.hop_finalize(0, 3, _region(p, 8), _region(p, 8), _region(p, 8), out[:-1])
    with pytest.raises(TypeError):
        p.hop_finalize(0, 3, _region(p, 8), _region(p, 8), _region(p, 8), out.to(torch.float64))
    # a step outside the schedule goes to the library, which rejects it
    _passes(p.hop, 0, 4, _region(p, 8), g, _region(p, 8))


def test_own_fp32_kept_child_is_a_partial_buffer():
    p = _plan(256 * 64, 4, dq.BUTTERFLY, own=dq.OWN_F32)
    g = torch.zeros(p.d, dtype=torch.bfloat16)
    part = torch.zeros(p.partial_bytes_max(4) // 4, dtype=torch.float32)
    for w in range(4):
        keep = (w >> 0) & 1          # level 1 of 2: the child bit is w's lowest
        outs = [None, None]
        outs[keep] = part
        outs[1 - keep] = _region(p, 4)
        _passes(p.hop, w, 1, _region(p, 2), g, outs[0], outs[1])
        outs[keep] = _region(p, 4)   # a region is too small for the fp32 partial
        with pytest.raises(ValueError):
            p.hop(w, 1, _region(p, 2), g, outs[0], outs[1])
    # level 2 reads the kept partial as its local operand
    _passes(p.hop, 0, 2, _region(p, 4), part, _region(p, 4), local_kind=dq.F32_PARTIAL)
    with pytest.raises(ValueError):
        p.hop(0, 2, _region(p, 4), part[:-1], _region(p, 4), local_kind=dq.F32_PARTIAL)


def test_ring_hop_and_finalize():
    p = _plan(256 * 12, 3, dq.RING)
    g = torch.zeros(p.d, dtype=torch.float32)
    out = torch.zeros(p.d, dtype=torch.float32)
    _passes(p.hop, 1, 1, _region(p, 3), g, _region(p, 3))
    with pytest.raises(ValueError):
        p.hop(1, 1, _region(p, 3), g[:-1], _region(p, 3))
    _passes(p.finalize, 0, _region(p, 3), out)
    with pytest.raises(ValueError):
        p.finalize(0, _region(p, 3, short=256), out)


def test_whole_round_checks_every_gradient():
    p = _plan(256 * 8, 4, dq.RING)
    gs = [torch.zeros(p.d, dtype=torch.bfloat16) for _ in range(4)]
    arena = torch.zeros(8, dtype=torch.uint8)      # the library checks the arena size
    out = torch.zeros(p.d, dtype=torch.float32)
    _passes(p.allreduce, gs, out=out, arena=arena)
    with pytest.raises(ValueError):
        p.allreduce(gs[:3], out=out, arena=arena)
    with pytest.raises(TypeError):
        p.allreduce(gs[:3] + [gs[3].float()], out=out, arena=arena)
    with pytest.raises(ValueError):
        p.allreduce(gs[:3] + [gs[3][:-256]], out=out, arena=arena)
    with pytest.raises(ValueError):
        p.mxfp8_allreduce(gs, out=out[:-1], arena=arena)
