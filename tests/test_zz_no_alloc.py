"""dq_allreduce_noalloc: the whole round with the plan state and the region
arena in the library's static device scratch, against dq_allreduce with
caller buffers, bit for bit; two calls in a row share the scratch, the second
on a smaller input."""
import ctypes as C

import pytest
import torch

from compressed_hop_gradient_amd import dq, synth

pytestmark = pytest.mark.gpu


def _noalloc(plan, grads, out):
    ptrs = (C.c_void_p * plan.n)(*[g.data_ptr() for g in grads])
    kind = dq.BF16 if grads[0].dtype == torch.bfloat16 else dq.F32
    return dq.lib().dq_allreduce_noalloc(plan.h, ptrs, kind, C.c_void_p(out.data_ptr()),
                                         C.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_round_matches_allreduce_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    cases = [("gemma", 20_000, 8, dq.BUTTERFLY), ("bert", 3_001, 4, dq.RING)]
    lib = dq.lib()
    limit = lib.dq_noalloc_max_bytes()
    for name, J, n, topo in cases:
        print(f"[noalloc] {name}: {J} super-groups x {n} workers", flush=True)
        grads = synth.generate(name, d=256 * J, device="cuda", workers=range(n))
        ref_plan = dq.Plan(256 * J, n, topo, 5.0, seed=3)
        need = ((ref_plan.layout["total"] + 255) // 256) * 256 + ref_plan.arena_bytes()
        assert need <= limit
        ref = ref_plan.allreduce(grads)
        plan = dq.Plan(256 * J, n, topo, 5.0, seed=3)
        out = torch.full((256 * J,), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(plan, grads, out) == dq.DQ_OK
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
        # the plan's state lives in the scratch now: the allocation it reports
        # is the reference plan's
        a, b = plan.info(), ref_plan.info()
        assert (a["rho_bits"], a["class_counts"]) == (b["rho_bits"], b["class_counts"])


def test_noalloc_rejects_a_round_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = dq.lib()
    limit = lib.dq_noalloc_max_bytes()
    J, n = 400_000, 8            # about 2 x 110 MB of arena: beyond 64 MiB
    plan = dq.Plan(256 * J, n, dq.RING, 5.0)
    assert plan.layout["total"] + plan.arena_bytes() > limit
    grads = [torch.zeros(256 * J, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    out = torch.full((256 * J,), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc(plan, grads, out) == dq.DQ_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
