"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, stage by stage, bit for bit.

Compared in order: per-SG sums and squared norms, rho, widths, perm / inv,
mean in stream order, every region every hop writes (codes, scale units,
group codes), and the final fp32 sum.  The first mismatch names its stage.
"""
import numpy as np
import pytest
import torch

from compressed_hop_gradient_amd import dq, synth
from oracle import pyoracle as po
from tests import regions as R

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _np(t):
    return synth.as_numpy(t)


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _grads_np(grads):
    return [_np(g) for g in grads]


def _schedule(n, topo):
    """Yield the steps of one round: ('compress', w, step) / ('hop', w, step)."""
    if n == 1:
        yield ("compress", 0, 0)
        return
    if topo == dq.RING:
        for w in range(n):
            yield ("compress", w, 0)
        for t in range(1, n):
            for w in range(n):
                yield ("hop", w, t)
        return
    L = n.bit_length() - 1
    for w in range(n):
        yield ("compress", w, 1)
    for s in range(1, L + 1):
        for w in range(n):
            yield ("hop", w, s)


def _out_parts(n, topo, kind, w, step):
    """(m, part) of each output region of a step."""
    if n == 1:
        return [(1, 0)]
    if topo == dq.RING:
        return [(n, w if kind == "compress" else (w - step) % n)]
    L = n.bit_length() - 1
    if kind == "compress":
        return [(2, (w >> (L - 1)) ^ 1)]
    c = w >> (L - step)
    if step < L:
        return [(2 ** (step + 1), 2 * c), (2 ** (step + 1), 2 * c + 1)]
    return [(n, c)]


class Round:
    """Drives the same schedule on the GPU and on the oracle, keeping every
    region both produce (fresh zeroed buffers per step)."""

    def __init__(self, grads, topo, budget=5.0, seed=1, rnd=0, rounding=dq.STRATIFIED,
                 alloc=dq.ALLOC_THRESHOLD, eps=None, max_width=8):
        self.grads = grads
        self.gnp = _grads_np(grads)
        self.n = len(grads)
        self.d = grads[0].numel()
        self.topo = topo
        self.plan = dq.Plan(self.d, self.n, topo, budget, seed=seed, rnd=rnd, rounding=rounding,
                            alloc=alloc, eps=eps, max_width=max_width)
        self.orc = po.Oracle(self.d, self.n, topo, budget, seed=seed, rnd=rnd, rounding=rounding,
                             alloc=alloc, eps=eps, max_width=max_width)

    def stages(self):
        for w in range(self.n):
            self.plan.stats(w, self.grads[w])
            self.orc.stats(w, self.gnp[w])
        self.plan.allocate()
        self.orc.allocate()
        self.plan.reorder()
        self.orc.reorder()
        torch.cuda.synchronize()

    def check_stages(self):
        s_g, F_g = [x.cpu().numpy() for x in self.plan.stats_arrays()]
        s_o, F_o, mu_o = self.orc.stats_arrays()
        assert np.array_equal(_bits(s_g), _bits(s_o)), "stats: sum"
        assert np.array_equal(_bits(F_g), _bits(F_o)), "stats: squared norm"
        info = self.plan.info()
        assert not info["nonfinite"], "inputs must be finite"
        assert info["rho_bits"] == self.orc.rho_bits(), "allocate: rho"
        assert np.array_equal(self.plan.widths().cpu().numpy(), self.orc.widths()), "allocate: widths"
        C = self.orc.class_counts()
        assert list(info["class_counts"]) == C.tolist(), "allocate: class counts"
        assert info["used_bits"] <= info["budget_bits"]
        perm_g, inv_g = [x.cpu().numpy() for x in self.plan.perm()]
        perm_o, inv_o = self.orc.perm()
        assert np.array_equal(perm_g, perm_o), "reorder: perm"
        assert np.array_equal(inv_g, inv_o), "reorder: inv"
        mus = self.plan.mu_stream().cpu().numpy()
        assert np.array_equal(_bits(mus), _bits(mu_o[perm_o])), "reorder: mean in stream order"
        self.C = C
        return info

    def run_hops(self, check_every=True):
        n, topo = self.n, self.topo
        g_reg, o_reg = {}, {}
        L = max(0, n.bit_length() - 1)
        for kind, w, step in _schedule(n, topo):
            parts = _out_parts(n, topo, kind, w, step)
            gout = [self.plan.new_region(m) for m, _ in parts]
            oout = [np.zeros(self.orc.worst_region_bytes(), np.uint8) for _ in parts]
            if kind == "compress":
                self.plan.compress(w, step, self.grads[w], gout[0])
                self.orc.compress(w, step, self.gnp[w], oout[0])
            else:
                if topo == dq.RING:
                    key_in = ((w - 1) % n, step - 1)
                    g_in, o_in = g_reg[key_in][0], o_reg[key_in][0]
                    g_loc, o_loc = self.grads[w], self.gnp[w]
                else:
                    partner = w ^ (n >> step)
                    keep = (w >> (L - step)) & 1
                    if step == 1:
                        g_in, o_in = g_reg[(partner, "c")][0], o_reg[(partner, "c")][0]
                        g_loc, o_loc = self.grads[w], self.gnp[w]
                    else:
                        g_in, o_in = g_reg[(partner, step - 1)][keep], o_reg[(partner, step - 1)][keep]
                        g_loc, o_loc = g_reg[(w, step - 1)][keep], o_reg[(w, step - 1)][keep]
                self.plan.hop(w, step, g_in, g_loc, gout[0], gout[1] if len(gout) > 1 else None)
                self.orc.hop(w, step, o_in, o_loc, oout[0], oout[1] if len(oout) > 1 else None)
            key = (w, "c") if (kind == "compress" and topo == dq.BUTTERFLY and n > 1) else (w, step)
            g_reg[key] = gout
            o_reg[key] = oout
            if check_every:
                torch.cuda.synchronize()
                for (m, c), gb, ob in zip(parts, gout, oout):
                    size = R.region_bytes(self.C, m, c)
                    gbytes = gb[:size].cpu().numpy()
                    if not np.array_equal(gbytes, ob[:size]):
                        bad = np.nonzero(gbytes != ob[:size])[0]
                        raise AssertionError(f"{kind} worker {w} step {step} part {c}/{m}: "
                                             f"{bad.size} of {size} bytes differ, first at {bad[0]}")
        self.g_reg, self.o_reg = g_reg, o_reg

    def finalize(self):
        n = self.n
        out_g = torch.full((self.d,), float("nan"), dtype=torch.float32, device=DEV)
        out_o = np.full(self.d, np.nan, np.float32)
        L = max(0, n.bit_length() - 1)
        for w in range(n):
            part = self.plan.final_part(w)
            assert part == self.orc.final_part(w)
            if n == 1:
                key = (0, 0)
            elif self.topo == dq.RING:
                key = (w, n - 1)
            else:
                key = (w, L)
            self.plan.finalize(part, self.g_reg[key][0], out_g)
            self.orc.finalize(part, self.o_reg[key][0], out_o)
        torch.cuda.synchronize()
        out_g = out_g.cpu().numpy()
        assert np.array_equal(_bits(out_g), _bits(out_o)), "finalize: output"
        return out_g


def full_round(grads, topo, **kw):
    r = Round(grads, topo, **kw)
    r.stages()
    info = r.check_stages()
    r.run_hops()
    out = r.finalize()
    return r, info, out


def _scaled(name, J, workers=None, seed=0):
    return synth.generate(name, d=256 * J, device=DEV, seed=seed, workers=workers)


# ---------------------------------------------------------------------------

def test_tiny_workload_bit_exact():
    """The tiny workload exactly as specified: 65,536 fp32 coordinates, 4
    workers, ring, 5 bits, data seed 0, rounding seed 1."""
    _need_gpu()
    grads = synth.generate("tiny", device=DEV)
    r, info, out = full_round(grads, dq.RING, budget=5.0, seed=1)
    assert info["achieved_bits"] <= 5.0
    # the native whole-round entry point gives the same bytes
    p = dq.Plan(65536, 4, dq.RING, 5.0, seed=1)
    out2 = p.allreduce(grads)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out2.cpu().numpy()), _bits(out))


@pytest.mark.parametrize("name,n,topo,own", [("bert", 8, dq.RING, dq.OWN_PACKED),
                                             ("llama", 3, dq.RING, dq.OWN_PACKED),
                                             ("gemma", 8, dq.BUTTERFLY, dq.OWN_PACKED),
                                             ("gemma", 16, dq.BUTTERFLY, dq.OWN_F32)])
def test_two_stream_round_bit_exact(name, n, topo, own):
    """DQ_OPT_STREAMS = 2 (odd workers' launches on a second stream, fork/join
    around every step) gives the oracle's bytes, on the caller's stream's
    timeline: the output is read after synchronising only that stream."""
    _need_gpu()
    J = 1537
    grads = _scaled(name, J, workers=range(n))
    p = dq.Plan(256 * J, n, topo, 5.0, own=own, streams=2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = p.allreduce(grads, stream=s)
    s.synchronize()
    o = po.Oracle(256 * J, n, po.BUTTERFLY if topo == dq.BUTTERFLY else po.RING, 5.0,
                  own=po.OWN_F32 if own == dq.OWN_F32 else po.OWN_PACKED)
    ref = o.allreduce(_grads_np(grads))
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref))


@pytest.mark.parametrize("name,J,topo", [
    ("bert", 3001, dq.RING),          # 8 workers, ragged parts
    ("gemma", 4099, dq.BUTTERFLY),    # 8 workers, 3 levels, two-child outputs
    ("large", 2053, dq.RING),         # zero super-groups
])
def test_scaled_workloads_bit_exact(name, J, topo):
    _need_gpu()
    full_round(_scaled(name, J), topo)


@pytest.mark.parametrize("budget", [3.0, 4.0, 5.0, 6.0])
def test_llama_shape_budget_sweep(budget):
    _need_gpu()
    grads = _scaled("llama", 1537)
    r, info, out = full_round(grads, dq.RING, budget=budget)
    assert info["used_bits"] <= budget * r.plan.J


def _with_offsets(grads, seed=5):
    """Add a per-SG offset, the same on every worker, to a third of the SGs, of
    the size of the SG's spread: the mean-corrected key then differs from F."""
    J = grads[0].numel() // 256
    gen = torch.Generator(device="cpu").manual_seed(seed)
    spread = torch.stack([g.float().view(J, 256).abs().amax(1) for g in grads]).amax(0).cpu()
    pick = (torch.rand(J, generator=gen) < 1 / 3).float()
    off = (pick * spread * (2 * torch.rand(J, generator=gen) - 1) * 4).to(DEV)
    return [(g.float().view(J, 256) + off[:, None]).view(-1).to(g.dtype) for g in grads]


@pytest.mark.parametrize("alloc,budget,topo", [
    (dq.ALLOC_MEAN_CORRECTED, 5.0, dq.RING), (dq.ALLOC_MEAN_CORRECTED, 3.0, dq.BUTTERFLY),
    (dq.ALLOC_UNIFORM, 5.0, dq.RING), (dq.ALLOC_UNIFORM, 2.0, dq.BUTTERFLY),
    (dq.ALLOC_UNIFORM, 8.0, dq.RING)])
def test_allocation_variants_bit_exact(alloc, budget, topo):
    """The variants of the allocation (mean-corrected key, uniform widths)
    through every stage of a round, against the oracle."""
    _need_gpu()
    grads = _with_offsets(_scaled("llama" if topo == dq.RING else "gemma", 1031, workers=range(8)))
    r, info, out = full_round(grads, topo, budget=budget, alloc=alloc)
    if alloc == dq.ALLOC_UNIFORM:
        q = 8 if budget >= 8 else (4 if budget >= 4 else 2)
        assert info["class_counts"][{2: 0, 4: 1, 8: 2}[q]] == r.plan.J
        assert info["rho_bits"] == 0x7FC00000
    else:
        plain = Round(grads, topo, budget=budget)
        plain.stages()
        assert not np.array_equal(plain.plan.widths().cpu().numpy(), r.plan.widths().cpu().numpy())


@pytest.mark.parametrize("eps,topo", [(1.0, dq.RING), (0.25, dq.BUTTERFLY), (0.05, dq.RING),
                                      (0.8, dq.BUTTERFLY), (0.03, dq.RING), (0.0274, dq.BUTTERFLY)])
def test_level_shapes_bit_exact(eps, topo):
    """Other level shapes phi(t) = t (eps + (1 - eps) t): eps = 1 is the
    uniform grid; smaller eps packs the levels towards zero, down to the
    smallest shape whose central 8-bit levels still fall in distinct
    buckets of the interval search (eps = 0.0274)."""
    _need_gpu()
    grads = _scaled("llama" if topo == dq.RING else "gemma", 1031, workers=range(8))
    full_round(grads, topo, budget=5.0, eps=eps)


@pytest.mark.parametrize("eps", [0.5, 1.0, 0.1, 0.0274])
def test_device_tables_match_the_definition(eps):
    """The tables the plan builds in its workspace: levels and (L, W) pairs
    equal the oracle's; compare levels end in +inf; every bucket entry is
    the number of interior levels in the buckets below it."""
    _need_gpu()
    d = 256 * 64
    grads = [torch.zeros(d, dtype=torch.bfloat16, device=DEV)]
    p = dq.Plan(d, 1, dq.RING, 5.0, eps=eps)
    p.stats(0, grads[0])                     # the first stage builds the tables
    torch.cuda.synchronize()
    off = p.layout["tables"]
    raw = p.workspace[off:off + 4364 + 8192 + 1024].cpu().numpy()
    f = lambda o, n: raw[o:o + 4 * n].view(np.float32)
    L2, L4, L8, W2 = f(0, 4), f(16, 16), f(80, 256), f(1104, 3)
    CL4, CL8 = f(1116, 16), f(1180, 256)
    LW4, LW8 = f(2204, 30).reshape(15, 2), f(2324, 510).reshape(255, 2)
    for q, L, CL, LW in ((2, L2, None, None), (4, L4, CL4, LW4), (8, L8, CL8, LW8)):
        Lo, Wo = po.levels(q, eps)
        assert np.array_equal(_bits(L), _bits(Lo))
        if q == 2:
            assert np.array_equal(_bits(W2), _bits(Wo[:3]))
            continue
        assert np.array_equal(_bits(CL[:-1]), _bits(Lo[:-1])) and np.isposinf(CL[-1])
        assert np.array_equal(_bits(LW[:, 0]), _bits(Lo[:-1]))
        assert np.array_equal(_bits(LW[:, 1]), _bits(Wo[:len(Lo) - 1]))
    # bucket entries: est[k] = interior levels whose linear bucket
    # NB/2 + rne(L M) (M = NB/2 - 1) lies below k
    for q, o, NB in ((8, 4364, 8192), (4, 4364 + 8192, 1024)):
        est = raw[o:o + NB]
        Lo = po.levels(q, eps)[0]
        bl = NB // 2 + np.rint(Lo[1:-1].astype(np.float64) * (NB // 2 - 1)).astype(np.int64)
        want = np.searchsorted(bl, np.arange(NB), side="left")
        assert np.array_equal(est.astype(np.int64), want)


@pytest.mark.parametrize("n,topo", [(1, dq.RING), (1, dq.BUTTERFLY), (2, dq.RING), (2, dq.BUTTERFLY),
                                    (4, dq.BUTTERFLY), (16, dq.BUTTERFLY), (32, dq.BUTTERFLY),
                                    (64, dq.BUTTERFLY), (3, dq.RING), (5, dq.RING), (13, dq.RING)])
def test_worker_counts(n, topo):
    _need_gpu()
    grads = _scaled("bert", 733, workers=range(n))
    full_round(grads, topo)


@pytest.mark.parametrize("mode", [dq.INDEPENDENT, dq.CORRELATED], ids=["independent", "rank-correlated"])
@pytest.mark.parametrize("topo", [dq.RING, dq.BUTTERFLY])
def test_rounding_modes_bit_exact(topo, mode):
    """The non-default rounding modes (the default, level-stratified, runs in
    every other test)."""
    _need_gpu()
    full_round(_scaled("gemma", 1031), topo, rounding=mode, seed=2 ** 40 + 17, rnd=9)


@pytest.mark.parametrize("J,n,topo", [(1, 8, dq.RING), (3, 8, dq.BUTTERFLY), (7, 4, dq.RING),
                                      (17, 16, dq.RING)])
def test_tiny_and_empty_parts(J, n, topo):
    """Fewer super-groups than parts: some parts are empty."""
    _need_gpu()
    full_round(_scaled("bert", J, workers=range(n)), topo)


@pytest.mark.parametrize("budget", [2.0, 8.0, 100.0, 2.0001, 7.999, float("inf")])
def test_budget_extremes(budget):
    _need_gpu()
    r, info, out = full_round(_scaled("llama", 517, workers=range(4)), dq.RING, budget=budget)
    if budget >= 8:
        assert info["class_counts"] == [0, 0, 517] and info["rho_bits"] == 0
        assert info["budget_bits"] == 8 * 517
    if budget == 2.0:
        assert info["class_counts"] == [517, 0, 0]


def test_zero_and_constant_super_groups_f32():
    _need_gpu()
    n, J = 4, 40
    g = [torch.randn(256 * J, device=DEV) * 1e-3 for _ in range(n)]
    for t in g:
        t[:256] = 0.0
        t[256 * 5:256 * 6] = 0.375
        t[256 * 9:256 * 10] = -2.0 ** -130   # subnormal constant
    r, info, out = full_round(g, dq.RING)
    assert np.all(out[:256] == 0.0)
    assert np.all(out[256 * 5:256 * 6] == np.float32(1.5))


def _subnormal_scale_grads(n, J, seed):
    """fp32 gradients whose super-groups 3, 7, 11, ... hold values of a few
    2^-145 (pairs +a, -a, so every worker's sum and the mean are exactly 0)
    and exact zeros: their scale units are subnormal and 1/sigma overflows,
    so y * inv would be +-inf, or NaN where y = 0.  The other super-groups
    are ordinary."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        g = (rng.standard_normal(256 * J) * 1e-3).astype(np.float32)
        for j in range(3, J, 4):
            k = rng.integers(1, 2000, 128).astype(np.float32)
            vals = np.empty(256, np.float32)
            vals[0::2] = k * np.float32(2.0 ** -145)
            vals[1::2] = -vals[0::2]
            vals[rng.random(256) < 0.3] = 0.0
            vals[1::2] = -vals[0::2]                    # keep the pairs after zeroing
            g[256 * j:256 * (j + 1)] = vals
        out.append(torch.from_numpy(g).to(DEV))
    return out


@pytest.mark.parametrize("budget,alloc,max_width,topo", [
    (2.0, dq.ALLOC_THRESHOLD, 8, dq.RING), (8.0, dq.ALLOC_THRESHOLD, 8, dq.BUTTERFLY),
    (4.0, dq.ALLOC_UNIFORM, 8, dq.RING), (5.0, dq.ALLOC_THRESHOLD, 8, dq.BUTTERFLY),
    (16.0, dq.ALLOC_THRESHOLD, 16, dq.RING)])
def test_subnormal_scale_super_groups_bit_exact(budget, alloc, max_width, topo):
    """Groups whose 1/sigma overflows (sigma < 2^-128) follow the definition
    exactly: v = 0 where y = 0 and clamp(y * inf) = +-1 elsewhere, in every
    width class, through compress and every hop."""
    _need_gpu()
    n, J = 4, 64
    grads = _subnormal_scale_grads(n, J, seed=int(budget * 10) + max_width)
    r, info, out = full_round(grads, topo, budget=budget, alloc=alloc, max_width=max_width)
    counts = info["class_counts"]
    assert sum(counts) == J


def test_all_zero_gradients():
    _need_gpu()
    g = [torch.zeros(256 * 33, dtype=torch.bfloat16, device=DEV) for _ in range(8)]
    r, info, out = full_round(g, dq.BUTTERFLY)
    assert np.all(out == 0.0)


def test_nonfinite_flag():
    _need_gpu()
    g = [torch.randn(256 * 8, device=DEV) for _ in range(2)]
    g[1][300] = float("inf")
    p = dq.Plan(256 * 8, 2, dq.RING, 5.0)
    p.stats(0, g[0])
    p.stats(1, g[1])
    p.allocate()
    info = p.info()
    assert info["nonfinite"] and info["status"] == dq.DQ_ENONFINITE
    # a new round with finite data clears it
    g[1][300] = 0.0
    p.stats(0, g[0])
    p.stats(1, g[1])
    p.allocate()
    assert not p.info()["nonfinite"]


@pytest.mark.parametrize("topo,max_width", [(dq.RING, 8), (dq.BUTTERFLY, 8), (dq.BUTTERFLY, 16)],
                         ids=["ring", "butterfly", "butterfly-16bit"])
def test_nonfinite_gradients_stay_in_their_super_groups(topo, max_width):
    """Gradients must be finite, and a round over non-finite ones is flagged
    (DQ_ENONFINITE).  It still runs to the end with every table read in
    bounds, and a non-finite value spoils only its own super-group: every
    super-group that is finite on every worker comes out bit-exact against
    the oracle.  Planted: +inf, -inf, a NaN, a whole group of NaN, and +inf
    on one worker against -inf on another in the same coordinate (a NaN
    sum); with the 16-bit class allowed, the infinite squared norm puts its
    super-group in that class."""
    _need_gpu()
    J, n = 96, 4
    grads = _scaled("gemma", J, workers=range(n))
    plants = [(0, 3 * 256 + 5, float("inf")), (1, 10 * 256 + 17, float("nan")),
              (3, 40 * 256, float("inf")), (1, 40 * 256, float("-inf")),
              (0, 77 * 256 + 255, float("-inf"))]
    plants += [(2, 20 * 256 + 32 + i, float("nan")) for i in range(16)]
    for w, i, x in plants:
        grads[w][i] = x
    bad = sorted({i // 256 for _, i, _ in plants})
    plan = dq.Plan(256 * J, n, topo, 5.0, seed=1, max_width=max_width)
    out = plan.allreduce(grads)
    torch.cuda.synchronize()
    info = plan.info()
    assert info["nonfinite"] and info["status"] == dq.DQ_ENONFINITE
    if max_width == 16:
        assert info["class_counts"][3] >= 1
    ref = po.Oracle(256 * J, n, topo, 5.0, seed=1, max_width=max_width).allreduce(_grads_np(grads))
    ok = np.ones(J, bool)
    ok[bad] = False
    keep = np.repeat(ok, 256)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got[keep]))
    assert np.array_equal(_bits(got[keep]), _bits(ref[keep]))


@pytest.mark.parametrize("max_width", [8, 16])
@pytest.mark.parametrize("budget,n_over", [(5.0, 3), (3.0, 12)], ids=["within-budget", "budget-out-of-reach"])
def test_overflowed_squared_norms_like_the_oracle(max_width, budget, n_over):
    """Finite gradients whose squared norms overflow (one entry of 1e20 per
    super-group): the round is flagged, and rho, every width and the class
    counts equal the oracle's.  Keys of +inf take the widest width of the
    plan's set and nothing outside it; when even rho = +inf misses the
    budget, rho is +inf.  The whole round then runs in bounds and the
    super-groups that did not overflow come out bit-exact."""
    _need_gpu()
    J, n = 16, 2
    gen = torch.Generator().manual_seed(41)
    gs = [torch.randn(256 * J, generator=gen).to(DEV) for _ in range(n)]
    gs[1][0:n_over * 256:256] = 1e20
    gnp = [g.cpu().numpy() for g in gs]
    plan = dq.Plan(256 * J, n, dq.RING, budget, max_width=max_width)
    orc = po.Oracle(256 * J, n, po.RING, budget, max_width=max_width)
    for w in range(n):
        plan.stats(w, gs[w])
        orc.stats(w, gnp[w])
    plan.allocate()
    orc.allocate()
    info = plan.info()
    assert info["nonfinite"] and info["status"] == dq.DQ_ENONFINITE
    assert info["rho_bits"] == orc.rho_bits()
    if n_over == 12:
        assert orc.rho_bits() == 0x7F800000
    assert np.array_equal(plan.widths().cpu().numpy(), orc.widths())
    assert list(info["class_counts"]) == orc.class_counts().tolist()
    assert sum(info["class_counts"]) == J
    out = dq.Plan(256 * J, n, dq.RING, budget, max_width=max_width).allreduce(gs)
    torch.cuda.synchronize()
    ref = po.Oracle(256 * J, n, po.RING, budget, max_width=max_width).allreduce(gnp)
    keep = np.repeat(np.arange(J) >= n_over, 256)
    assert np.array_equal(_bits(out.cpu().numpy()[keep]), _bits(ref[keep]))


def test_deterministic_and_native_schedule_matches():
    _need_gpu()
    grads = _scaled("gemma", 2050)
    outs = []
    for _ in range(2):
        p = dq.Plan(grads[0].numel(), 8, dq.BUTTERFLY, 5.0, seed=5)
        outs.append(p.allreduce(grads).cpu().numpy())
    assert np.array_equal(_bits(outs[0]), _bits(outs[1]))
    o = po.Oracle(grads[0].numel(), 8, po.BUTTERFLY, 5.0, seed=5)
    ref = o.allreduce(_grads_np(grads))
    assert np.array_equal(_bits(outs[0]), _bits(ref))


def test_timing_counts_coordinates():
    _need_gpu()
    grads = _scaled("bert", 999)
    p = dq.Plan(grads[0].numel(), 8, dq.RING, 5.0, timing=True)
    p.allreduce(grads)
    t = p.timing()
    J = p.J
    assert t["hop_grad"]["launches"] == 8 * 6
    assert t["hop_grad"]["coords"] == 6 * J * 256       # each ring step covers every SG once
    assert t["compress"]["coords"] == J * 256
    # the last ring step's hops also decode the final sum: no finalize launch
    assert t["hop_final"]["launches"] == 8
    assert t["hop_final"]["coords"] == J * 256
    assert t["finalize"]["launches"] == 0
    assert t["stats"]["coords"] == 8 * J * 256
    assert all(v["ms"] >= 0 for v in t.values())


@pytest.mark.parametrize("own,per_level", [(dq.OWN_PACKED, 8), (dq.OWN_F32, 16)], ids=["packed-own", "fp32-own"])
def test_timing_counts_butterfly_launches(own, per_level):
    """A hop that writes both children of its part is one launch, timed as
    the parent part; the fp32 own-partial variant writes its kept child in
    another mode and keeps a launch per child.  Per round of 8 workers:
    level 1 covers 4 J super-groups, level 2 covers 2 J, level 3 covers J."""
    _need_gpu()
    grads = _scaled("gemma", 999)
    p = dq.Plan(grads[0].numel(), 8, dq.BUTTERFLY, 5.0, own=own, timing=True)
    p.allreduce(grads)
    t = p.timing()
    J = p.J
    assert t["compress"]["launches"] == 8 and t["compress"]["coords"] == 4 * J * 256
    assert t["hop_grad"]["launches"] == per_level and t["hop_grad"]["coords"] == 4 * J * 256
    assert t["hop_packed"]["launches"] == per_level and t["hop_packed"]["coords"] == 2 * J * 256
    assert t["hop_final"]["launches"] == 8 and t["hop_final"]["coords"] == J * 256


# ---------------------------------------------------------------------------
# butterfly variant: the kept child stays fp32 (DQ_OWN_F32)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,rounding", [(2, dq.STRATIFIED), (4, dq.INDEPENDENT), (8, dq.STRATIFIED),
                                        (16, dq.CORRELATED)])
def test_own_fp32_round_bit_exact(n, rounding):
    _need_gpu()
    J = 777
    grads = _scaled("gemma", J, workers=range(n))
    p = dq.Plan(256 * J, n, dq.BUTTERFLY, 5.0, rounding=rounding, own=dq.OWN_F32)
    out = p.allreduce(grads)
    torch.cuda.synchronize()
    o = po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rounding=rounding, own=po.OWN_F32)
    ref = o.allreduce(_grads_np(grads))
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref))


def test_own_fp32_every_step_bit_exact():
    """n = 8, step by step: every sent region and every kept fp32 partial of
    every hop, GPU against oracle."""
    _need_gpu()
    n, J = 8, 1031
    L = 3
    grads = _scaled("gemma", J, workers=range(n))
    gnp = _grads_np(grads)
    plan = dq.Plan(256 * J, n, dq.BUTTERFLY, 5.0, own=dq.OWN_F32)
    orc = po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, own=po.OWN_F32)
    for w in range(n):
        plan.stats(w, grads[w])
        orc.stats(w, gnp[w])
    plan.allocate(); orc.allocate()
    plan.reorder(); orc.reorder()
    torch.cuda.synchronize()
    C = orc.class_counts()
    RB = orc.worst_region_bytes()
    g_out, o_out = {}, {}
    for w in range(n):
        gr = plan.new_region(2)
        orr = np.zeros(RB, np.uint8)
        plan.compress(w, 1, grads[w], gr)
        orc.compress(w, 1, gnp[w], orr)
        g_out[(w, 0)], o_out[(w, 0)] = [gr], [orr]
    for s in range(1, L + 1):
        for w in range(n):
            partner = w ^ (n >> s)
            keep_prev = (w >> (L - s)) & 1
            if s == 1:
                g_in, o_in, g_loc, o_loc = g_out[(partner, 0)][0], o_out[(partner, 0)][0], grads[w], gnp[w]
            else:
                g_in, o_in = g_out[(partner, s - 1)][keep_prev], o_out[(partner, s - 1)][keep_prev]
                g_loc, o_loc = g_out[(w, s - 1)][keep_prev], o_out[(w, s - 1)][keep_prev]
            c = w >> (L - s)
            if s < L:
                keep = (w >> (L - s - 1)) & 1
                m = 2 ** (s + 1)
                gs_, os_ = [], []
                for h in range(2):
                    if h == keep:
                        gs_.append(torch.full((plan.partial_bytes_max(m) // 4,), float("nan"),
                                              dtype=torch.float32, device=DEV))
                        os_.append(np.full(plan.partial_bytes_max(m) // 4, np.nan, np.float32))
                    else:
                        gs_.append(plan.new_region(m))
                        os_.append(np.zeros(RB, np.uint8))
            else:
                gs_, os_ = [plan.new_region(n)], [np.zeros(RB, np.uint8)]
            kind = None if s == 1 else dq.F32_PARTIAL
            plan.hop(w, s, g_in, g_loc, gs_[0], gs_[1] if len(gs_) > 1 else None, local_kind=kind)
            orc.hop(w, s, o_in, o_loc, os_[0], os_[1] if len(os_) > 1 else None, partial=(s > 1))
            torch.cuda.synchronize()
            for h, (gb, ob) in enumerate(zip(gs_, os_)):
                m_out, c_out = (2 ** (s + 1), 2 * c + h) if s < L else (n, c)
                if s < L and h == keep:
                    N = sum(cnt for _, cnt in R.part_ranges(C, m_out, c_out))
                    a = gb.cpu().numpy()[:256 * N]
                    assert np.array_equal(_bits(a), _bits(ob[:256 * N])), f"partial w{w} s{s}"
                else:
                    size = R.region_bytes(C, m_out, c_out)
                    assert np.array_equal(gb[:size].cpu().numpy(), ob[:size]), f"region w{w} s{s} h{h}"
            g_out[(w, s)], o_out[(w, s)] = gs_, os_
    out_g = torch.empty(256 * J, dtype=torch.float32, device=DEV)
    out_o = np.zeros(256 * J, np.float32)
    for w in range(n):
        plan.finalize(plan.final_part(w), g_out[(w, L)][0], out_g)
        orc.finalize(orc.final_part(w), o_out[(w, L)][0], out_o)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out_g.cpu().numpy()), _bits(out_o))


@pytest.mark.parametrize("n,topo", [(4, dq.RING), (8, dq.BUTTERFLY), (3, dq.RING)])
def test_fused_final_hop_matches_hop_then_finalize(n, topo):
    """dq_hop_finalize at the schedule's last step writes the region dq_hop
    writes and the output dq_finalize computes from it; at other steps it is
    refused."""
    _need_gpu()
    J = 515
    grads = _scaled("gemma" if topo == dq.BUTTERFLY else "llama", J, workers=range(n))
    r = Round(grads, topo)
    r.stages()
    r.check_stages()
    r.run_hops(check_every=False)
    out_ref = r.finalize()
    L = n.bit_length() - 1
    last = n - 1 if topo == dq.RING else L
    out = torch.full((256 * J,), float("nan"), dtype=torch.float32, device=DEV)
    for w in range(n):
        if topo == dq.RING:
            g_in, loc = r.g_reg[((w - 1) % n, last - 1)][0], grads[w]
        else:
            partner = w ^ (n >> last)
            keep = (w >> (L - last)) & 1
            g_in, loc = r.g_reg[(partner, last - 1)][keep], r.g_reg[(w, last - 1)][keep]
        reg = r.plan.new_region(n)
        r.plan.hop_finalize(w, last, g_in, loc, reg, out)
        torch.cuda.synchronize()
        part = r.plan.final_part(w)
        size = R.region_bytes(r.C, n, part)
        assert np.array_equal(reg[:size].cpu().numpy(), r.g_reg[(w, last)][0][:size].cpu().numpy())
        if topo == dq.RING and last > 1:
            with pytest.raises(dq.DQError):
                r.plan.hop_finalize(w, last - 1, g_in, loc, reg, out)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(out_ref))


# ---------------------------------------------------------------------------
# the 16-bit class (DQ_OPT_MAX_WIDTH = 16): widths, streams, regions and
# output bit-exact with the oracle's 16-bit class
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,n,topo,budget", [("gemma", 8, dq.BUTTERFLY, 6.0), ("bert", 4, dq.RING, 9.0),
                                                ("llama", 5, dq.RING, 12.0), ("tiny", 4, dq.RING, 5.0),
                                                ("large", 4, dq.BUTTERFLY, 16.0)])
def test_sixteen_bit_class_bit_exact(name, n, topo, budget):
    _need_gpu()
    J = 1200 if name != "tiny" else 256
    grads = _scaled(name, J, workers=range(n))
    r, info, out = full_round(grads, topo, budget=budget, max_width=16)
    assert len(info["class_counts"]) == 4
    assert info["used_bits"] <= info["budget_bits"]
    if budget >= 9.0:
        assert info["class_counts"][3] > 0         # some super-groups at 16 bits
    if budget == 16.0:
        assert info["class_counts"][3] == J


def test_sixteen_bit_class_level_tables_and_eps():
    """The workspace's 65,536 levels and weights equal the oracle's table,
    for the default shape and another one; so do the (level, weight) pairs
    the search reads."""
    _need_gpu()
    for eps in (None, 0.2):
        p = dq.Plan(256 * 64, 2, dq.RING, 10.0, max_width=16, eps=eps)
        g = [torch.ones(256 * 64, dtype=torch.float32, device=DEV) for _ in range(2)]
        p.stats(0, g[0])
        p.stats(1, g[1])
        torch.cuda.synchronize()
        off = p.layout["tables16"]
        T = p.workspace[off:off + 4 * 65536 * 4].view(torch.float32).cpu().numpy()
        L, W = po.levels(16, 0.5 if eps is None else eps)
        assert np.array_equal(_bits(T[:65536]), _bits(L))
        assert np.array_equal(_bits(T[65536:65536 + 65535]), _bits(W))
        pairs = T[2 * 65536:].reshape(65536, 2)
        assert np.array_equal(_bits(pairs[:, 0]), _bits(L))
        assert np.array_equal(_bits(pairs[:65535, 1]), _bits(W))
