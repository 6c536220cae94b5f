"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses (the same library calls on the same buffer sizes).

The oracle computes every statistic, the allocation and the reorder itself from
a host copy of the inputs, and these are compared over every super-group.

Whole rounds (BERT-, Gemma- and LLaMA-shaped workloads): the oracle then runs
every compress and hop of the schedule over every super-group, and after each
step every byte of every region the GPU wrote is compared with the oracle's,
and at the end every coordinate of the fp32 output.

Sampled rounds (the Large share, whose eight 8.6 GB gradients and 3e10
coordinates of oracle work per round are too heavy for a test, and the
largest-region case): the oracle follows a sample of super-groups (class and
part boundaries plus random ones) through the schedule and their region bytes
and decoded output are compared.  Inputs come from the shared seeded
generator (drawn on the GPU).
"""
import numpy as np
import pytest
import torch

from compressed_hop_gradient_amd import dq, synth
from oracle import pyoracle as po
from tests import regions as R

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _host(t):
    return synth.as_numpy(t)


def _sample_positions(C, n, topo, rng, extra=96):
    """Stream positions at class and part boundaries, plus random ones."""
    J = int(sum(C))
    pos = set()
    ms = [n] if topo == dq.RING else [2 ** s for s in range(1, n.bit_length())]
    for m in ms:
        for c in range(m):
            for lo, cnt in R.part_ranges(C, m, c):
                if cnt:
                    pos.update((lo, lo + cnt - 1))
    pos.update(int(x) for x in rng.integers(0, J, extra))
    return np.array(sorted(pos), dtype=np.int64)


def _gather(region_gpu, C, m, c, positions):
    """GPU region bytes (codes, scale, group codes) of the sampled positions in part c of m."""
    rng_ = R.part_ranges(C, m, c)
    lay = R.layout([cnt for _, cnt in rng_])
    idx = []
    keep = []
    for p in positions:
        for k, (lo, cnt) in enumerate(rng_):
            if lo <= p < lo + cnt:
                i = p - lo
                local = sum(x for _, x in rng_[:k]) + i
                q = R.QS[k]
                a = lay["codes"][k] + i * 32 * q
                idx.append(np.concatenate([np.arange(a, a + 32 * q), lay["s"] + 4 * local + np.arange(4),
                                           lay["c"] + 16 * local + np.arange(16)]))
                keep.append(p)
    if not keep:
        return [], []
    flat = torch.from_numpy(np.concatenate(idx)).to(region_gpu.device)
    got = region_gpu[flat].cpu().numpy()
    out, o = [], 0
    for ii in idx:
        out.append(got[o:o + ii.size])
        o += ii.size
    return keep, out


def _oracle_bytes(region_np, C, m, c, p):
    codes, s, cg = R.sg_raw(region_np, C, m, c, p)
    return np.frombuffer(codes + s + cg, np.uint8)


def _steps(n, topo):
    if topo == dq.RING:
        yield ("compress", None, 0)
        for t in range(1, n):
            yield ("hop", None, t)
    else:
        L = n.bit_length() - 1
        yield ("compress", None, 1)
        for s in range(1, L + 1):
            yield ("hop", None, s)


def _region_diff(got, exp, C, m, c):
    """Where two region byte arrays first differ: (section, super-group)."""
    bad = int(np.flatnonzero(got != exp)[0])
    lay = R.layout([cnt for _, cnt in R.part_ranges(C, m, c)])
    for k in range(3):
        a = lay["codes"][k]
        n_k = R.part_ranges(C, m, c)[k][1]
        if a <= bad < a + n_k * 32 * R.QS[k]:
            return f"codes of class {R.QS[k]}, super-group {(bad - a) // (32 * R.QS[k])} of the class"
    if lay["s"] <= bad < lay["c"]:
        return f"scale unit of part-local super-group {(bad - lay['s']) // 4}"
    return f"group codes of part-local super-group {(bad - lay['c']) // 16}"


def _run(name, budget, capsys, budgets_stage_only=(), d=None, n=None, whole=False):
    """The workload's recipe and schedule; d and n override its size.  whole:
    the oracle runs every super-group and every region byte and output
    coordinate is compared; otherwise a sample of super-groups."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = synth.WORKLOADS[name]
    topo = dq.BUTTERFLY if wl.topology == "butterfly" else dq.RING
    n = wl.n if n is None else n
    d = wl.d if d is None else d
    label = name if (n, d) == (wl.n, wl.d) else f"{name} recipe, {d} coords x {n}"

    def say(msg):
        with capsys.disabled():
            print(f"[fullsize {label}] {msg}", flush=True)

    say("generating")
    grads = synth.generate(name, device=DEV, d=d, workers=range(n))
    torch.cuda.synchronize()
    say("host copy")
    gnp = [_host(g) for g in grads]

    plan = dq.Plan(d, n, topo, budget, seed=wl.rounding_seed)
    orc = po.Oracle(d, n, topo, budget, seed=wl.rounding_seed)
    say("stats / allocate / reorder")
    for w in range(n):
        plan.stats(w, grads[w])
        orc.stats(w, gnp[w])
    plan.allocate()
    plan.reorder()
    orc.allocate()
    orc.reorder()
    torch.cuda.synchronize()
    s_g, F_g = [x.cpu().numpy() for x in plan.stats_arrays()]
    s_o, F_o, mu_o = orc.stats_arrays()
    assert np.array_equal(_bits(s_g), _bits(s_o)), "stats: sum"
    assert np.array_equal(_bits(F_g), _bits(F_o)), "stats: squared norm"
    info = plan.info()
    assert not info["nonfinite"]
    assert info["rho_bits"] == orc.rho_bits(), "allocate: rho"
    assert np.array_equal(plan.widths().cpu().numpy(), orc.widths()), "allocate: widths"
    C = orc.class_counts()
    assert info["class_counts"] == C.tolist()
    perm_o, inv_o = orc.perm()
    perm_g, inv_g = [x.cpu().numpy() for x in plan.perm()]
    assert np.array_equal(perm_g, perm_o) and np.array_equal(inv_g, inv_o), "reorder"
    assert np.array_equal(_bits(plan.mu_stream().cpu().numpy()), _bits(mu_o[perm_o])), "reorder: mean"

    J = d // 256
    if whole:
        positions = None
        say(f"all {J} super-groups through the schedule")
    else:
        positions = _sample_positions(C, n, topo, np.random.default_rng(7))
        say(f"{positions.size} sampled super-groups through the schedule")
    region_bytes_checked = 0
    L = max(0, n.bit_length() - 1)
    last = n - 1 if topo == dq.RING else L
    # the schedule's last hops run fused with the finalize of their part, as a
    # whole round does (dq_hop_finalize): they write the region and the output
    out_g = torch.full((d,), float("nan"), dtype=torch.float32, device=DEV)
    g_prev, o_prev = {}, {}
    checked = 0
    for kind, _, step in _steps(n, topo):
        g_cur, o_cur = {}, {}
        for w in range(n):
            if topo == dq.RING:
                parts = [(n, w if kind == "compress" else (w - step) % n)]
            elif kind == "compress":
                parts = [(2, (w >> (L - 1)) ^ 1)]
            else:
                c = w >> (L - step)
                parts = [(2 ** (step + 1), 2 * c), (2 ** (step + 1), 2 * c + 1)] if step < L else [(n, c)]
            gout = [plan.new_region(m) for m, _ in parts]
            oout = [np.zeros(R.region_bytes(C, m, c) + 64, np.uint8) for m, c in parts]
            if kind == "compress":
                plan.compress(w, step, grads[w], gout[0])
                orc.compress(w, step, gnp[w], oout[0], filt=positions)
            elif topo == dq.RING:
                src = (w - 1) % n
                if step == last:
                    plan.hop_finalize(w, step, g_prev[src][0], grads[w], gout[0], out_g)
                else:
                    plan.hop(w, step, g_prev[src][0], grads[w], gout[0])
                orc.hop(w, step, o_prev[src][0], gnp[w], oout[0], filt=positions)
            else:
                partner, keep = w ^ (n >> step), (w >> (L - step)) & 1
                if step == 1:
                    gi, oi = g_prev[partner][0], o_prev[partner][0]
                    gl, ol = grads[w], gnp[w]
                else:
                    gi, oi = g_prev[partner][keep], o_prev[partner][keep]
                    gl, ol = g_prev[w][keep], o_prev[w][keep]
                if step == last:
                    plan.hop_finalize(w, step, gi, gl, gout[0], out_g)
                else:
                    plan.hop(w, step, gi, gl, gout[0], gout[1] if len(gout) > 1 else None)
                orc.hop(w, step, oi, ol, oout[0], oout[1] if len(oout) > 1 else None, filt=positions)
            torch.cuda.synchronize()
            for (m, c), gb, ob in zip(parts, gout, oout):
                if whole:
                    nb = R.region_bytes(C, m, c)
                    gbb = gb[:nb].cpu().numpy()
                    if not np.array_equal(gbb, ob[:nb]):
                        where = _region_diff(gbb, ob[:nb], C, m, c)
                        raise AssertionError(f"{kind} worker {w} step {step}, part {c} of {m}: {where} differs")
                    region_bytes_checked += nb
                    checked += sum(cnt for _, cnt in R.part_ranges(C, m, c))
                    continue
                keep_pos, gbytes = _gather(gb, C, m, c, positions)
                for p, gbb in zip(keep_pos, gbytes):
                    obb = _oracle_bytes(ob, C, m, c, p)
                    assert np.array_equal(gbb, obb), f"{kind} worker {w} step {step}: position {p} differs"
                    checked += 1
            g_cur[w], o_cur[w] = gout, oout
        g_prev, o_prev = g_cur, o_cur
        say(f"{kind} step {step} ok")
    out_o = np.zeros(d, np.float32)
    for w in range(n):
        orc.finalize(plan.final_part(w), o_prev[w][0], out_o, filt=positions)
    torch.cuda.synchronize()
    assert not torch.isnan(out_g).any(), "the fused last hops left a coordinate unwritten"
    if whole:
        got = out_g.cpu().numpy()
        if not np.array_equal(_bits(got), _bits(out_o)):
            bad = np.flatnonzero(_bits(got) != _bits(out_o))
            raise AssertionError(f"fused finalize: {bad.size} output coordinates differ, first {bad[0]} "
                                 f"(super-group {bad[0] // 256})")
    else:
        cols = (perm_o[positions].astype(np.int64)[:, None] * 256 + np.arange(256)[None, :]).ravel()
        got = out_g[torch.from_numpy(cols).to(DEV)].cpu().numpy()
        assert np.array_equal(_bits(got), _bits(out_o[cols])), "fused finalize: output"
    # the stand-alone finalize of the same final regions gives the same bytes everywhere
    out_f = torch.full((d,), float("nan"), dtype=torch.float32, device=DEV)
    for w in range(n):
        plan.finalize(plan.final_part(w), g_prev[w][0], out_f)
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.int32), out_g.view(torch.int32)), "finalize vs fused last hop"
    if whole:
        say(f"all {region_bytes_checked} region bytes ({checked} super-group records) of every step and "
            f"all {J} output super-groups ({d} coordinates) bit-exact")
    else:
        say(f"{checked} sampled region records and {positions.size} output super-groups bit-exact")

    for b in budgets_stage_only:
        p2 = dq.Plan(d, n, topo, b, seed=wl.rounding_seed)
        o2 = po.Oracle(d, n, topo, b, seed=wl.rounding_seed)
        for w in range(n):
            p2.stats(w, grads[w])
            o2.stats(w, gnp[w])
        p2.allocate()
        p2.reorder()
        o2.allocate()
        o2.reorder()
        i2 = p2.info()
        assert i2["rho_bits"] == o2.rho_bits() and i2["used_bits"] <= i2["budget_bits"]
        assert np.array_equal(p2.widths().cpu().numpy(), o2.widths())
        assert np.array_equal(p2.perm()[0].cpu().numpy(), o2.perm()[0])
        say(f"budget {b}: allocation and reorder bit-exact ({i2['achieved_bits']:.4f} bits)")


@pytest.mark.timeout(600)
def test_bert_full(capsys):
    _run("bert", 5.0, capsys, whole=True)


@pytest.mark.timeout(900)
def test_gemma_full(capsys):
    _run("gemma", 5.0, capsys, whole=True)


@pytest.mark.timeout(1200)
def test_llama_full(capsys):
    _run("llama", 5.0, capsys, budgets_stage_only=(3.0, 4.0, 6.0), whole=True)


@pytest.mark.timeout(900)
def test_large_full(capsys):
    _run("large", 5.0, capsys)


# the largest part a plan admits: (J/m + 3) * 276 + 256 bytes must stay below
# 2^32 (32-bit offsets inside a region), so J/m <= 15,561,471
MAX_PART_SG = 15_561_471


@pytest.mark.timeout(900)
def test_largest_region_full(capsys):
    """Two workers on a ring at the largest size a plan admits (J/2 at the
    limit, 7.97e9 coordinates) and a budget of 8 bits, so that every
    super-group is 8-bit and each part's region is 4,294,966,012 bytes: code,
    scale and group-code offsets run past 2^31 to within 1,284 bytes of
    2^32.  The Large-share recipe; the oracle follows sampled super-groups at
    the part ends as everywhere else."""
    assert (MAX_PART_SG + 3) * 276 + 256 < 2 ** 32 <= (MAX_PART_SG + 4) * 276 + 256
    _run("large", 8.0, capsys, d=256 * 2 * MAX_PART_SG, n=2)
