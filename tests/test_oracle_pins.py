"""Pins of the CPU oracle against what the DynamiQ pages and mathematics fix.

Each test checks the oracle against something other than itself: the pages'
printed constants, closed forms, invariants, brute force on tiny inputs,
textbook special cases or Monte Carlo statistics.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import pyoracle as po
from tests import regions as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def frac(s):
    n, d = s.split("/")
    return Fraction(int(n), int(d))


def f32_bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


def f32_from_bits(b):
    return np.array([b], np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------------------
# thresholds and allocation (pith review: "What carries the argument",
# referee comments, Fig. 3 caption)
# ---------------------------------------------------------------------------

def test_threshold_ratios_follow_from_per_bit_benefit():
    """Equalising the per-bit benefit of the 4^-b error model gives the pages'
    locked ratios; the oracle's thresholds carry exactly those ratios."""
    g = gold("pages_constants.json")
    err = {b: Fraction(1, 4 ** b) for b in (1, 2, 4, 8, 16)}

    def per_bit(a, b):
        return (err[a] - err[b]) / (b - a)

    assert per_bit(1, 2) == frac(g["per_bit_benefit_1_to_2"]["value"])
    assert per_bit(2, 4) * 2 == frac(g["per_bit_benefit_2_to_4_per_2_bits"]["value"])
    assert per_bit(4, 8) == frac(g["per_bit_benefit_4_to_8"]["value"])
    # threshold T_ab sits where F * per_bit(a, b) is the same for all steps
    assert per_bit(2, 4) / per_bit(1, 2) == frac(g["ratio_T12_over_T24"]["value"])
    assert per_bit(4, 8) / per_bit(2, 4) == frac(g["ratio_T24_over_T48"]["value"])
    assert per_bit(8, 16) / per_bit(4, 8) == frac(g["ratio_T48_over_T816"]["value"])
    # the oracle's thresholds at rho = 1 and at a power of two are exact
    for rho in (1.0, 2.0 ** -20, 0.75):
        t = po.thresholds(f32_bits(rho))
        assert Fraction(float(t[0])) / Fraction(float(t[1])) == frac(g["ratio_T12_over_T24"]["value"])
        assert Fraction(float(t[1])) / Fraction(float(t[2])) == frac(g["ratio_T24_over_T48"]["value"])


def test_threshold_ratios_within_one_rounding_for_random_rho():
    g = gold("pages_constants.json")
    r12 = float(frac(g["ratio_T12_over_T24"]["value"]))
    r24 = float(frac(g["ratio_T24_over_T48"]["value"]))
    rng = np.random.default_rng(1)
    for rho in rng.uniform(1e-12, 1e3, 200).astype(np.float32):
        t = po.thresholds(f32_bits(rho)).astype(np.float64)
        assert abs(t[0] / t[1] - r12) <= 2 * 2.0 ** -24 * r12
        assert abs(t[1] / t[2] - r24) <= 2 * 2.0 ** -24 * r24


def _alloc(F, budget):
    J = len(F)
    o = po.Oracle(256 * J, 1, po.RING, budget)
    # stats for n = 1: F_j is the squared norm of super-group j; build inputs whose
    # squared norm is exactly F_j: one entry sqrt(F) would round, so put F_j as a
    # sum of a single square of an exactly representable value
    g = np.zeros(256 * J, np.float32)
    g[::256] = np.sqrt(F).astype(np.float32)
    o.stats(0, g)
    o.allocate()
    _, Fo, _ = o.stats_arrays()
    return o, Fo


def test_allocation_brute_force_8_super_groups():
    """On 8-super-group inputs, against all 3^8 width assignments:
    (i) the allocation minimises sum F 4^-q among assignments with no more bits
        (the threshold rule is the Lagrangian minimiser of the 4^-b model);
    (ii) it is the threshold-realisable assignment with the most bits within
        budget; (iii) rho is the smallest fp32 that meets the budget."""
    rng = np.random.default_rng(7)
    assigns = np.array(list(itertools.product((2, 4, 8), repeat=8)), dtype=np.int64)
    bits = assigns.sum(1)
    pw = 4.0 ** (-assigns.astype(np.float64))
    n_checked = 0
    for trial in range(300):
        kind = trial % 3
        if kind == 0:
            F = np.exp(rng.uniform(-30, 5, 8))
        elif kind == 1:
            F = rng.lognormal(0, 3, 8)
        else:
            F = np.exp(rng.uniform(-3, 3, 8)) * 1e-6
        budget = float(rng.choice([2.0, 2.5, 3.0, 3.25, 4.0, 4.5, 5.0, 5.5, 6.0, 7.0, 7.9, 8.0, 9.0]))
        o, Fo = _alloc(F, budget)
        F64 = Fo.astype(np.float64)
        q = o.widths().astype(np.int64)
        total = int(q.sum())
        assert total <= budget * 8 + 1e-9
        # (iii) minimal rho
        rb = o.rho_bits()
        assert o.count_bits(rb) == total
        if rb > 0:
            assert o.count_bits(rb - 1) > o.budget_bits()
        # (i) Lagrangian optimality against brute force
        err = pw @ F64
        mine = float((F64 * 4.0 ** (-q.astype(np.float64))).sum())
        best = err[bits <= total].min()
        assert mine <= best * (1 + 1e-9)
        # (ii) widths match the threshold rule at rho, from the printed ratios
        rho = Fraction(float(f32_from_bits(rb)))
        T48 = rho * 16384
        T24 = T48 * Fraction(17, 512)
        for Fj, qj in zip(F64, q):
            Fr = Fraction(float(Fj))
            exp_q = 8 if Fr >= T48 else (4 if Fr >= T24 else 2)
            if exp_q != qj:
                # only a tie inside one fp32 rounding of T24 may differ
                assert abs(Fr - T24) <= T24 * Fraction(1, 2 ** 23)
        n_checked += 1
    assert n_checked == 300


def test_allocation_special_budgets():
    rng = np.random.default_rng(3)
    F = rng.lognormal(0, 2, 64)
    o, _ = _alloc(F, 8.0)
    assert (o.widths() == 8).all() and o.rho_bits() == 0
    o, _ = _alloc(F, 100.0)
    assert (o.widths() == 8).all()
    o, _ = _alloc(F, 2.0)
    assert (o.widths() == 2).all()
    with pytest.raises(ValueError):
        po.Oracle(256, 1, po.RING, 1.99)
    with pytest.raises(ValueError):
        po.Oracle(256, 1, po.RING, float("nan"))


def test_allocation_monotone_in_budget():
    rng = np.random.default_rng(5)
    F = rng.lognormal(0, 3, 500)
    prev = None
    for b in np.linspace(2, 8, 25):
        o, _ = _alloc(F, float(b))
        q = o.widths().astype(np.int64)
        assert q.sum() <= b * 500
        if prev is not None:
            assert (q >= prev).all()  # more budget never lowers a width
        prev = q
    # larger F never gets fewer bits
    order = np.argsort(F)
    assert (np.diff(prev[order]) >= 0).all()


# ---------------------------------------------------------------------------
# statistics (scribe notes, "Key idea and contribution"; referee major 1)
# ---------------------------------------------------------------------------

def test_stats_summation_order_golden():
    cases = {c["name"]: c for c in gold("stats_order.json")["cases"]}
    e = np.zeros(256, np.float32)
    e[0] = 2.0 ** 24
    e[1:8] = 1.0
    o = po.Oracle(256, 1)
    o.stats(0, e)
    s, _, _ = o.stats_arrays()
    assert s[0] == np.float32(cases["sequential_inside_partial"]["expected"])
    e = np.full(256, 0.125, np.float32)
    e[0] = 2.0 ** 24
    e[1:8] = 0.0
    o = po.Oracle(256, 1)
    o.stats(0, e)
    s, _, _ = o.stats_arrays()
    assert s[0] == np.float32(cases["tree_over_partials"]["expected"])


def test_stats_against_fp64_and_mean_corrected_identity():
    rng = np.random.default_rng(11)
    n, J = 4, 64
    gs = [(rng.standard_normal(256 * J) * 10.0 ** rng.uniform(-4, 1, 256 * J) + 0.3).astype(np.float32)
          for _ in range(n)]
    o = po.Oracle(256 * J, n)
    for w in range(n):
        o.stats(w, gs[w])
    o.allocate()
    s, F, mu = o.stats_arrays()
    X = np.stack([g.reshape(J, 256).astype(np.float64) for g in gs])
    s64 = X.sum((0, 2))
    F64 = (X * X).sum((0, 2))
    # per worker: <= 7 sequential adds + 5 tree levels per path, then n-1 folds
    tol = (12 + n) * 2.0 ** -24
    assert (np.abs(s - s64) <= tol * np.abs(X).sum((0, 2)) + 1e-30).all()
    assert (np.abs(F - F64) <= tol * F64 * 1.01 + 1e-30).all()
    assert (np.abs(mu - s64 / (256 * n)) <= np.abs(s64 / (256 * n)) * 2 * tol + 1e-30).all()
    # referee's identity: the mean-subtracted squared norm is F - n S mu^2
    centred = ((X - mu.astype(np.float64)[None, :, None]) ** 2).sum((0, 2))
    ident = F.astype(np.float64) - 256 * n * mu.astype(np.float64) ** 2
    assert np.allclose(centred, ident, rtol=1e-4, atol=1e-6 * F64.max())


def test_stats_bf16_input_equals_f32_of_same_values():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(256 * 8).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation gives exact bf16 values
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    a = po.Oracle(256 * 8, 1)
    a.stats(0, bits)
    b = po.Oracle(256 * 8, 1)
    b.stats(0, xb)
    assert (a.stats_arrays()[0] == b.stats_arrays()[0]).all()
    assert (a.stats_arrays()[1] == b.stats_arrays()[1]).all()


def test_stats_rank_order_enforced():
    o = po.Oracle(256, 2)
    with pytest.raises(RuntimeError):
        o.stats(1, np.zeros(256, np.float32))


# ---------------------------------------------------------------------------
# reorder (scribe notes: equal widths made contiguous)
# ---------------------------------------------------------------------------

def test_reorder_invariants():
    rng = np.random.default_rng(4)
    J = 1000
    g = (rng.standard_normal(256 * J) * np.repeat(10.0 ** rng.uniform(-6, 0, J), 256)).astype(np.float32)
    o = po.Oracle(256 * J, 1, po.RING, 4.3)
    o.stats(0, g)
    o.allocate()
    o.reorder()
    w = o.widths()
    perm, inv = o.perm()
    C = o.class_counts()
    assert sorted(perm.tolist()) == list(range(J))
    assert (inv[perm] == np.arange(J)).all()
    assert (perm[inv] == np.arange(J)).all()
    assert [int((w == q).sum()) for q in (2, 4, 8)] == C.tolist()
    ws = w[perm]
    assert (np.diff(ws.astype(int)) >= 0).all()          # 2s, then 4s, then 8s
    for q in (2, 4, 8):
        idx = perm[ws == q]
        assert (np.diff(idx) > 0).all()                    # stable


# ---------------------------------------------------------------------------
# level tables (scribe notes: more levels near zero; ledger: f(eps, r))
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("q", [2, 4, 8])
def test_level_table_shape(q):
    L, W = po.levels(q)
    Q = 1 << q
    assert L[0] == -1.0 and L[-1] == 1.0
    assert (L == -L[::-1]).all()                          # symmetric
    assert (np.diff(L) > 0).all()                         # strictly increasing
    gaps = np.diff(L.astype(np.float64))
    half = gaps[Q // 2:]                                  # gaps above zero
    assert (np.diff(half) > 0).all()                      # denser near zero
    assert 0.0 not in L                                   # no zero level
    # W is 65536 / gap to within one fp32 rounding
    assert np.allclose(W.astype(np.float64) * gaps, 65536.0, rtol=2 ** -23)


def test_level_table_closed_forms():
    L, _ = po.levels(2)
    assert L[2] == np.float32(2.0 / 9.0) and L[1] == -np.float32(2.0 / 9.0)
    for q in (2, 4, 8):
        Q = 1 << q
        Lu, _ = po.levels(q, eps=1.0)                      # eps = 1 is the uniform grid
        expect = np.array([(2 * r + 1 - Q) / (Q - 1) for r in range(Q)], np.float64).astype(np.float32)
        assert (Lu == expect).all()
    L8, _ = po.levels(8)
    # outermost gap / innermost gap tends to 3 for phi(t) = t (1 + t) / 2
    g = np.diff(L8.astype(np.float64))
    assert 2.9 < g[-1] / g[127] < 3.0


# ---------------------------------------------------------------------------
# codec (scribe notes: hierarchical UINT8 scales, unbiased stochastic rounding)
# ---------------------------------------------------------------------------

def _test_vectors(rng):
    out = []
    y = (rng.standard_normal(256) * 10.0 ** rng.uniform(-3, 0, 256)).astype(np.float32)
    out.append(y)
    y = np.zeros(256, np.float32)
    y[37] = 5.0
    y[200] = -0.01
    out.append(y)                                        # single outliers, zero groups
    y = rng.laplace(0, 1e-5, 256).astype(np.float32)
    y[:16] = 0.0
    out.append(y)
    return out


def _d23_gate(z):
    z = z[np.isfinite(z)]
    N = z.size
    frac3 = np.mean(np.abs(z) > 3)
    assert frac3 <= 0.0027 + 4 * np.sqrt(0.0027 / N), frac3
    assert abs(z.mean()) <= 4 / np.sqrt(N), z.mean()
    assert abs(np.mean(z * z) - 1) <= 5 * np.sqrt(2 / N), np.mean(z * z)


@pytest.mark.parametrize("q", [2, 4, 8])
def test_codec_unbiased_monte_carlo(q):
    """Mean of the decoded value over 10^4 independent dithers equals the
    input within the sampling error (z-test gate over all coordinates)."""
    rng = np.random.default_rng(100 + q)
    K = 10000
    zs = []
    for y in _test_vectors(rng):
        d = rng.integers(0, 65536, size=(K, 256), dtype=np.uint16)
        dec = po.roundtrip_batch(np.tile(y, (K, 1)), q, d).astype(np.float64)
        m = dec.mean(0)
        sd = dec.std(0, ddof=1)
        const = sd == 0
        # coordinates with no randomness are decoded exactly, up to the 2^-17
        # resolution of the 16-bit dither compare
        A = float(np.abs(y).max())
        assert np.all(np.abs(m[const] - y[const]) <= A * 2.0 ** -15)
        z = (m[~const] - y[~const]) / (sd[~const] / np.sqrt(K))
        zs.append(z)
    _d23_gate(np.concatenate(zs))


@pytest.mark.parametrize("q", [2, 4, 8])
def test_codec_deterministic_bounds(q):
    rng = np.random.default_rng(200 + q)
    L, _ = po.levels(q)
    for y in _test_vectors(rng):
        for _ in range(20):
            d = rng.integers(0, 65536, 256, dtype=np.uint16)
            dec, codes, s, cg = po.roundtrip_sg(y, q, d)
            a = np.abs(y.reshape(16, 16)).max(1)
            A = a.max()
            # scale unit s covers A after its 255 steps, and is the fp32 A/255 or just above
            assert np.float32(255) * np.float32(s) >= A
            assert s >= np.float32(A) / np.float32(255)
            for g in range(16):
                sig = np.float32(cg[g]) * np.float32(s)
                assert sig >= a[g]                                   # coverage
                if cg[g] > 0:
                    assert np.float32(cg[g] - 1) * np.float32(s) < a[g]  # minimality
            sig = (cg.astype(np.float32) * np.float32(s)).repeat(16)
            v = np.clip(y * np.where(sig > 0, np.float32(1) / np.where(sig > 0, sig, 1), 0), -1, 1)
            # the decoded value is one of the two levels around v
            r = np.searchsorted(L, v, side="right") - 1
            r = np.clip(r, 0, (1 << q) - 2)
            assert np.all((codes == r) | (codes == r + 1))
            width = sig.astype(np.float64) * (L[r + 1].astype(np.float64) - L[r])
            assert np.all(np.abs(dec.astype(np.float64) - y) <= width * (1 + 1e-6) + 1e-30)


def test_codec_zero_and_exact_levels():
    d = np.arange(256, dtype=np.uint16) * 251
    dec, codes, s, cg = po.roundtrip_sg(np.zeros(256, np.float32), 8, d)
    assert s == 0 and (cg == 0).all() and (dec == 0).all()
    # inputs exactly on levels (group max 1 so sigma = 1 on every group) are kept
    L, _ = po.levels(4)
    y = np.tile(L, 16).astype(np.float32)
    rng = np.random.default_rng(0)
    for _ in range(5):
        dec, codes, s, cg = po.roundtrip_sg(y, 4, rng.integers(0, 65536, 256, dtype=np.uint16))
        sig = (cg.astype(np.float32) * np.float32(s))
        assert np.all(dec == (sig.repeat(16) * L[codes]))
        assert np.all(np.float32(cg) * np.float32(s) >= 1.0)


def test_codec_eps1_q8_is_uniform_stochastic_rounding():
    """With eps = 1 and q = 8 the codec is plain unbiased stochastic rounding
    onto a 256-point uniform grid scaled by the group scale (the QSGD-style
    textbook quantiser)."""
    rng = np.random.default_rng(9)
    y = rng.standard_normal(256).astype(np.float32)
    grid = np.array([(2 * r - 255) / 255 for r in range(256)], np.float64).astype(np.float32)
    for _ in range(10):
        d = rng.integers(0, 65536, 256, dtype=np.uint16)
        dec, codes, s, cg = po.roundtrip_sg(y, 8, d, eps=1.0)
        sig = (cg.astype(np.float32) * np.float32(s)).repeat(16)
        assert np.all(dec == sig * grid[codes])
        # stochastic rounding onto that grid: the floor or the ceiling of v
        v = np.clip(y * (np.float32(1) / sig), -1, 1).astype(np.float64)
        pos = (v * 255 + 255) / 2
        assert np.all((codes == np.floor(pos).clip(0, 254)) | (codes == np.floor(pos).clip(0, 254) + 1))


def test_codec_rounding_probability_matches_dither_threshold():
    """For a fixed input the code is r+1 exactly for dithers d with
    d + 0.5 <= 65536 p, so the count of rounding-up dithers is 65536 p
    to within one dither."""
    y = np.zeros(256, np.float32)
    y[0] = 1.0           # group 0: sigma >= 1
    y[1] = 0.3
    y[2] = -0.61
    L, _ = po.levels(4)
    ups = np.zeros(3)
    for d0 in range(0, 65536, 16):
        d = np.full(256, d0, np.uint16)
        dec, codes, s, cg = po.roundtrip_sg(y, 4, d)
        sigma = np.float32(cg[0]) * np.float32(s)
        v = np.float64(np.float32(y[1:3]) * (np.float32(1) / sigma))
        r = np.searchsorted(L, v, side="right") - 1
        ups[1:] += codes[1:3] == r + 1
    sigma = np.float64(np.float32(cg[0]) * np.float32(s))
    for t, idx in ((1, 1), (2, 2)):
        v = np.float64(np.float32(y[idx]) * (np.float32(1) / np.float32(sigma)))
        r = np.searchsorted(L, v, side="right") - 1
        p = (v - L[r]) / (np.float64(L[r + 1]) - L[r])
        assert abs(ups[t] / 4096 - p) <= 2.0 / 4096


def test_codec_rounding_counts_every_dither_at_a_tie():
    """Over all 65,536 dithers the number that round up is floor(P + 1/2)
    for P = 65536 x (position in the interval), computed in fp32 as the
    codec defines it; at a tie P = k + 1/2 that is k + 1 (d + 0.5 <= P
    rounds up).  Enumerated on a coordinate whose P is an exact tie."""
    Q, q = 16, 4
    L, W = po.levels(q)
    base = np.zeros(256, np.float32)
    base[::16] = 1.0                      # every group: a_g = 1, the same sigma
    _, _, s, cg = po.roundtrip_sg(base, q, np.zeros(256, np.uint16))
    sigma = np.float32(cg[0]) * np.float32(s)
    inv = np.float32(1) / sigma
    rng = np.random.default_rng(5)
    y1 = rng.uniform(-0.95, 0.95, 2_000_000).astype(np.float32)
    v = (y1 * inv).astype(np.float32)
    r = np.clip(np.searchsorted(L, v, side="right") - 1, 0, Q - 2)
    P = ((v - L[r]).astype(np.float32) * W[r]).astype(np.float32)
    ties = np.flatnonzero((P - np.floor(P) == 0.5) & (P > 1000))
    assert ties.size > 0
    i = ties[0]
    y = base.copy()
    mask = np.ones(256, bool)
    mask[::16] = False
    y[mask] = y1[i]
    slots = np.flatnonzero(mask)          # 240 coordinates with this P
    ups = 0
    for d0 in range(0, 65536, slots.size):
        d = np.zeros(256, np.uint16)
        ds = np.arange(d0, min(d0 + slots.size, 65536))
        d[slots[:ds.size]] = ds
        _, codes, _, _ = po.roundtrip_sg(y, q, d)
        c = codes[slots[:ds.size]].astype(np.int64)
        assert np.all((c == r[i]) | (c == r[i] + 1))
        ups += int(np.sum(c == r[i] + 1))
    assert ups == int(np.floor(P[i])) + 1, (ups, P[i])


def test_codec_unbiased_where_one_over_sigma_overflows():
    """A group of values of a few 2^-145 has a subnormal scale unit and
    1/sigma = inf: its zeros still quantise without bias (v = 0: the two
    central levels, half each, mean 0) and its other values go to +-1."""
    rng = np.random.default_rng(8)
    k = rng.integers(1, 2000, 128).astype(np.float32)
    y = np.empty(256, np.float32)
    y[0::2] = k * np.float32(2.0 ** -145)
    y[1::2] = -y[0::2]
    zero = rng.random(256) < 0.3
    y[zero] = 0.0
    for q in (2, 4, 8, 16):
        Q = 1 << q
        K = 2000
        dec = np.stack([po.roundtrip_sg(y, q, rng.integers(0, 65536, 256).astype(np.uint16))[0]
                        for _ in range(K)])
        _, codes, s, cg = po.roundtrip_sg(y, q, rng.integers(0, 65536, 256).astype(np.uint16))
        sigma = np.float32(cg[0]) * np.float32(s)
        assert sigma > 0 and np.isinf(np.float32(1) / sigma)
        assert set(np.unique(codes[zero])) <= {Q // 2 - 1, Q // 2}
        assert np.all(codes[~zero & (y > 0)] == Q - 1) and np.all(codes[~zero & (y < 0)] == 0)
        z = dec[:, zero].astype(np.float64)
        sd = z.std(0)
        assert np.all(z[:, sd == 0] == 0)     # 16 bits: sigma L underflows to 0
        if np.any(sd > 0):
            zs = z.mean(0)[sd > 0] / (sd[sd > 0] / np.sqrt(K))
            assert np.abs(zs).max() < 5, (q, np.abs(zs).max())


# ---------------------------------------------------------------------------
# Philox and dithers (SC'11 Philox4x32-10; scribe notes: shared randomness)
# ---------------------------------------------------------------------------

def test_philox_matches_rocrand(tmp_path):
    """The oracle's Philox4x32-10 equals rocRAND's, an independent
    implementation of the same published generator: its header-only engine,
    compiled for the host (tests/native/philox_rocrand.cpp), on edge-value and
    random counters and keys.  rocRAND's engine takes the counter's words x, y
    from offset / 4 (so y < 2^30 here) and z, w from the subsequence."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc or the rocRAND headers are not available")
    src = os.path.join(os.path.dirname(__file__), "native", "philox_rocrand.cpp")
    exe = str(tmp_path / "philox_rocrand")
    subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, capture_output=True)
    rng = np.random.default_rng(2024)
    M = 0xFFFFFFFF
    cases = [[0, 0, 0, 0, 0, 0], [1, 0, 0, 0, 0, 0], [M, 0, 0, 0, 0, 0], [0, 1, 0, 0, 0, 0],
             [0, 0, 1, 0, 0, 0], [0, 0, 0, 1, 0, 0], [0, 0, 0, 0, 1, 0], [0, 0, 0, 0, 0, 1],
             [M, (1 << 30) - 1, M, M, M, M]]
    for _ in range(2000):
        w = rng.integers(0, 1 << 32, 6, dtype=np.uint64)
        w[1] &= (1 << 30) - 1
        cases.append([int(v) for v in w])
    text = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    assert len([l for l in out if l.strip()]) == len(cases)
    for c, line in zip(cases, out):
        theirs = [int(h, 16) for h in line.split()]
        mine = [int(v) for v in po.philox4x32(c[:4], c[4:])]
        assert mine == theirs, (c, mine, theirs)


def test_philox_statistics():
    """Statistics of the oracle's Philox4x32-10 (its identity with the
    published generator is checked against rocRAND above)."""
    key = np.array([0x12345678, 0x9ABCDEF0], np.uint32)
    outs = np.array([po.philox4x32([i, 7, 0, 0], key) for i in range(20000)], np.uint32)
    lanes = np.concatenate([outs & 0xFFFF, outs >> 16]).ravel()
    # chi-square on the top 8 bits of 16-bit lanes
    hist = np.bincount((lanes >> 8).astype(np.int64), minlength=256)
    exp = lanes.size / 256
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert 150 < chi2 < 370                        # 255 dof, far tails excluded
    # serial correlation of consecutive 16-bit lanes
    u = lanes.astype(np.float64) / 65536
    c = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(c) < 0.01
    # avalanche: flipping one counter bit flips about half of the 128 output bits
    flips = []
    for i in range(300):
        a = po.philox4x32([i, 5, 9, 1], key)
        for bit in (0, 13, 31):
            b = po.philox4x32([i ^ (1 << bit), 5, 9, 1], key)
            flips.append(sum(bin(int(x) ^ int(y)).count("1") for x, y in zip(a, b)))
    assert abs(np.mean(flips) - 64) < 1.5
    # rounds matter; zero rounds is the identity
    assert (po.philox4x32([1, 2, 3, 4], key, rounds=0) == [1, 2, 3, 4]).all()
    assert (po.philox4x32([1, 2, 3, 4], key, 10) != po.philox4x32([1, 2, 3, 4], key, 9)).any()


def test_dither_layout_and_correlation():
    n = 8
    base = po.dithers(123, 4, 77, po.CORRELATED, 0, n, 0)
    for w in range(1, n):
        dw = po.dithers(123, 4, 77, po.CORRELATED, w, n, 5)  # event is ignored in correlated mode
        assert np.all((dw.astype(np.int64) - base) % 65536 == (w * 65536) // n)
    # the 16-bit lanes come from consecutive Philox words
    key = np.array([123, 0], np.uint32)
    out = po.philox4x32([3, 77, 4, 0], key)
    for t in range(8):
        word = int(out[t >> 1])
        assert base[24 + t] == ((word >> 16) if t & 1 else (word & 0xFFFF))
    # independent events, other super-groups, rounds and seeds give other dithers
    ind = [po.dithers(123, 4, 77, po.INDEPENDENT, 0, n, e) for e in range(3)]
    assert (ind[0] != ind[1]).mean() > 0.99 and (ind[1] != ind[2]).mean() > 0.99
    assert (po.dithers(123, 4, 78, po.CORRELATED, 0, n, 0) != base).mean() > 0.99
    assert (po.dithers(123, 5, 77, po.CORRELATED, 0, n, 0) != base).mean() > 0.99
    assert (po.dithers(124, 4, 77, po.CORRELATED, 0, n, 0) != base).mean() > 0.99
    hi = po.dithers(123 + (1 << 32), 4, 77, po.CORRELATED, 0, n, 0)
    assert (hi != base).mean() > 0.99


def test_correlated_rounding_lowers_variance_canonical():
    """n workers quantise fixed inputs in parallel (the setting of the
    correlated-quantisation reference): staggered shared dithers give a lower
    variance of the sum than independent dithers, and each worker stays
    unbiased."""
    rng = np.random.default_rng(21)
    n, K, q = 8, 4000, 4
    xs = (rng.standard_normal((n, 256)) * 0.3 + rng.standard_normal(256) * 0.5).astype(np.float32)
    U = rng.integers(0, 65536, size=(K, 256), dtype=np.int64)
    tot_c = np.zeros((K, 256))
    tot_i = np.zeros((K, 256))
    for w in range(n):
        dc = ((U + (w * 65536) // n) % 65536).astype(np.uint16)
        di = rng.integers(0, 65536, size=(K, 256), dtype=np.uint16)
        dec_c = po.roundtrip_batch(np.tile(xs[w], (K, 1)), q, dc).astype(np.float64)
        dec_i = po.roundtrip_batch(np.tile(xs[w], (K, 1)), q, di).astype(np.float64)
        tot_c += dec_c
        tot_i += dec_i
        sd = dec_c.std(0, ddof=1)
        ok = sd > 0
        z = (dec_c.mean(0)[ok] - xs[w][ok]) / (sd[ok] / np.sqrt(K))
        assert np.mean(np.abs(z) > 4) < 0.01
    var_c = tot_c.var(0).sum()
    var_i = tot_i.var(0).sum()
    assert var_c < 0.8 * var_i


# ---------------------------------------------------------------------------
# parts and regions
# ---------------------------------------------------------------------------

def test_region_layout_and_part_nesting():
    rng = np.random.default_rng(8)
    J = 777
    g = (rng.standard_normal(256 * J) * np.repeat(10.0 ** rng.uniform(-6, 0, J), 256)).astype(np.float32)
    o = po.Oracle(256 * J, 8, po.BUTTERFLY, 5.0)
    for w in range(8):
        o.stats(w, g)
    o.allocate()
    o.reorder()
    C = o.class_counts()
    for m in (1, 2, 4, 8):
        tot = 0
        for c in range(m):
            b, cnt = o.region_bytes(m, c)
            assert b == R.region_bytes(C, m, c)
            assert list(cnt) == [n for _, n in R.part_ranges(C, m, c)]
            tot += int(cnt.sum())
            if m < 8:
                ch = [R.part_ranges(C, 2 * m, 2 * c + h) for h in (0, 1)]
                pr = R.part_ranges(C, m, c)
                for k in range(3):
                    assert ch[0][k][0] == pr[k][0]
                    assert ch[0][k][0] + ch[0][k][1] == ch[1][k][0]
                    assert ch[1][k][0] + ch[1][k][1] == pr[k][0] + pr[k][1]
        assert tot == J


# ---------------------------------------------------------------------------
# whole pipeline
# ---------------------------------------------------------------------------

def _grads(rng, n, J, scale_spread=3.0):
    s = np.repeat(10.0 ** rng.uniform(-scale_spread, 0, J), 256)
    return [(rng.standard_normal(256 * J) * s).astype(np.float32) for _ in range(n)]


def test_pipeline_n1_is_single_vector_quantisation():
    """With one worker the round is compress then decode: the output is the
    codec's decode of g - mu plus mu."""
    rng = np.random.default_rng(31)
    J = 5
    g = _grads(rng, 1, J)[0] + np.float32(0.01)
    for mode in (po.STRATIFIED, po.CORRELATED, po.INDEPENDENT):
        o = po.Oracle(256 * J, 1, po.RING, 5.0, seed=9, rounding=mode)
        out = o.allreduce([g])
        _, _, mu = o.stats_arrays()
        w = o.widths()
        for j in range(J):
            y = (g[256 * j:256 * (j + 1)] - mu[j]).astype(np.float32)
            # one worker: stratified takes tag 1, correlated tag 0 with no
            # stagger, independent tag 1 + event 0
            d = po.dithers_tagged(9, 0, j, 0 if mode == po.CORRELATED else 1, 0)
            dec, _, _, _ = po.roundtrip_sg(y, int(w[j]), d)
            assert np.all(out[256 * j:256 * (j + 1)] == dec + np.float32(1) * mu[j])


def test_pipeline_constant_and_zero_super_groups_exact():
    n, J = 4, 6
    rng = np.random.default_rng(5)
    gs = _grads(rng, n, J)
    for g in gs:
        g[0:256] = 0.0             # all-zero super-group
        g[512:768] = 0.375         # the same constant on every worker
    for topo in (po.RING, po.BUTTERFLY):
        o = po.Oracle(256 * J, n, topo, 5.0)
        out = o.allreduce(gs)
        assert np.all(out[0:256] == 0.0)
        assert np.all(out[512:768] == np.float32(n * 0.375))


def test_pipeline_budget_and_determinism():
    rng = np.random.default_rng(6)
    n, J = 4, 300
    gs = _grads(rng, n, J, 6)
    for b in (3.0, 4.0, 5.0, 6.0):
        o = po.Oracle(256 * J, n, po.RING, b)
        out1 = o.allreduce(gs)
        assert o.widths().astype(np.int64).sum() <= b * J
        o2 = po.Oracle(256 * J, n, po.RING, b)
        po.set_threads(1)
        out2 = o2.allreduce(gs)
        po.set_threads(os.cpu_count() or 1)
        assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))


def test_pipeline_error_bound_per_event():
    """Per coordinate, |out - exact sum| is at most the sum over quantisation
    events of that event's interval width (plus fp32 additions)."""
    rng = np.random.default_rng(12)
    n, J = 4, 40
    gs = _grads(rng, n, J)
    o = po.Oracle(256 * J, n, po.RING, 4.0)
    for w in range(n):
        o.stats(w, gs[w])
    o.allocate()
    o.reorder()
    C = o.class_counts()
    perm, _ = o.perm()
    RB = o.worst_region_bytes()
    bufs = [[np.zeros(RB, np.uint8) for _ in range(n)] for _ in range(2)]
    bound = np.zeros(256 * J)
    maxgap = {q: np.diff(po.levels(q)[0].astype(np.float64)).max() for q in (2, 4, 8)}

    def add_bound(region, part):
        for k, (lo, cnt) in enumerate(R.part_ranges(C, n, part)):
            for pos in range(lo, lo + cnt):
                kk, codes, s, cg = R.sg_fields(region, C, n, part, pos)
                sig = (cg.astype(np.float64) * float(s)).repeat(16)
                j = perm[pos]
                bound[256 * j:256 * (j + 1)] += sig * maxgap[R.QS[kk]]

    for w in range(n):
        o.compress(w, 0, gs[w], bufs[0][w])
        add_bound(bufs[0][w], w)
    for t in range(1, n):
        for w in range(n):
            o.hop(w, t, bufs[(t - 1) % 2][(w - 1) % n], gs[w], bufs[t % 2][w])
            add_bound(bufs[t % 2][w], (w - t) % n)
    out = np.zeros(256 * J, np.float32)
    for w in range(n):
        o.finalize(o.final_part(w), bufs[(n - 1) % 2][w], out)
    exact = np.sum([g.astype(np.float64) for g in gs], 0)
    slack = 64 * 2.0 ** -24 * (np.abs(exact) + bound + np.abs(np.sum([np.abs(g) for g in gs], 0)))
    assert np.all(np.abs(out - exact) <= bound + slack)
    # and the schedule-level call reproduces the step-by-step run bit for bit
    o2 = po.Oracle(256 * J, n, po.RING, 4.0)
    assert np.array_equal(o2.allreduce(gs).view(np.uint32), out.view(np.uint32))


def _round_z(mode, topo, n=4, J=2, K=10000, seed=13):
    """z-scores of the mean all-reduced sum over K rounds against the exact sum."""
    rng = np.random.default_rng(seed)
    gs = _grads(rng, n, J, 2)
    exact = np.sum([g.astype(np.float64) for g in gs], 0)
    o = po.Oracle(256 * J, n, topo, 3.0, seed=77, rounding=mode)
    outs = np.zeros((K, 256 * J))
    for r in range(K):
        po.lib().or_set_round(o.h, r)
        outs[r] = o.allreduce(gs)
    sd = outs.std(0, ddof=1)
    ok = sd > 0
    return (outs.mean(0)[ok] - exact[ok]) / (sd[ok] / np.sqrt(K))


@pytest.mark.parametrize("mode", [po.INDEPENDENT, po.STRATIFIED], ids=["independent", "stratified"])
def test_pipeline_unbiased(mode):
    """Independent and level-stratified dithers: every quantisation's dither
    is independent of its input, so the all-reduced sum is unbiased (Monte
    Carlo over 10^4 rounds, z-test gate of D23), ring and butterfly."""
    _d23_gate(np.concatenate([_round_z(mode, topo) for topo in (po.RING, po.BUTTERFLY)]))


def test_pipeline_rank_staggered_rounding_is_biased():
    """One shared uniform for every hop of a chain, staggered by rank: a
    later hop reuses randomness its input already depends on, and the mean
    over rounds drifts away from the exact sum (why it is not the default)."""
    z = _round_z(po.CORRELATED, po.RING)
    assert np.abs(z).max() > 10


def test_stratified_rounding_lowers_butterfly_error():
    """Level-stratified dithers reduce the error of the butterfly, whose
    levels hold workers quantising the same coordinates in parallel, below
    independent dithers; the ring's hops are all in series, so there the two
    agree in distribution."""
    rng = np.random.default_rng(44)
    n, J = 8, 64
    gs = _grads(rng, n, J, 2)
    b_s = _vnmse(po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rounding=po.STRATIFIED), gs, range(12))
    b_i = _vnmse(po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rounding=po.INDEPENDENT), gs, range(12))
    r_s = _vnmse(po.Oracle(256 * J, n, po.RING, 5.0, rounding=po.STRATIFIED), gs, range(12))
    r_i = _vnmse(po.Oracle(256 * J, n, po.RING, 5.0, rounding=po.INDEPENDENT), gs, range(12))
    assert b_s < 0.9 * b_i, (b_s, b_i)
    assert abs(r_s / r_i - 1) < 0.1, (r_s, r_i)


def _vnmse(o, gs, rounds):
    exact = np.sum([g.astype(np.float64) for g in gs], 0)
    v = []
    for r in rounds:
        po.lib().or_set_round(o.h, r)
        out = o.allreduce(gs)
        v.append(np.sum((out - exact) ** 2) / np.sum(exact ** 2))
    return float(np.mean(v))


@pytest.mark.parametrize("n", [8, 16])
def test_butterfly_error_below_ring(n):
    """Fewer requantisations of large partial sums: with independent dithers the
    butterfly vNMSE is below the ring's at equal n (pith review, 'If this is
    right').  Quantisation variance grows with the size of the partial sum, so
    the ring's events add up as 1 + 2 + ... + n and the butterfly's as
    (n/2)(1 + 2) + n (log2 n - 1): 36 vs 28 at n = 8, 136 vs 88 at n = 16.
    With correlated dithers the ring's staggered shared dithers also cancel
    errors along its hops, so that mode is reported, not gated."""
    rng = np.random.default_rng(40 + n)
    J = 64
    gs = _grads(rng, n, J, 2)
    ring = _vnmse(po.Oracle(256 * J, n, po.RING, 5.0, rounding=po.INDEPENDENT), gs, range(10))
    bfly = _vnmse(po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rounding=po.INDEPENDENT), gs, range(10))
    units = {8: 28 / 36, 16: 88 / 136}[n]
    assert bfly < ring
    assert abs(bfly / ring - units) < 0.15, (bfly / ring, units)
    ring_c = _vnmse(po.Oracle(256 * J, n, po.RING, 5.0, rounding=po.CORRELATED), gs, range(10))
    bfly_c = _vnmse(po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rounding=po.CORRELATED), gs, range(10))
    print(f"n={n} independent ring {ring:.3e} butterfly {bfly:.3e}; "
          f"correlated ring {ring_c:.3e} butterfly {bfly_c:.3e}")


def test_ring_and_butterfly_agree_at_n2():
    """At n = 2 both schedules quantise each coordinate once alone and once as
    a two-worker sum, so their vNMSE agree in distribution."""
    rng = np.random.default_rng(2)
    J = 64
    gs = _grads(rng, 2, J, 2)
    ring = _vnmse(po.Oracle(256 * J, 2, po.RING, 5.0, rounding=po.INDEPENDENT), gs, range(20))
    bfly = _vnmse(po.Oracle(256 * J, 2, po.BUTTERFLY, 5.0, rounding=po.INDEPENDENT), gs, range(20))
    assert abs(bfly / ring - 1) < 0.1


def test_mxfp8_reference_quantiser():
    # exactly representable values survive; magnitudes saturate at the block max
    x = np.array([1.0, -1.5, 448.0 / 256, 0.0, 2.0 ** -6 / 256, 0.875] + [0.0] * 26, np.float32)
    assert np.array_equal(po.mxfp8_roundtrip(x), x)
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(32 * 1000) * np.repeat(10.0 ** rng.uniform(-8, 2, 1000), 32)).astype(np.float32)
    y = po.mxfp8_roundtrip(x)
    blk = np.abs(x).reshape(-1, 32).max(1).repeat(32).astype(np.float64)
    X = 2.0 ** (np.floor(np.log2(blk)) - 8)            # E8M0 shared scale
    v = np.abs(x) / X
    # E4M3 normal range: relative error <= 2^-4 (3 mantissa bits, nearest)
    normal = (v >= 2.0 ** -6) & (v <= 448)
    assert np.all(np.abs(y - x)[normal] <= np.abs(x[normal]) * 2.0 ** -4 * (1 + 1e-6))
    # above the largest normal the element saturates at 448
    sat = v > 448
    assert sat.any() and np.all(np.abs(y[sat]) == (448 * X[sat]).astype(np.float32))
    # subnormal range: absolute error <= half the 2^-9 quantum
    sub = v < 2.0 ** -6
    assert np.all(np.abs(y - x)[sub] <= 2.0 ** -10 * X[sub] * (1 + 1e-6))
    # a block's max never moves by more than one E4M3 step
    assert np.all(np.abs(y) <= blk * (1 + 2.0 ** -3))


def test_mxfp8_schedule_composition():
    """The MXFP8 reference round is the plain composition of block
    quantisations along the schedule: one worker = one quantisation; a 2-worker
    ring quantises each half once alone and once as a two-worker sum."""
    rng = np.random.default_rng(17)
    J = 12
    g = [(rng.standard_normal(256 * J) * np.repeat(10.0 ** rng.uniform(-4, 0, J), 256)).astype(np.float32)
         for _ in range(2)]
    o1 = po.Oracle(256 * J, 1)
    assert np.array_equal(o1.mxfp8_allreduce(g[:1]), po.mxfp8_roundtrip(g[0]))
    h = 256 * (J // 2)
    o2 = po.Oracle(256 * J, 2, po.RING)
    out = o2.mxfp8_allreduce(g)
    # ring n = 2: worker 0 sends part 0, worker 1 reduces it; and the reverse for part 1
    exp0 = po.mxfp8_roundtrip(po.mxfp8_roundtrip(g[0][:h]) + g[1][:h])
    exp1 = po.mxfp8_roundtrip(po.mxfp8_roundtrip(g[1][h:]) + g[0][h:])
    assert np.array_equal(out, np.concatenate([exp0, exp1]))
    ob = po.Oracle(256 * J, 2, po.BUTTERFLY)
    outb = ob.mxfp8_allreduce(g)
    # butterfly n = 2: worker 0 keeps half 0 and receives worker 1's quantised half 0
    exp0 = po.mxfp8_roundtrip(po.mxfp8_roundtrip(g[1][:h]) + g[0][:h])
    exp1 = po.mxfp8_roundtrip(po.mxfp8_roundtrip(g[0][h:]) + g[1][h:])
    assert np.array_equal(outb, np.concatenate([exp0, exp1]))


# ---------------------------------------------------------------------------
# allocation variants (pith.science review, referee major 1; Table 6; the
# "Load-bearing premise" on spatial locality and Fig. 1's shuffled norms)
# ---------------------------------------------------------------------------

def _variant_round(gs, budget, alloc, topo=po.RING):
    n, d = len(gs), gs[0].size
    o = po.Oracle(d, n, topo, budget, alloc=alloc)
    for w in range(n):
        o.stats(w, gs[w])
    o.allocate()
    return o


def test_mean_corrected_key_is_centred_energy():
    """G_j against the exact squared norm of the mean-subtracted values,
    sum_w sum_i (x - mu_j)^2 in fp64, with large per-SG offsets so that the
    correction term is most of F_j, and constant SGs (exactly 0 in exact
    arithmetic)."""
    rng = np.random.default_rng(21)
    n, J = 4, 96
    off = np.repeat(rng.standard_normal(J) * 10.0 ** rng.uniform(-3, 1, J), 256)
    spread = np.repeat(10.0 ** rng.uniform(-6, 0, J), 256)
    gs = [(off + spread * rng.standard_normal(256 * J)).astype(np.float32) for _ in range(n)]
    for g in gs:   # constant super-groups, the same value on every worker
        g[256 * 5:256 * 6] = np.float32(0.37)
    o = _variant_round(gs, 5.0, po.ALLOC_MEAN_CORRECTED)
    G = o.alloc_key().astype(np.float64)
    _, F, mu = o.stats_arrays()
    X = np.stack([g.reshape(J, 256).astype(np.float64) for g in gs])
    mu64 = X.mean((0, 2))
    centred = ((X - mu64[None, :, None]) ** 2).sum((0, 2))
    F64 = (X * X).sum((0, 2))
    eps = 2.0 ** -24
    corr = 256 * n * mu.astype(np.float64) ** 2
    bound = (12 + n) * eps * F64 * 1.01 + 4 * eps * corr + eps * centred \
        + 256 * n * (mu.astype(np.float64) - mu64) ** 2 + 1e-30
    assert (np.abs(G - centred) <= bound).all()
    assert (G >= 0).all()
    # with the offsets, the plain key overstates the quantised energy by far
    assert np.median(F64 / np.maximum(centred, 1e-300)) > 10
    # a sign error or a missing factor n would miss the bound by orders of magnitude
    wrong = F.astype(np.float64) - 256 * mu.astype(np.float64) ** 2
    assert (np.abs(wrong - centred) > bound).any()


def test_mean_corrected_allocation_follows_its_key():
    """Widths are the threshold rule on G at the returned rho; rho is the
    smallest fp32 meeting the budget; SGs with large offsets and small
    spread move to narrow widths."""
    rng = np.random.default_rng(22)
    n, J = 2, 256
    off = np.repeat(np.where(rng.random(J) < 0.3, 50.0, 0.0), 256)
    spread = np.repeat(10.0 ** rng.uniform(-2, 1, J), 256)
    gs = [(off + spread * rng.standard_normal(256 * J)).astype(np.float32) for _ in range(n)]
    for budget in (2.5, 4.0, 5.0, 6.5):
        o = _variant_round(gs, budget, po.ALLOC_MEAN_CORRECTED)
        G = o.alloc_key()
        rb = o.rho_bits()
        rho = f32_from_bits(rb)
        t4, t8 = np.float32(544) * rho, np.float32(16384) * rho

        def count(r):
            r = f32_from_bits(r)
            a4, a8 = np.float32(544) * r, np.float32(16384) * r
            return int((2 + 2 * (G >= a4) + 4 * (G >= a8)).sum())

        q = o.widths().astype(np.int64)
        assert np.array_equal(q, 2 + 2 * (G >= t4) + 4 * (G >= t8))
        assert q.sum() <= o.budget_bits()
        if rb > 0:
            assert count(rb - 1) > o.budget_bits()
        plain = _variant_round(gs, budget, po.ALLOC_THRESHOLD).widths()
        offset_sgs = off[::256] > 0
        assert q[offset_sgs].mean() <= plain[offset_sgs].mean()
        if budget == 5.0:
            assert q[offset_sgs].mean() < plain[offset_sgs].mean()


@pytest.mark.parametrize("budget,q", [(2.0, 2), (3.0, 2), (3.99, 2), (4.0, 4), (5.0, 4), (7.9, 4), (8.0, 8), (9.5, 8)])
def test_uniform_allocation(budget, q):
    rng = np.random.default_rng(23)
    gs = [rng.standard_normal(256 * 40).astype(np.float32) for _ in range(3)]
    o = _variant_round(gs, budget, po.ALLOC_UNIFORM)
    assert (o.widths() == q).all()
    assert o.rho_bits() == 0x7FC00000
    assert o.class_counts().tolist() == [40 * (q == 2), 40 * (q == 4), 40 * (q == 8)]
    assert 40 * q <= o.budget_bits()


@pytest.mark.parametrize("budget", [8.0, 9.5, 1e30, float("inf")])
def test_budgets_of_eight_bits_or_more_give_all_eight(budget):
    """The widths sum to at most 8 J, so any budget of 8 bits or more is met
    at rho = 0 with every super-group 8-bit; the bit budget is then 8 J even
    for a budget whose product with J leaves the integer range."""
    rng = np.random.default_rng(29)
    gs = [rng.standard_normal(256 * 40).astype(np.float32) for _ in range(3)]
    o = _variant_round(gs, budget, po.ALLOC_THRESHOLD)
    assert o.budget_bits() == 8 * 40
    assert o.rho_bits() == 0 and (o.widths() == 8).all()


def test_variable_widths_beat_uniform_unless_shuffled():
    """Table 6 direction: at 4 bits per coordinate, variable widths give a
    lower vNMSE than uniform 4-bit codes on gradients with skewed, spatially
    local SG norms.  Fig. 1 / the load-bearing premise: after a random
    shuffle of coordinates (the same for every worker) the SG norms flatten
    and the advantage mostly disappears."""
    rng = np.random.default_rng(24)
    n, J = 4, 1024
    scale = np.repeat(10.0 ** rng.uniform(-4, 0, J), 256)
    gs = [(scale * rng.standard_normal(256 * J)).astype(np.float32) for _ in range(n)]
    perm = rng.permutation(256 * J)
    shuffled = [g[perm].copy() for g in gs]

    def vnmse(grads, alloc):
        exact = np.sum([g.astype(np.float64) for g in grads], axis=0)
        o = po.Oracle(256 * J, n, po.RING, 4.0, alloc=alloc, rounding=po.INDEPENDENT)
        out = o.allreduce(grads)
        return float(((out - exact) ** 2).sum() / (exact ** 2).sum())

    local_ratio = vnmse(gs, po.ALLOC_UNIFORM) / vnmse(gs, po.ALLOC_THRESHOLD)
    shuffled_ratio = vnmse(shuffled, po.ALLOC_UNIFORM) / vnmse(shuffled, po.ALLOC_THRESHOLD)
    assert local_ratio > 2.0
    assert shuffled_ratio < 1.5
    assert shuffled_ratio < local_ratio / 2


# ---------------------------------------------------------------------------
# MX element formats (OCP Microscaling v1.0), pinned by brute force: every
# element value enumerated from the format's (E, M) fields, nearest value
# with ties to the even code, saturation at the largest finite value
# ---------------------------------------------------------------------------

MX_FORMATS = {  # fmt: (ebits, mbits, emin, emax, max)
    po.MX_E4M3: (4, 3, -6, 8, 448.0),
    po.MX_E3M2: (3, 2, -2, 4, 28.0),
    po.MX_E2M3: (2, 3, 0, 2, 7.5),
    po.MX_E2M1: (2, 1, 0, 2, 6.0),
}


def _mx_values(fmt):
    ebits, mbits, emin, emax, vmax = MX_FORMATS[fmt]
    vals = []
    for E in range(2 ** ebits):
        for M in range(2 ** mbits):
            v = M * 2.0 ** (emin - mbits) if E == 0 else (1 + M / 2 ** mbits) * 2.0 ** (E - 1 + emin)
            if v <= vmax:
                vals.append(v)
    vals = np.array(vals)
    assert np.all(np.diff(vals) > 0) and vals[-1] == vmax
    assert np.floor(np.log2(vmax)) == emax
    return vals


def _mx_brute(fmt, x):
    vals = _mx_values(fmt)
    emax, vmax = MX_FORMATS[fmt][3], MX_FORMATS[fmt][4]
    out = np.zeros_like(x)
    for b in range(0, x.size, 32):
        blk = x[b:b + 32].astype(np.float64)
        amax = np.abs(blk).max()
        se = -127 if amax == 0 else int(np.clip(np.floor(np.log2(amax)) - emax, -127, 127))
        X = 2.0 ** se
        for i, v in enumerate(blk / X):
            a = abs(v)
            if a >= vmax:
                r = vmax
            else:
                k = np.searchsorted(vals, a)          # vals[k-1] < a <= vals[k]
                lo, hi = vals[max(k - 1, 0)], vals[min(k, len(vals) - 1)]
                if a - lo < hi - a:
                    r = lo
                elif hi - a < a - lo:
                    r = hi
                else:                                 # tie: the even code
                    r = lo if (k - 1) % 2 == 0 else hi
            out[b + i] = np.float32((-r if v < 0 else r) * X)
    return out


@pytest.mark.parametrize("fmt", [po.MX_E4M3, po.MX_E3M2, po.MX_E2M3, po.MX_E2M1])
def test_mx_quantiser_brute_force(fmt):
    rng = np.random.default_rng(31 + fmt)
    nb = 300
    x = (rng.standard_normal(32 * nb) * np.repeat(10.0 ** rng.uniform(-6, 3, nb), 32)).astype(np.float32)
    # ties and exact values: blocks built from element values and midpoints
    vals = _mx_values(fmt)
    mids = (vals[:-1] + vals[1:]) / 2
    for b in range(0, 60):
        pick = np.concatenate([vals, mids])[rng.integers(0, 2 * len(vals) - 1, 32)]
        pick[0] = vals[-1]                            # block max at the top value: scale 2^0
        x[32 * b:32 * b + 32] = (pick * np.where(rng.random(32) < 0.5, -1, 1)).astype(np.float32)
    x[32 * 60:32 * 61] = 0.0                          # an all-zero block
    assert np.array_equal(po.mx_roundtrip(fmt, x), _mx_brute(fmt, x))
    if fmt == po.MX_E4M3:
        assert np.array_equal(po.mxfp8_roundtrip(x), po.mx_roundtrip(fmt, x))


def test_mx_e4m3_elements_match_torch_float8():
    """E4M3 element rounding equals torch's float8_e4m3fn cast (an independent
    round-to-nearest-even implementation) wherever the two are defined alike:
    blocks whose maximum lies in [256, 448] have the scale 2^0, and no element
    reaches 464, where torch's cast gives NaN instead of saturating."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    nb = 2000
    x = (np.where(rng.random(32 * nb) < 0.5, -1.0, 1.0) *
         10.0 ** rng.uniform(-4.5, np.log10(448.0), 32 * nb)).astype(np.float32)
    x[::32] = rng.uniform(256.0, 448.0, nb).astype(np.float32)
    # midpoints between neighbouring E4M3 values (ties) in some blocks
    vals = _mx_values(po.MX_E4M3)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    for b in range(200):
        x[32 * b + 1:32 * b + 32] = mids[rng.integers(0, len(mids), 31)] * np.where(rng.random(31) < 0.5, -1, 1)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(po.mx_roundtrip(po.MX_E4M3, x), theirs)


def test_mx_schedule_composition_fp4():
    rng = np.random.default_rng(18)
    J = 12
    g = [(rng.standard_normal(256 * J) * np.repeat(10.0 ** rng.uniform(-4, 0, J), 256)).astype(np.float32)
         for _ in range(2)]
    h = 256 * (J // 2)
    q = lambda v: po.mx_roundtrip(po.MX_E2M1, v)
    out = po.Oracle(256 * J, 2, po.RING).mx_allreduce(po.MX_E2M1, g)
    assert np.array_equal(out, np.concatenate([q(q(g[0][:h]) + g[1][:h]), q(q(g[1][h:]) + g[0][h:])]))


# ---------------------------------------------------------------------------
# butterfly variant: the worker's kept half stays fp32 (no re-quantisation by
# its owner at levels >= 2), against the method's packed own child
# ---------------------------------------------------------------------------

def test_own_fp32_partial_variant():
    rng = np.random.default_rng(41)
    n, J = 8, 96
    scale = np.repeat(10.0 ** rng.uniform(-4, 0, J), 256)
    gs = [(scale * rng.standard_normal(256 * J)).astype(np.float32) for _ in range(n)]
    exact = np.sum([g.astype(np.float64) for g in gs], axis=0)

    def vnmse(own, rounds):
        err = 0.0
        for r in rounds:
            o = po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, rnd=r, rounding=po.INDEPENDENT, own=own)
            err += ((o.allreduce(gs) - exact) ** 2).sum()
        return err / len(rounds) / (exact ** 2).sum()

    packed, f32 = vnmse(po.OWN_PACKED, range(6)), vnmse(po.OWN_F32, range(6))
    # the kept half skips one quantisation per level >= 2: lower error
    assert f32 < 0.85 * packed
    # n = 2 has no level >= 2: the variants coincide bit for bit
    o1 = po.Oracle(256 * J, 2, po.BUTTERFLY, 5.0, own=po.OWN_PACKED).allreduce(gs[:2])
    o2 = po.Oracle(256 * J, 2, po.BUTTERFLY, 5.0, own=po.OWN_F32).allreduce(gs[:2])
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    # the ring never uses an own operand: unchanged
    r1 = po.Oracle(256 * J, 4, po.RING, 5.0, own=po.OWN_PACKED).allreduce(gs[:4])
    r2 = po.Oracle(256 * J, 4, po.RING, 5.0, own=po.OWN_F32).allreduce(gs[:4])
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))


def test_own_fp32_partial_is_the_exact_partial_sum():
    """n = 4: after level 1 the kept child holds x_in + (g - mu) without any
    rounding beyond the one fp32 add, and level 2 adds the partner's decoded
    region to it."""
    rng = np.random.default_rng(42)
    n, J = 4, 40
    gs = [rng.standard_normal(256 * J).astype(np.float32) for _ in range(n)]
    o = po.Oracle(256 * J, n, po.BUTTERFLY, 5.0, own=po.OWN_F32)
    for w in range(n):
        o.stats(w, gs[w])
    o.allocate()
    o.reorder()
    perm, _ = o.perm()
    _, _, mu = o.stats_arrays()
    C = o.class_counts()
    RB = o.worst_region_bytes()
    cmp = {w: np.zeros(RB, np.uint8) for w in range(n)}
    for w in range(n):
        o.compress(w, 1, gs[w], cmp[w])
    # worker 0 at level 1: part 0 of 2; keeps child 0 (bit of w at level 1 is 0)
    w, partner = 0, 2
    sent = np.zeros(RB, np.uint8)
    kept = np.zeros((J, 256), np.float32)
    o.hop(w, 1, cmp[partner], gs[w], kept, sent)
    # expected kept values: decoded incoming + (g - mu) for the SGs of child (4, 0)
    levels = [po.levels(q)[0] for q in (2, 4, 8)]
    for t, p in enumerate(R.part_positions(C, 4, 0)):
        j = perm[p]
        dec = R.decode_sg(cmp[partner], C, 2, 0, p, levels)
        y = (dec + (gs[w][256 * j:256 * j + 256] - mu[j]).astype(np.float32)).astype(np.float32)
        assert np.array_equal(kept[t].view(np.uint32), y.view(np.uint32))
    # and the sent child is a packed region of part (4, 1)
    assert R.region_bytes(C, 4, 1) > 0 and sent[:R.region_bytes(C, 4, 1)].any()


# ---------------------------------------------------------------------------
# MX all-reduce schedule beyond two workers (ring n = 3, 4, 5; butterfly n = 4,
# 8): exact sums and an independent part-by-part composition
# (tests/mx_schedule_checks.py), and copies of the oracle with a planted
# schedule mistake that these checks must catch
# ---------------------------------------------------------------------------

def test_mx_schedule_exact_sums_and_composition():
    from tests import mx_schedule_checks as M
    res = M.run_checks()
    assert len(res) == 2 * 4 * len(M.CASES)
    failed = [k for k, ok in res.items() if not ok]
    assert not failed, failed


def test_mx_exact_sum_inputs_are_exact():
    """The exact-sum inputs really keep every partial sum exact: one
    quantisation of any partial sum of the workers returns it unchanged."""
    from tests import mx_schedule_checks as M
    rng = np.random.default_rng(3)
    for fmt in (po.MX_E4M3, po.MX_E3M2, po.MX_E2M3, po.MX_E2M1):
        g, v = M.exact_sum_inputs(fmt, 5, 16, seed=fmt)
        assert np.array_equal(np.sum(g, axis=0, dtype=np.float32), v)
        for _ in range(20):
            sub = rng.random(5) < 0.5
            part = np.sum([g[w] for w in range(5) if sub[w]] or [np.zeros_like(v)], axis=0, dtype=np.float32)
            assert np.array_equal(po.mx_roundtrip(fmt, part), part)


# each mutation: (what it plants, text in or_mx_allreduce, replacement)
_MX_MUTATIONS = [
    ("ring hop reads worker w+1's region",
     "const int src = (w - 1 + n) % n;", "const int src = (w + 1) % n;"),
    ("ring hop works on part (w + t) mod n",
     "mx_part(c, n, ((int64_t)w - t % n + n) % n, &lo, &hi);", "mx_part(c, n, ((int64_t)w + t) % n, &lo, &hi);"),
    ("butterfly levels >= 2 read another worker's partial than the partner's",
     "const float in = (s == 1) ? nxt[partner][i] : cur[partner][i];",
     "const float in = (s == 1) ? nxt[partner][i] : cur[w ^ 1][i];"),
    ("butterfly level 1 takes the partner's raw gradient",
     "const float in = (s == 1) ? nxt[partner][i] : cur[partner][i];",
     "const float in = (s == 1) ? load_elem(grads[partner], dtype, i) : cur[partner][i];"),
]


@pytest.mark.parametrize("what,old,new", _MX_MUTATIONS, ids=[m[0] for m in _MX_MUTATIONS])
def test_mx_schedule_checks_catch_planted_mistakes(tmp_path, what, old, new):
    """A copy of the oracle with one schedule mistake planted in its MX
    all-reduce, built here and run in a child process, fails the checks."""
    import shutil
    import subprocess
    import sys
    from oracle import build as ob
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    src = open(os.path.join(os.path.dirname(ob.__file__), "oracle.c")).read()
    start = src.index("int or_mx_allreduce(")
    end = src.index("int or_mxfp8_allreduce(")
    body = src[start:end]
    assert body.count(old) == 1, what
    mutated = src[:start] + body.replace(old, new) + src[end:]
    c_path = tmp_path / "oracle_mutant.c"
    c_path.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run([cc] + ob.FLAGS + ["-I", os.path.dirname(ob.__file__), str(c_path), "-o", str(so), "-lm"],
                   check=True)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, DQ_ORACLE_LIB=str(so), PYTHONPATH=root, OMP_NUM_THREADS="4")
    out = subprocess.run([sys.executable, "-m", "tests.mx_schedule_checks"], cwd=root, env=env,
                         check=True, capture_output=True, text=True).stdout
    r = json.loads(out.strip().splitlines()[-1])
    assert r["passed"] < r["total"], f"planted mistake not caught: {what}"


# ---------------------------------------------------------------------------
# exact allocation under the same budget (pith.science review, referee major
# 1 and "What would settle it"): the minimiser of sum_j F_j 4^-q_j, against
# brute force and against the threshold rule
# ---------------------------------------------------------------------------

def _model_cost(F, q):
    return float(np.sum(F.astype(np.float64) * 4.0 ** (-q.astype(np.float64))))


def test_exact_allocation_brute_force_8_super_groups():
    """The dynamic programme returns the least cost over all 3^8 width
    assignments that keep the budget, on skewed random norms and every budget
    from 2 to 8 bits in steps of 1/8 bit per coordinate."""
    rng = np.random.default_rng(21)
    allq = np.array(list(itertools.product((2, 4, 8), repeat=8)), dtype=np.int64)
    for trial in range(60):
        F = (10.0 ** rng.uniform(-8, 0, 8) * rng.uniform(0.5, 2, 8)).astype(np.float32)
        costs = (F.astype(np.float64)[None, :] * 4.0 ** (-allq.astype(np.float64))).sum(1)
        bits = allq.sum(1)
        for b8 in range(16, 65, 3 if trial % 2 else 1):
            budget = b8                     # floor(B * 8) with B = b8 / 8
            w, cost = po.alloc_exact(F, budget)
            assert int(w.astype(np.int64).sum()) <= budget
            assert set(np.unique(w)) <= {2, 4, 8}
            best = costs[bits <= budget].min()
            assert abs(cost - best) <= 1e-12 * best
            assert abs(_model_cost(F, w) - cost) <= 1e-12 * cost


def test_exact_allocation_never_worse_than_threshold_rule():
    """The threshold allocation keeps the budget, so the exact minimum is at
    most its cost; on skewed inputs the threshold rule already comes within a
    small fraction of it."""
    rng = np.random.default_rng(22)
    worse = 0
    for trial in range(40):
        J = 64
        scale = np.repeat(10.0 ** rng.uniform(-5, -1, J), 256)
        gs = [(scale * rng.standard_normal(256 * J)).astype(np.float32) for _ in range(4)]
        for budget in (3.0, 4.0, 5.0, 6.0):
            o = po.Oracle(256 * J, 4, po.RING, budget)
            for w in range(4):
                o.stats(w, gs[w])
            o.allocate()
            _, F, _ = o.stats_arrays()
            q_thr = o.widths().astype(np.int64)
            w_ex, cost = po.alloc_exact(F, o.budget_bits())
            c_thr = _model_cost(F, q_thr)
            assert cost <= c_thr * (1 + 1e-12)
            if cost < c_thr * (1 - 1e-9):
                worse += 1
            assert c_thr <= 1.5 * cost
    # the discrete 4 -> 8 step leaves the threshold rule short of the optimum
    # in some instances (its allocation is optimal only for its own bit count)
    assert worse > 0


def test_exact_allocation_special_budgets_and_pipeline():
    rng = np.random.default_rng(23)
    F = (10.0 ** rng.uniform(-6, 0, 100)).astype(np.float32)
    assert np.all(po.alloc_exact(F, 200)[0] == 2)          # 2 bits per super-group
    assert np.all(po.alloc_exact(F, 800)[0] == 8)          # 8 bits
    assert np.all(po.alloc_exact(F, 10 ** 6)[0] == 8)      # more than 8 bits
    with pytest.raises(ValueError):
        po.alloc_exact(F, 199)                             # below 2 bits per super-group
    with pytest.raises(ValueError):
        po.alloc_exact(np.ones(4097, np.float32), 8 * 4097)
    # the allocation mode runs the whole round: widths as the programme gives
    # them, no scalar (NaN), and the round is exact on constant super-groups
    J, n = 32, 4
    gs = [(np.repeat(10.0 ** rng.uniform(-4, 0, J), 256) * rng.standard_normal(256 * J)).astype(np.float32)
          for _ in range(n)]
    o = po.Oracle(256 * J, n, po.RING, 5.0, alloc=po.ALLOC_EXACT)
    out = o.allreduce(gs)
    _, F, _ = o.stats_arrays()
    assert np.array_equal(o.widths(), po.alloc_exact(F, o.budget_bits())[0])
    assert np.isnan(o.rho())
    exact = np.sum([g.astype(np.float64) for g in gs], axis=0)
    assert np.sum((out - exact) ** 2) / np.sum(exact ** 2) < 1e-2


# ---------------------------------------------------------------------------
# the 16-bit class (pith.science review, Fig. 3 caption: the threshold chain
# continues to T48 = 257/2^17 T816; "What carries the argument": the per-bit
# benefit of the 4^-b model); off by default, where the widths are {2,4,8}
# ---------------------------------------------------------------------------

def test_wide_threshold_chain_is_exact():
    """The four multipliers of the 16-bit chain (the 85 : 544 : 16384 chain
    scaled by 257, then 2^31) carry the pages' ratios exactly, the last one
    equalising the 8 -> 16 per-bit benefit 65535 / 2^35 with the 4 -> 8 one;
    and fp32 thresholds at powers of two keep them exactly."""
    g = gold("pages_constants.json")
    K = [Fraction(21845), Fraction(139808), Fraction(4210688), Fraction(2 ** 31)]
    assert K[0] / K[1] == frac(g["ratio_T12_over_T24"]["value"])
    assert K[1] / K[2] == frac(g["ratio_T24_over_T48"]["value"])
    assert K[2] / K[3] == frac(g["ratio_T48_over_T816"]["value"])
    b816 = (Fraction(1, 4 ** 8) - Fraction(1, 4 ** 16)) / 8
    assert b816 == Fraction(65535, 2 ** 35)
    assert b816 / frac(g["per_bit_benefit_4_to_8"]["value"]) == frac(g["ratio_T48_over_T816"]["value"])
    for rho in (1.0, 2.0 ** -30, 2.0 ** 5):
        t = [Fraction(float(x)) for x in po.thresholds_wide(f32_bits(rho))]
        assert t[1] / t[2] == frac(g["ratio_T24_over_T48"]["value"])
        assert t[2] / t[3] == frac(g["ratio_T48_over_T816"]["value"])


def _alloc_wide(F, budget):
    J = len(F)
    o = po.Oracle(256 * J, 1, po.RING, budget, max_width=16)
    g = np.zeros(256 * J, np.float32)
    g[::256] = np.sqrt(F).astype(np.float32)
    o.stats(0, g)
    o.allocate()
    _, Fo, _ = o.stats_arrays()
    return o, Fo


def test_wide_allocation_brute_force_8_super_groups():
    """Against all 4^8 assignments of {2,4,8,16}: Lagrangian optimality,
    threshold consistency at rho (the chain 544 : 16384 : 16384 * 2^17 / 257
    in exact rationals), minimal rho, budget kept; and the exact programme
    over the four widths returns the brute-force optimum."""
    rng = np.random.default_rng(71)
    assigns = np.array(list(itertools.product((2, 4, 8, 16), repeat=8)), dtype=np.int64)
    bits = assigns.sum(1)
    pw = 4.0 ** (-assigns.astype(np.float64))
    for trial in range(120):
        F = np.exp(rng.uniform(-40, 5, 8)) if trial % 2 else rng.lognormal(0, 6, 8)
        budget = float(rng.choice([2.0, 3.0, 4.5, 6.0, 8.0, 9.5, 11.0, 13.0, 15.9, 16.0, 20.0]))
        o, Fo = _alloc_wide(F, budget)
        F64 = Fo.astype(np.float64)
        q = o.widths().astype(np.int64)
        total = int(q.sum())
        assert set(np.unique(q)) <= {2, 4, 8, 16}
        assert total <= min(budget, 16.0) * 8 + 1e-9
        rb = o.rho_bits()
        assert o.count_bits(rb) == total
        if rb > 0:
            assert o.count_bits(rb - 1) > o.budget_bits()
        err = pw @ F64
        mine = float((F64 * 4.0 ** (-q.astype(np.float64))).sum())
        assert mine <= err[bits <= total].min() * (1 + 1e-9)
        rho = Fraction(float(f32_from_bits(rb)))
        T816 = rho * 2 ** 31
        T48 = T816 * Fraction(257, 2 ** 17)
        T24 = T48 * Fraction(17, 512)
        for Fj, qj in zip(F64, q):
            Fr = Fraction(float(Fj))
            exp_q = 16 if Fr >= T816 else (8 if Fr >= T48 else (4 if Fr >= T24 else 2))
            if exp_q != qj:
                # only a tie inside one fp32 rounding of T48 or T24 may differ
                assert min(abs(Fr - T48) / T48, abs(Fr - T24) / T24) <= Fraction(1, 2 ** 23)
        # the exact programme over the four widths
        w, cost = po.alloc_exact(Fo, o.budget_bits(), qmax=16)
        best = err[bits <= o.budget_bits()].min()
        assert abs(cost - best) <= 1e-12 * best and int(w.astype(np.int64).sum()) <= o.budget_bits()


def test_wide_allocation_special_budgets():
    rng = np.random.default_rng(72)
    F = rng.lognormal(0, 3, 64)
    o, _ = _alloc_wide(F, 16.0)
    assert (o.widths() == 16).all() and o.rho_bits() == 0
    o, _ = _alloc_wide(F, 1e9)
    assert (o.widths() == 16).all()
    o, _ = _alloc_wide(F, 2.0)
    assert (o.widths() == 2).all()
    o8, _ = _alloc(F, 8.0)
    assert (o8.widths() == 8).all()          # the default width set caps at 8
    with pytest.raises(ValueError):
        po.Oracle(256, 1, po.RING, 5.0, max_width=12)


@pytest.mark.parametrize("max_width", [8, 16])
def test_overflowed_squared_norms_keep_the_width_set(max_width):
    """A finite gradient can still overflow its squared norm (|e| above about
    1.8e19 gives fl(e^2) = +inf; the statistics flag such a round).  A key of
    +inf meets every finite threshold and takes the widest width of the
    plan's set: 8 without the 16-bit class (the width set {2,4,8} of the
    threshold chain, Fig. 3 caption), never a width outside it.  A NaN key
    meets no threshold and takes 2.  Every super-group lands in a class."""
    J = 40
    rng = np.random.default_rng(31)
    g = rng.standard_normal(256 * J).astype(np.float32)
    g[5 * 256 + 7] = 1e20
    g[9 * 256] = 3e19
    g[12 * 256 + 3] = np.nan
    o = po.Oracle(256 * J, 1, po.RING, 5.0, max_width=max_width)
    o.stats(0, g)
    o.allocate()
    _, F, _ = o.stats_arrays()
    assert np.isposinf(F[[5, 9]]).all() and np.isnan(F[12])
    q = o.widths().astype(int)
    assert q[5] == q[9] == max_width and q[12] == 2
    assert set(np.unique(q).tolist()) <= ({2, 4, 8, 16} if max_width == 16 else {2, 4, 8})
    assert int(o.class_counts().sum()) == J
    assert q.sum() <= o.budget_bits()


@pytest.mark.parametrize("max_width", [8, 16])
def test_budget_out_of_reach_with_infinite_norms_gives_rho_inf(max_width):
    """When even rho = +inf misses the budget (keys of +inf keep the widest
    width at every rho), rho is the end of the search range, +inf: finite
    keys take 2 bits and the infinite ones the widest width of the set."""
    J = 16
    g = np.ones(256 * J, np.float32)
    g[0:12 * 256:256] = 1e20          # 12 of 16 super-groups overflow
    o = po.Oracle(256 * J, 1, po.RING, 3.0, max_width=max_width)
    o.stats(0, g)
    o.allocate()
    assert o.rho_bits() == 0x7F800000
    q = o.widths()
    assert (q[:12] == max_width).all() and (q[12:] == 2).all()
    assert int(o.class_counts().sum()) == J


def test_level_table_16_bits():
    L, W = po.levels(16)
    assert L.size == 65536 and L[0] == -1.0 and L[-1] == 1.0
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    assert np.array_equal(L[::-1], -L)
    # the widest interval is at the ends, the narrowest at zero (denser near 0)
    gaps = np.diff(L.astype(np.float64))
    assert gaps[32767] < gaps[0] and gaps[0] / gaps[32767] > 2.5
    # the same closed form as the narrower classes at their shared levels:
    # u = (2r + 1 - Q) / (Q - 1), L = u (1 + |u|) / 2 for eps = 1/2
    r = np.array([0, 1, 100, 32767, 32768, 65534, 65535])
    u = (2.0 * r + 1 - 65536) / 65535
    assert np.array_equal(L[r], (u * (0.5 + 0.5 * np.abs(u))).astype(np.float32))


def test_codec_16_bits_unbiased_and_bounded():
    """Monte Carlo over 10^4 dithers (D23 gate) and the deterministic bound
    |x_hat - y| <= sigma (L[r+1] - L[r]) at 65,536 levels."""
    rng = np.random.default_rng(73)
    K = 10000
    y = (rng.standard_normal(256) * np.repeat(10.0 ** rng.uniform(-3, 0, 16), 16)).astype(np.float32)
    Y = np.tile(y, (K, 1))
    D = rng.integers(0, 65536, size=(K, 256), dtype=np.uint16)
    dec = po.roundtrip_batch(Y, 16, D).astype(np.float64)
    sd = dec.std(0, ddof=1)
    ok = sd > 0
    _d23_gate((dec.mean(0)[ok] - y[ok]) / (sd[ok] / np.sqrt(K)))
    L, _ = po.levels(16)
    for t in range(20):
        x, codes, s, cg = po.roundtrip_sg(y, 16, D[t])
        sigma = (cg.astype(np.float32).repeat(16) * np.float32(s)).astype(np.float64)
        r = np.clip(codes.astype(np.int64), 1, 65534)
        width = sigma * np.maximum(L[r].astype(np.float64) - L[r - 1], L[r + 1].astype(np.float64) - L[r])
        assert np.all(np.abs(x - y) <= width * (1 + 1e-6) + 1e-30)
        assert codes.max() <= 65535


def test_wide_round_budget_exactness_and_gain():
    """Whole rounds with the 16-bit class: the budget holds, constant and
    zero super-groups are exact, and at 10 bits per coordinate the error is
    below the {2,4,8} round at its 8-bit cap."""
    rng = np.random.default_rng(74)
    n, J = 4, 48
    gs = _grads(rng, n, J, 3)
    for g in gs:
        g[0:256] = 0.0
        g[512:768] = 0.25
    exact = np.sum([g.astype(np.float64) for g in gs], 0)
    for topo in (po.RING, po.BUTTERFLY):
        o = po.Oracle(256 * J, n, topo, 10.0, max_width=16)
        out = o.allreduce(gs)
        q = o.widths().astype(np.int64)
        assert q.sum() <= 10 * J and (q == 16).any()
        assert np.all(out[0:256] == 0.0) and np.all(out[512:768] == np.float32(n * 0.25))
        v16 = np.sum((out - exact) ** 2) / np.sum(exact ** 2)
        o8 = po.Oracle(256 * J, n, topo, 8.0)
        v8 = np.sum((o8.allreduce(gs) - exact) ** 2) / np.sum(exact ** 2)
        assert v16 < v8
