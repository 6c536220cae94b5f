"""Checks of the oracle's MX all-reduce schedule (test infrastructure).

Two independent statements of what the ring and butterfly schedules compute,
used by tests/test_oracle_pins.py directly and, in a child process, against
copies of the oracle with a planted mistake:

* exact sums: every coordinate has one owning worker whose value is a power
  of two inside the element format's exact range relative to any block
  maximum, and every other worker holds 0 there, so every partial sum the
  schedule forms is exactly representable after each block quantisation and
  the all-reduce must return the exact sum; a worker added twice, missed, or
  read from the wrong buffer changes it;
* composition: the reduced value of each part written part by part (ring:
  the part's chain starts at the worker that owns it and visits the others
  in rank order; butterfly: the value a worker holds after level s is the
  quantised sum of its own and its partner's values after level s - 1 on
  the worker's new part), built from single block quantisations only.
"""
import numpy as np

from oracle import pyoracle as po

# exponent span of exactly representable powers of two below a block maximum:
# emax of the element format plus the depth of its smallest subnormal
MX_SPAN = {po.MX_E4M3: 8 + 9, po.MX_E3M2: 4 + 4, po.MX_E2M3: 2 + 3, po.MX_E2M1: 2 + 1}


def exact_sum_inputs(fmt, n, J, seed):
    rng = np.random.default_rng(seed)
    d = 256 * J
    i = np.arange(d)
    owner = (i + 7 * (i // 32) + (i // 256)) % n
    top = np.repeat(rng.integers(-30, 12, d // 32), 32)             # block exponent E
    a = top - rng.integers(0, MX_SPAN[fmt] + 1, d)                    # in [E - span, E]
    v = (np.where(rng.random(d) < 0.5, -1.0, 1.0) * np.ldexp(1.0, a)).astype(np.float32)
    g = [np.where(owner == w, v, np.float32(0)).astype(np.float32) for w in range(n)]
    return g, v


def _part(J, m, c):
    return 256 * (c * J // m), 256 * ((c + 1) * J // m)


def ring_composition(fmt, g, n, J):
    q = lambda x: po.mx_roundtrip(fmt, x)
    out = np.zeros(256 * J, np.float32)
    for p in range(n):
        lo, hi = _part(J, n, p)
        acc = q(g[p][lo:hi])
        for k in range(1, n):
            acc = q((acc + g[(p + k) % n][lo:hi]).astype(np.float32))
        out[lo:hi] = acc
    return out


def butterfly_composition(fmt, g, n, J):
    q = lambda x: po.mx_roundtrip(fmt, x)
    L = n.bit_length() - 1
    V = {}
    for w in range(n):
        lo, hi = _part(J, 2, w >> (L - 1))
        sent = q(g[w ^ (n >> 1)][lo:hi])
        V[w] = (lo, q((sent + g[w][lo:hi]).astype(np.float32)))
    for s in range(2, L + 1):
        nv = {}
        for w in range(n):
            lo, hi = _part(J, 1 << s, w >> (L - s))
            (plo, pv), (olo, ov) = V[w ^ (n >> s)], V[w]
            nv[w] = (lo, q((pv[lo - plo:hi - plo] + ov[lo - olo:hi - olo]).astype(np.float32)))
        V = nv
    out = np.zeros(256 * J, np.float32)
    for w in range(n):
        lo, x = V[w]
        out[lo:lo + x.size] = x
    return out


CASES = [(po.RING, 3), (po.RING, 4), (po.RING, 5), (po.BUTTERFLY, 4), (po.BUTTERFLY, 8)]


def run_checks(J=40):
    """{(topology, n, fmt, check): passed} over CASES and the four formats."""
    res = {}
    for topo, n in CASES:
        for fmt in (po.MX_E4M3, po.MX_E3M2, po.MX_E2M3, po.MX_E2M1):
            g, v = exact_sum_inputs(fmt, n, J, seed=100 * n + 10 * topo + fmt)
            out = po.Oracle(256 * J, n, topo).mx_allreduce(fmt, g)
            res[(topo, n, fmt, "exact")] = bool(np.array_equal(out.view(np.uint32), v.view(np.uint32)))
            rng = np.random.default_rng(7 + n + 10 * topo + 100 * fmt)
            gr = [(rng.standard_normal(256 * J) * np.repeat(10.0 ** rng.uniform(-5, 1, 8 * J), 32)).astype(np.float32)
                  for _ in range(n)]
            out = po.Oracle(256 * J, n, topo).mx_allreduce(fmt, gr)
            ref = (ring_composition if topo == po.RING else butterfly_composition)(fmt, gr, n, J)
            res[(topo, n, fmt, "composition")] = bool(np.array_equal(out.view(np.uint32), ref.view(np.uint32)))
    return res


if __name__ == "__main__":
    import json
    r = run_checks()
    print(json.dumps({"passed": sum(r.values()), "total": len(r),
                      "failed": [list(k) for k, ok in r.items() if not ok]}))
