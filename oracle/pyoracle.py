"""ctypes wrapper around ``liboracle.so`` -- TEST INFRASTRUCTURE ONLY.

Marshals numpy arrays into the plain C oracle (``oracle.c``).  Nothing here
computes any part of the method.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

RING, BUTTERFLY = 0, 1
BF16, F32, PACKED, PARTIAL = 0, 1, 2, 3
CORRELATED, INDEPENDENT, STRATIFIED = 0, 1, 2
ALLOC_THRESHOLD, ALLOC_MEAN_CORRECTED, ALLOC_UNIFORM, ALLOC_EXACT = 0, 1, 2, 3
OWN_PACKED, OWN_F32 = 0, 1
Q_OF_CLASS = (2, 4, 8)

_lib = None


def lib():
    global _lib
    if _lib is None:
        # DQ_ORACLE_LIB: another build of oracle.c (the mutation tests load
        # copies with a planted mistake in a separate process)
        path = os.environ.get("DQ_ORACLE_LIB") or _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        vp, i32, i64, u32, u64, f32, f64 = (C.c_void_p, C.c_int32, C.c_int64, C.c_uint32,
                                            C.c_uint64, C.c_float, C.c_double)
        sig = {
            "or_set_threads": (None, [C.c_int]),
            "or_get_threads": (C.c_int, []),
            "or_philox4x32": (None, [vp, vp, C.c_int, vp]),
            "or_levels": (None, [C.c_int, f64, vp, vp]),
            "or_create": (vp, [i64, i32, i32, f32]),
            "or_destroy": (None, [vp]),
            "or_set_seed": (None, [vp, u64]),
            "or_set_round": (None, [vp, u32]),
            "or_set_rounding": (None, [vp, i32]),
            "or_set_alloc": (None, [vp, i32]),
            "or_set_own": (None, [vp, i32]),
            "or_get_alloc_key": (None, [vp, vp]),
            "or_set_eps": (None, [vp, f64]),
            "or_stats": (C.c_int, [vp, i32, vp, i32]),
            "or_allocate": (C.c_int, [vp]),
            "or_reorder": (C.c_int, [vp]),
            "or_get_stats": (None, [vp, vp, vp, vp]),
            "or_get_rho_bits": (u32, [vp]),
            "or_get_widths": (None, [vp, vp]),
            "or_get_perm": (None, [vp, vp, vp]),
            "or_get_class_counts": (None, [vp, vp]),
            "or_budget_bits": (i64, [vp]),
            "or_count_bits": (i64, [vp, u32]),
            "or_thresholds": (None, [u32, vp]),
            "or_alloc_exact": (f64, [vp, i64, i64, vp]),
            "or_alloc_exact_q": (f64, [vp, i64, i64, i32, vp]),
            "or_set_max_width": (C.c_int, [vp, i32]),
            "or_get_class_counts4": (None, [vp, vp]),
            "or_thresholds_wide": (None, [u32, vp]),
            "or_region_bytes": (i64, [vp, i64, i64, vp]),
            "or_compress": (C.c_int, [vp, i32, i32, vp, i32, vp, vp, i64]),
            "or_hop": (C.c_int, [vp, i32, i32, vp, vp, i32, vp, vp, vp, i64]),
            "or_finalize": (C.c_int, [vp, i64, vp, vp, vp, i64]),
            "or_final_part": (i64, [vp, i32]),
            "or_allreduce": (C.c_int, [vp, vp, i32, vp]),
            "or_roundtrip_sg": (None, [vp, i32, vp, f64, vp, vp, vp, vp]),
            "or_roundtrip_batch": (None, [vp, i64, i32, vp, f64, vp]),
            "or_dithers": (None, [u64, u32, i64, i32, i32, i32, i32, vp]),
            "or_dithers_tagged": (None, [u64, u32, i64, u32, u32, vp]),
            "or_mxfp8_roundtrip": (None, [vp, i64, vp]),
            "or_mx_roundtrip": (None, [i32, vp, i64, vp]),
            "or_mx_allreduce": (C.c_int, [vp, i32, vp, i32, vp]),
            "or_mxfp8_allreduce": (C.c_int, [vp, vp, i32, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def set_threads(n):
    lib().or_set_threads(int(n))


def get_threads():
    return lib().or_get_threads()


def philox4x32(ctr, key, rounds=10):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().or_philox4x32(_p(c), _p(k), int(rounds), _p(out))
    return out


def levels(q, eps=0.5):
    L = np.zeros(max(256, 1 << q), np.float32)
    W = np.zeros(max(256, 1 << q), np.float32)
    lib().or_levels(int(q), float(eps), _p(L), _p(W))
    Q = 1 << q
    return L[:Q].copy(), W[:Q - 1].copy()


def alloc_exact(F, budget_bits, qmax=8):
    """(widths, cost): the widths in {2,4,8} (or {2,4,8,16} for qmax 16)
    minimising sum F 4^-q under sum q <= budget_bits, and that minimum."""
    F = np.ascontiguousarray(F, dtype=np.float32)
    w = np.zeros(F.size, np.uint8)
    cost = lib().or_alloc_exact_q(_p(F), F.size, int(budget_bits), int(qmax), _p(w))
    if cost < 0:
        raise ValueError("or_alloc_exact: J out of range or budget below 2 bits")
    return w, cost


def thresholds_wide(rho_bits):
    out = np.zeros(4, np.float32)
    lib().or_thresholds_wide(int(rho_bits), _p(out))
    return out


def thresholds(rho_bits):
    out = np.zeros(3, np.float32)
    lib().or_thresholds(int(rho_bits), _p(out))
    return out


def dithers(seed, rnd, j, mode, worker, n, event):
    d = np.zeros(256, np.uint16)
    lib().or_dithers(int(seed), int(rnd), int(j), int(mode), int(worker), int(n), int(event), _p(d))
    return d


def dithers_tagged(seed, rnd, j, tag, stagger):
    d = np.zeros(256, np.uint16)
    lib().or_dithers_tagged(int(seed), int(rnd), int(j), int(tag), int(stagger), _p(d))
    return d


def roundtrip_sg(y, q, dither, eps=0.5):
    y = np.ascontiguousarray(y, dtype=np.float32)
    d = np.ascontiguousarray(dither, dtype=np.uint16)
    dec = np.zeros(256, np.float32)
    codes = np.zeros(256, np.uint16)
    s = np.zeros(1, np.float32)
    cg = np.zeros(16, np.uint8)
    lib().or_roundtrip_sg(_p(y), int(q), _p(d), float(eps), _p(dec), _p(codes), _p(s), _p(cg))
    return dec, codes, float(s[0]), cg


def roundtrip_batch(y, q, dither, eps=0.5):
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1, 256)
    d = np.ascontiguousarray(dither, dtype=np.uint16).reshape(-1, 256)
    assert y.shape == d.shape
    out = np.zeros_like(y)
    lib().or_roundtrip_batch(_p(y), y.shape[0], int(q), _p(d), float(eps), _p(out))
    return out


MX_E4M3, MX_E3M2, MX_E2M3, MX_E2M1 = 0, 1, 2, 3


def mxfp8_roundtrip(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros_like(x)
    lib().or_mxfp8_roundtrip(_p(x), x.size, _p(out))
    return out


def mx_roundtrip(fmt, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros_like(x)
    lib().or_mx_roundtrip(int(fmt), _p(x), x.size, _p(out))
    return out


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bits
        return BF16
    raise TypeError("gradients must be float32 or uint16 (bf16 bits)")


class Oracle:
    """One simulated round on the CPU (mirrors the stage order of the library)."""

    def __init__(self, n_coords, n_workers, topology=RING, avg_bits=5.0, seed=1, rnd=0,
                 rounding=STRATIFIED, eps=None, alloc=ALLOC_THRESHOLD, own=OWN_PACKED, max_width=8):
        self.d = int(n_coords)
        self.n = int(n_workers)
        self.topology = int(topology)
        self.J = self.d // 256
        self.h = lib().or_create(self.d, self.n, self.topology, float(avg_bits))
        if not self.h:
            raise ValueError("invalid oracle arguments")
        lib().or_set_seed(self.h, int(seed))
        lib().or_set_round(self.h, int(rnd))
        lib().or_set_rounding(self.h, int(rounding))
        if eps is not None:
            lib().or_set_eps(self.h, float(eps))
        lib().or_set_alloc(self.h, int(alloc))
        lib().or_set_own(self.h, int(own))
        if max_width != 8 and lib().or_set_max_width(self.h, int(max_width)) != 0:
            raise ValueError("max_width must be 8 or 16")
        self.max_width = int(max_width)
        self.log2n = max(0, (self.n - 1).bit_length())

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            try:
                _lib.or_destroy(h)
            except Exception:
                pass
            self.h = None

    # stages
    def stats(self, w, g):
        _check(lib().or_stats(self.h, int(w), _p(g), _dtype_code(g)), "stats")

    def allocate(self):
        _check(lib().or_allocate(self.h), "allocate")

    def reorder(self):
        _check(lib().or_reorder(self.h), "reorder")

    def stats_arrays(self):
        s = np.zeros(self.J, np.float32)
        F = np.zeros(self.J, np.float32)
        mu = np.zeros(self.J, np.float32)
        lib().or_get_stats(self.h, _p(s), _p(F), _p(mu))
        return s, F, mu

    def rho_bits(self):
        return int(lib().or_get_rho_bits(self.h))

    def rho(self):
        return np.array([self.rho_bits()], np.uint32).view(np.float32)[0]

    def alloc_key(self):
        k = np.zeros(self.J, np.float32)
        lib().or_get_alloc_key(self.h, _p(k))
        return k

    def widths(self):
        w = np.zeros(self.J, np.uint8)
        lib().or_get_widths(self.h, _p(w))
        return w

    def perm(self):
        p = np.zeros(self.J, np.int32)
        i = np.zeros(self.J, np.int32)
        lib().or_get_perm(self.h, _p(p), _p(i))
        return p, i

    def class_counts(self):
        """Super-groups per class: (2, 4, 8), or (2, 4, 8, 16) with the 16-bit class."""
        c = np.zeros(4, np.int64)
        lib().or_get_class_counts4(self.h, _p(c))
        return c[:4 if self.max_width == 16 else 3]

    def budget_bits(self):
        return int(lib().or_budget_bits(self.h))

    def count_bits(self, rho_bits):
        return int(lib().or_count_bits(self.h, int(rho_bits)))

    def region_bytes(self, m, part):
        cnt = np.zeros(4, np.int64)
        b = lib().or_region_bytes(self.h, int(m), int(part), _p(cnt))
        return int(b), cnt[:4 if self.max_width == 16 else 3]

    def worst_region_bytes(self):
        return (self.J + 3) * (32 * self.max_width + 20) + 64

    def compress(self, w, step, g, region, filt=None):
        f = None if filt is None else np.ascontiguousarray(filt, np.int64)
        _check(lib().or_compress(self.h, int(w), int(step), _p(g), _dtype_code(g), _p(region),
                                 _p(f), 0 if f is None else f.size), "compress")

    def hop(self, w, step, region_in, local, out0, out1=None, filt=None, partial=False):
        """partial=True: `local` is the worker's fp32 partial sums (own-fp32 variant)."""
        kind = PARTIAL if partial else (PACKED if local.dtype == np.uint8 else _dtype_code(local))
        f = None if filt is None else np.ascontiguousarray(filt, np.int64)
        _check(lib().or_hop(self.h, int(w), int(step), _p(region_in), _p(local), kind, _p(out0),
                            _p(out1), _p(f), 0 if f is None else f.size), "hop")

    def finalize(self, part, region, out, filt=None):
        f = None if filt is None else np.ascontiguousarray(filt, np.int64)
        _check(lib().or_finalize(self.h, int(part), _p(region), _p(out), _p(f),
                                 0 if f is None else f.size), "finalize")

    def final_part(self, w):
        return int(lib().or_final_part(self.h, int(w)))

    def mxfp8_allreduce(self, grads):
        grads = [np.ascontiguousarray(g) for g in grads]
        ptrs = (C.c_void_p * self.n)(*[g.ctypes.data for g in grads])
        out = np.zeros(self.d, np.float32)
        _check(lib().or_mxfp8_allreduce(self.h, ptrs, _dtype_code(grads[0]), _p(out)), "mxfp8_allreduce")
        return out

    def mx_allreduce(self, fmt, grads):
        grads = [np.ascontiguousarray(g) for g in grads]
        ptrs = (C.c_void_p * self.n)(*[g.ctypes.data for g in grads])
        out = np.zeros(self.d, np.float32)
        _check(lib().or_mx_allreduce(self.h, int(fmt), ptrs, _dtype_code(grads[0]), _p(out)), "mx_allreduce")
        return out

    def allreduce(self, grads):
        grads = [np.ascontiguousarray(g) for g in grads]
        assert len(grads) == self.n
        ptrs = (C.c_void_p * self.n)(*[g.ctypes.data for g in grads])
        out = np.zeros(self.d, np.float32)
        _check(lib().or_allreduce(self.h, ptrs, _dtype_code(grads[0]), _p(out)), "allreduce")
        return out
