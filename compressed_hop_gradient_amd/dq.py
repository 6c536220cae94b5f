"""Python binding of the C ABI in ``include/dq.h``.

Argument marshalling only: every stage runs in the HIP kernels of
``libdq.so``.  PyTorch supplies device memory (tensors) and the stream
(``torch.cuda.current_stream()``).  If the shared library is missing the
import of this module's functions raises; there is no CPU fallback.
"""
import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdq.so")

DQ_OK, DQ_EINVAL, DQ_EBUDGET, DQ_ESTATE, DQ_EWORKSPACE, DQ_ENULL, DQ_EHIP, DQ_ENONFINITE = \
    0, -1, -2, -3, -4, -5, -6, -7
RING, BUTTERFLY = 0, 1
BF16, F32, PACKED, F32_PARTIAL = 0, 1, 2, 3
OWN_PACKED, OWN_F32 = 0, 1
CORRELATED, INDEPENDENT, STRATIFIED = 0, 1, 2
OPT_SEED, OPT_ROUND, OPT_ROUNDING, OPT_TIMING, OPT_ALLOC, OPT_TIMING_KINDS, OPT_OWN = 0, 1, 2, 3, 4, 5, 6
OPT_STREAMS = 7
OPT_MAX_WIDTH = 8
ALLOC_THRESHOLD, ALLOC_MEAN_CORRECTED, ALLOC_UNIFORM = 0, 1, 2
MX_FP8_E4M3, MX_FP6_E3M2, MX_FP6_E2M3, MX_FP4_E2M1 = 0, 1, 2, 3
OPT_EPS = 0   # dq_option_f64
KERNEL_KINDS = ("stats", "allocate", "reorder", "compress", "hop_grad", "hop_packed",
                "finalize", "mxfp8", "hop_final")


class dq_info(C.Structure):
    _fields_ = [("rho_bits", C.c_uint32), ("rho", C.c_float), ("t12", C.c_float),
                ("t24", C.c_float), ("t48", C.c_float), ("class_counts", C.c_int64 * 3),
                ("budget_bits", C.c_int64), ("used_bits", C.c_int64),
                ("achieved_bits", C.c_double), ("nonfinite", C.c_int32), ("t816", C.c_float),
                ("class_count16", C.c_int64)]


class dq_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("sum", "sumsq", "widths", "perm", "inv", "mu_stream",
                                          "tables", "ctrl", "total", "tables16")]


class dq_timing(C.Structure):
    _fields_ = [("ms", C.c_double * len(KERNEL_KINDS)), ("launches", C.c_int64 * len(KERNEL_KINDS)),
                ("coords", C.c_int64 * len(KERNEL_KINDS))]


class DQError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None

# exported symbols and their signatures (every declaration of include/dq.h)
_SIGS = {
    "dq_plan_create": (C.c_int, [C.c_int64, C.c_int32, C.c_int32, C.c_float, C.POINTER(C.c_void_p)]),
    "dq_plan_destroy": (None, [C.c_void_p]),
    "dq_plan_set_u64": (C.c_int, [C.c_void_p, C.c_int32, C.c_uint64]),
    "dq_workspace_bytes": (C.c_size_t, [C.c_void_p]),
    "dq_plan_bind": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
    "dq_workspace_layout": (C.c_int, [C.c_void_p, C.POINTER(dq_layout)]),
    "dq_region_bytes_max": (C.c_size_t, [C.c_void_p, C.c_int64]),
    "dq_stats": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]),
    "dq_allocate": (C.c_int, [C.c_void_p, C.c_void_p]),
    "dq_reorder": (C.c_int, [C.c_void_p, C.c_void_p]),
    "dq_compress": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                              C.c_void_p]),
    "dq_hop": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                         C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_finalize": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_final_part": (C.c_int64, [C.c_void_p, C.c_int32]),
    "dq_arena_bytes": (C.c_size_t, [C.c_void_p]),
    "dq_allreduce": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                               C.c_void_p, C.c_void_p]),
    "dq_noalloc_max_bytes": (C.c_size_t, []),
    "dq_allreduce_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "dq_mxfp8_arena_bytes": (C.c_size_t, [C.c_void_p]),
    "dq_mxfp8_allreduce": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                     C.c_void_p, C.c_void_p]),
    "dq_mx_arena_bytes": (C.c_size_t, [C.c_void_p]),
    "dq_hop_finalize": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_partial_bytes_max": (C.c_size_t, [C.c_void_p, C.c_int64]),
    "dq_plan_set_f64": (C.c_int, [C.c_void_p, C.c_int32, C.c_double]),
    "dq_mx_allreduce": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                  C.c_void_p, C.c_void_p]),
    "dq_check_reciprocal": (C.c_int, [C.c_uint32, C.c_uint32, C.c_void_p, C.c_void_p]),
    "dq_check_round_half_up": (C.c_int, [C.c_uint32, C.c_uint32, C.c_void_p, C.c_void_p]),
    "dq_probe_stream": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_size_t, C.c_int32,
                                  C.c_void_p]),
    "dq_get_info": (C.c_int, [C.c_void_p, C.POINTER(dq_info), C.c_void_p]),
    "dq_timing_read": (C.c_int, [C.c_void_p, C.POINTER(dq_timing)]),
    "dq_status_string": (C.c_char_p, [C.c_int32]),
    "dq_version": (C.c_int32, []),
}


def lib():
    """Load ``libdq.so`` (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(s):
    return lib().dq_status_string(int(s)).decode()


def _check(rc, what):
    if rc != DQ_OK:
        raise DQError(rc, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def _kind(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.uint8:
        return PACKED
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _tensor(t, what, device, numel=None, min_bytes=None, dtype=None):
    """Reject what the kernels cannot address safely: tensors on the host or on
    another device, non-contiguous views and buffers shorter than the call
    writes or reads (the C ABI takes bare pointers and cannot check sizes)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{what}: tensor on {t.device}, the plan works on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what}: {t.numel()} elements, expected {numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, the call needs {min_bytes}")
    return t


def check_reciprocal(lo_bits, count, device=None, stream=None):
    """Mismatches between the codec's reciprocal and the IEEE quotient 1/x over
    the fp32 bit patterns [lo_bits, lo_bits + count) (runs on the GPU)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    _check(lib().dq_check_reciprocal(int(lo_bits), int(count), _ptr(cnt), _stream(stream)),
           "dq_check_reciprocal")
    return int(cnt.item())


def check_round_half_up(lo_bits, count, device=None, stream=None):
    """Mismatches between the codec's round-half-up conversion and the exact
    floor(x + 0.5) (NaN saturated by its sign) over the fp32 bit patterns
    [lo_bits, lo_bits + count)
    (runs on the GPU)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    _check(lib().dq_check_round_half_up(int(lo_bits), int(count), _ptr(cnt), _stream(stream)),
           "dq_check_round_half_up")
    return int(cnt.item())


def probe_stream(src, dst, reads_per_write, stream=None):
    """Run the streaming probe over the bytes of ``src`` (device tensor) with
    the given read:write mix, writing into ``dst``."""
    dev = src.device
    _tensor(src, "src", dev)
    _tensor(dst, "dst", dev)
    _check(lib().dq_probe_stream(_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                 dst.numel() * dst.element_size(), int(reads_per_write),
                                 _stream(stream)), "dq_probe_stream")


class Plan:
    """One gradient-synchronisation round over ``n_workers`` virtual workers.

    Mirrors ``include/dq.h``: create -> options -> bind workspace -> stats (rank
    order) -> allocate -> reorder -> compress / hop -> finalize.
    """

    def __init__(self, n_coords, n_workers, topology=RING, avg_bits=5.0, seed=1, rnd=0,
                 rounding=STRATIFIED, device="cuda", timing=False, alloc=ALLOC_THRESHOLD, eps=None,
                 own=OWN_PACKED, streams=1, max_width=8):
        self.d = int(n_coords)
        self.n = int(n_workers)
        self.J = self.d // 256
        self.topology = int(topology)
        self.log2n = max(0, (self.n - 1).bit_length())
        self.own = int(own)
        if torch.device(device).type != "cuda":
            raise ValueError(f"the plan's workspace must be GPU memory, not {device}")
        h = C.c_void_p()
        _check(lib().dq_plan_create(self.d, self.n, self.topology, float(avg_bits), C.byref(h)),
               "dq_plan_create")
        self.h = h
        self.set(OPT_SEED, seed)
        self.set(OPT_ROUND, rnd)
        self.set(OPT_ROUNDING, rounding)
        self.set(OPT_TIMING, 1 if timing else 0)
        self.set(OPT_ALLOC, alloc)
        self.set(OPT_OWN, own)
        self.max_width = int(max_width)
        if self.max_width != 8:
            self.set(OPT_MAX_WIDTH, self.max_width)
        if eps is not None:
            _check(lib().dq_plan_set_f64(self.h, OPT_EPS, float(eps)), "dq_plan_set_f64")
        if streams != 1:
            with torch.cuda.device(torch.device(device)):   # the second stream lives on this device
                self.set(OPT_STREAMS, streams)
        nbytes = lib().dq_workspace_bytes(self.h)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        _check(lib().dq_plan_bind(self.h, _ptr(self.workspace), nbytes), "dq_plan_bind")
        lay = dq_layout()
        _check(lib().dq_workspace_layout(self.h, C.byref(lay)), "dq_workspace_layout")
        self.layout = {n: getattr(lay, n) for n, _ in dq_layout._fields_}

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and h.value and _lib is not None:
            _lib.dq_plan_destroy(h)
            self.h = None

    def set(self, option, value):
        _check(lib().dq_plan_set_u64(self.h, int(option), int(value)), "dq_plan_set_u64")

    # ---- buffer sizes the schedule implies (for the argument checks) ---------
    def _m_compress(self):
        """m of the part a compress writes: the whole vector for one worker,
        a ring part (m = n), or a butterfly level-1 half (m = 2)."""
        return 1 if self.n == 1 else (self.n if self.topology == RING else 2)

    def _m_hop(self, step):
        """(m of the part a hop reads, m of each region it writes), or None
        for a step outside the schedule (the library rejects those)."""
        if self.n == 1:
            return None
        if self.topology == RING:
            return (self.n, self.n) if 1 <= step < self.n else None
        if not 1 <= step <= self.log2n:
            return None
        m = 1 << step
        return (m, 2 * m if step < self.log2n else m)

    def _check_hop(self, worker, step, region_in, local, kind, outs):
        ms = self._m_hop(int(step))
        dev = self.device
        _tensor(region_in, "region_in", dev)
        _tensor(local, "local", dev)
        for i, o in enumerate(outs):
            if o is not None:
                _tensor(o, f"out{i}", dev)
        if ms is None:
            return
        m_in, m_out = ms
        _tensor(region_in, "region_in", dev, min_bytes=self.region_bytes_max(m_in))
        if kind in (BF16, F32):
            _tensor(local, "local", dev, numel=self.d)
        elif kind == PACKED:
            _tensor(local, "local", dev, min_bytes=self.region_bytes_max(m_in))
        elif kind == F32_PARTIAL:
            _tensor(local, "local", dev, min_bytes=self.partial_bytes_max(m_in))
        two = self.topology == BUTTERFLY and step < self.log2n
        # own-fp32: the child this worker keeps is written as fp32 partial sums
        keep = (int(worker) >> (self.log2n - int(step) - 1)) & 1 if two and self.own == OWN_F32 else -1
        for h, o in enumerate(outs):
            if o is not None:
                need = self.partial_bytes_max(m_out) if h == keep else self.region_bytes_max(m_out)
                _tensor(o, f"out{h}", dev, min_bytes=need)

    def _check_grads(self, grads):
        if len(grads) != self.n:
            raise ValueError(f"{len(grads)} gradients for {self.n} workers")
        kind = _kind(grads[0])
        for w, g in enumerate(grads):
            _tensor(g, f"grads[{w}]", self.device, numel=self.d, dtype=grads[0].dtype)
        return kind

    # ---- stages --------------------------------------------------------
    def stats(self, worker, grad, stream=None):
        _tensor(grad, "grad", self.device, numel=self.d)
        _check(lib().dq_stats(self.h, int(worker), _ptr(grad), _kind(grad), _stream(stream)),
               "dq_stats")

    def allocate(self, stream=None):
        _check(lib().dq_allocate(self.h, _stream(stream)), "dq_allocate")

    def reorder(self, stream=None):
        _check(lib().dq_reorder(self.h, _stream(stream)), "dq_reorder")

    def compress(self, worker, step, grad, region_out, stream=None):
        _tensor(grad, "grad", self.device, numel=self.d)
        _tensor(region_out, "region_out", self.device, min_bytes=self.region_bytes_max(self._m_compress()))
        _check(lib().dq_compress(self.h, int(worker), int(step), _ptr(grad), _kind(grad),
                                 _ptr(region_out), _stream(stream)), "dq_compress")

    def hop(self, worker, step, region_in, local, out0, out1=None, stream=None, local_kind=None):
        """local_kind: F32_PARTIAL for the own fp32 partial sums (OWN_F32);
        otherwise taken from the tensor's dtype."""
        kind = _kind(local) if local_kind is None else int(local_kind)
        self._check_hop(worker, step, region_in, local, kind, (out0, out1))
        _check(lib().dq_hop(self.h, int(worker), int(step), _ptr(region_in), _ptr(local),
                            kind, _ptr(out0), None if out1 is None else _ptr(out1),
                            _stream(stream)), "dq_hop")

    def hop_finalize(self, worker, step, region_in, local, region_out, out, stream=None, local_kind=None):
        kind = _kind(local) if local_kind is None else int(local_kind)
        self._check_hop(worker, step, region_in, local, kind, (region_out,))
        _tensor(out, "out", self.device, min_bytes=4 * self.d, dtype=torch.float32)
        _check(lib().dq_hop_finalize(self.h, int(worker), int(step), _ptr(region_in), _ptr(local), kind,
                                     _ptr(region_out), _ptr(out), _stream(stream)), "dq_hop_finalize")

    def finalize(self, part, region, out, stream=None):
        _tensor(region, "region", self.device, min_bytes=self.region_bytes_max(self.n))
        _tensor(out, "out", self.device, min_bytes=4 * self.d, dtype=torch.float32)
        _check(lib().dq_finalize(self.h, int(part), _ptr(region), _ptr(out), _stream(stream)),
               "dq_finalize")

    def final_part(self, worker):
        return int(lib().dq_final_part(self.h, int(worker)))

    # ---- whole round -----------------------------------------------------
    def region_bytes_max(self, m):
        return int(lib().dq_region_bytes_max(self.h, int(m)))

    def partial_bytes_max(self, m):
        return int(lib().dq_partial_bytes_max(self.h, int(m)))

    def new_region(self, m, device="cuda"):
        return torch.zeros(self.region_bytes_max(m), dtype=torch.uint8, device=device)

    def arena_bytes(self):
        return int(lib().dq_arena_bytes(self.h))

    def _round_buffers(self, grads, out, arena, arena_bytes):
        kind = self._check_grads(grads)
        if arena is None:
            arena = torch.empty(max(1, arena_bytes), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.d, dtype=torch.float32, device=self.device)
        _tensor(arena, "arena", self.device)
        _tensor(out, "out", self.device, min_bytes=4 * self.d, dtype=torch.float32)
        ptrs = (C.c_void_p * self.n)(*[g.data_ptr() for g in grads])
        return kind, out, arena, arena.numel() * arena.element_size(), ptrs

    def allreduce(self, grads, out=None, arena=None, stream=None):
        kind, out, arena, nbytes, ptrs = self._round_buffers(grads, out, arena, self.arena_bytes())
        _check(lib().dq_allreduce(self.h, ptrs, kind, _ptr(arena), nbytes, _ptr(out),
                                  _stream(stream)), "dq_allreduce")
        return out

    def allreduce_noalloc(self, grads, out, stream=None):
        """dq_allreduce_noalloc: the round in the library's static scratch
        (binds the plan there)."""
        kind = self._check_grads(grads)
        _tensor(out, "out", self.device, min_bytes=4 * self.d, dtype=torch.float32)
        ptrs = (C.c_void_p * self.n)(*[g.data_ptr() for g in grads])
        _check(lib().dq_allreduce_noalloc(self.h, ptrs, kind, _ptr(out), _stream(stream)),
               "dq_allreduce_noalloc")
        return out

    def mxfp8_allreduce(self, grads, out=None, arena=None, stream=None):
        kind, out, arena, nbytes, ptrs = self._round_buffers(
            grads, out, arena, int(lib().dq_mxfp8_arena_bytes(self.h)))
        _check(lib().dq_mxfp8_allreduce(self.h, ptrs, kind, _ptr(arena), nbytes, _ptr(out),
                                        _stream(stream)), "dq_mxfp8_allreduce")
        return out

    def mx_allreduce(self, fmt, grads, out=None, arena=None, stream=None):
        kind, out, arena, nbytes, ptrs = self._round_buffers(
            grads, out, arena, int(lib().dq_mx_arena_bytes(self.h)))
        _check(lib().dq_mx_allreduce(self.h, int(fmt), ptrs, kind, _ptr(arena), nbytes, _ptr(out),
                                     _stream(stream)), "dq_mx_allreduce")
        return out

    # ---- inspection ------------------------------------------------------
    def info(self, stream=None):
        i = dq_info()
        rc = lib().dq_get_info(self.h, C.byref(i), _stream(stream))
        if rc not in (DQ_OK, DQ_ENONFINITE):
            _check(rc, "dq_get_info")
        counts = list(i.class_counts) + ([i.class_count16] if self.max_width == 16 else [])
        return {"rho_bits": i.rho_bits, "rho": i.rho, "t12": i.t12, "t24": i.t24, "t48": i.t48,
                "t816": i.t816, "class_counts": counts, "budget_bits": i.budget_bits,
                "used_bits": i.used_bits, "achieved_bits": i.achieved_bits,
                "nonfinite": bool(i.nonfinite), "status": rc}

    def timing(self):
        t = dq_timing()
        _check(lib().dq_timing_read(self.h, C.byref(t)), "dq_timing_read")
        return {k: {"ms": t.ms[i], "launches": t.launches[i], "coords": t.coords[i]}
                for i, k in enumerate(KERNEL_KINDS)}

    def _view(self, name, dtype, count):
        off = self.layout[name]
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)

    def stats_arrays(self):
        return self._view("sum", torch.float32, self.J), self._view("sumsq", torch.float32, self.J)

    def widths(self):
        return self._view("widths", torch.uint8, self.J)

    def perm(self):
        return self._view("perm", torch.int32, self.J), self._view("inv", torch.int32, self.J)

    def mu_stream(self):
        return self._view("mu_stream", torch.float32, self.J)
