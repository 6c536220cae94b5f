// dq_api.cpp -- the C ABI of include/dq.h: plan state, argument checks, the
// ring / butterfly schedules and launch sequencing.  All device work is
// enqueued on the caller's stream; nothing here synchronises except
// dq_get_info and dq_timing_read.
#include "dq.h"

#include <cmath>
#include <cstddef>
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "dq_internal.h"
#include "dq_tables.h"

using namespace dq;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Launch {
    int kind;
    int64_t m, part;     // part processed (for coordinate counts), m = 0: whole vector
    hipEvent_t e0, e1;
};

}  // namespace

struct dq_plan {
    int64_t d = 0, J = 0;
    int32_t n = 1, topo = DQ_RING, L = 0;
    float budget = 5.0f;
    long long budget_bits = 0;
    uint64_t seed = 1;
    uint32_t round = 0;
    int32_t rounding = DQ_ROUND_STRATIFIED;
    int32_t alloc = DQ_ALLOC_THRESHOLD;
    int32_t own = DQ_OWN_PACKED;           // butterfly own operand at levels >= 2
    bool timing = false;
    uint32_t timing_kinds = (1u << DQ_K_COUNT) - 1u;   // kinds timed while timing is on
    double eps = kDefaultEps;                          // level shape
    int32_t qmax = 8;                                  // widest class: 8, or 16 (DQ_OPT_MAX_WIDTH)
    bool tables_dirty = true;                          // workspace tables to (re)build

    uint8_t *ws = nullptr;
    size_t ws_bytes = 0;
    dq_layout lay{};
    int64_t nblk = 0;

    int32_t stats_done = 0;
    bool allocated = false, reordered = false;

    std::vector<Launch> launches;
    std::vector<hipEvent_t> pool;
    // DQ_OPT_STREAMS = 2: dq_allreduce's second stream and its fork/join events
    int32_t streams = 1;
    hipStream_t aux = nullptr;
    hipEvent_t fork_ev = nullptr, join_ev = nullptr;
    dq_timing acc{};
    int64_t host_counts[kClasses] = {0, 0, 0, 0};
};

namespace {

Ctrl *ctrl_of(dq_plan *p) { return reinterpret_cast<Ctrl *>(p->ws + p->lay.ctrl); }
float *f32_at(dq_plan *p, size_t off) { return reinterpret_cast<float *>(p->ws + off); }
int32_t *i32_at(dq_plan *p, size_t off) { return reinterpret_cast<int32_t *>(p->ws + off); }
int32_t *blkcnt_of(dq_plan *p) {
    return reinterpret_cast<int32_t *>(p->ws + p->lay.ctrl + align_up(sizeof(Ctrl), kAlign));
}
PartInfo *parts_of(dq_plan *p) {
    return reinterpret_cast<PartInfo *>(p->ws + p->lay.ctrl + align_up(sizeof(Ctrl), kAlign) +
                                        align_up(4 * kClasses * (size_t)p->nblk, kAlign));
}
const PartInfo *part_entry(dq_plan *p, int64_t m, int64_t c) {
    return parts_of(p) + part_table_index(p->n, p->topo, m, c);
}

void compute_layout(dq_plan *p) {
    const size_t J = (size_t)p->J;
    size_t off = 0;
    p->lay.sum = off; off = align_up(off + 4 * J, kAlign);
    p->lay.sumsq = off; off = align_up(off + 4 * J, kAlign);
    p->lay.widths = off; off = align_up(off + J, kAlign);
    p->lay.perm = off; off = align_up(off + 4 * J, kAlign);
    p->lay.inv = off; off = align_up(off + 4 * J, kAlign);
    p->lay.mu_stream = off; off = align_up(off + 4 * J, kAlign);
    p->lay.tables = off; off = align_up(off + sizeof(DeviceTables), kAlign);
    p->lay.ctrl = off;
    off = align_up(off + sizeof(Ctrl), kAlign);
    off = align_up(off + 4 * kClasses * (size_t)p->nblk, kAlign);
    off = align_up(off + sizeof(PartInfo) * (size_t)part_table_entries(p->n, p->topo), kAlign);
    // the 16-bit class's 65,536 levels and weights, then the same as
    // (level, weight) pairs for the search
    p->lay.tables16 = 0;
    if (p->qmax == 16) {
        p->lay.tables16 = off;
        off = align_up(off + 4 * 65536 * sizeof(float), kAlign);
    }
    p->lay.total = off;
}

hipError_t timed_begin(dq_plan *p, int kind, int64_t m, int64_t part, hipStream_t s, Launch &L) {
    L.kind = kind;
    L.m = m;
    L.part = part;
    L.e0 = L.e1 = nullptr;
    if (!p->timing || !((p->timing_kinds >> kind) & 1u)) return hipSuccess;
    for (hipEvent_t *e : {&L.e0, &L.e1}) {
        if (!p->pool.empty()) {
            *e = p->pool.back();
            p->pool.pop_back();
        } else {
            hipError_t err = hipEventCreate(e);
            if (err != hipSuccess) return err;
        }
    }
    return hipEventRecord(L.e0, s);
}

hipError_t timed_end(dq_plan *p, Launch &L, hipStream_t s) {
    if (!p->timing || !L.e0) return hipSuccess;
    hipError_t err = hipEventRecord(L.e1, s);
    p->launches.push_back(L);
    return err;
}

dq_status hip_status(hipError_t e) { return e == hipSuccess ? DQ_OK : DQ_EHIP; }

// schedule: part written by a compress / processed by a hop
struct SchedPart {
    int64_t m, part;
    bool two_children;
};

bool compress_part(const dq_plan *p, int32_t w, int32_t step, SchedPart &sp) {
    sp.two_children = false;
    if (p->n == 1) {
        if (step != 0) return false;
        sp.m = 1;
        sp.part = 0;
        return true;
    }
    if (p->topo == DQ_RING) {
        if (step != 0) return false;
        sp.m = p->n;
        sp.part = w;
        return true;
    }
    if (step != 1) return false;
    sp.m = 2;
    sp.part = ((int64_t)w >> (p->L - 1)) ^ 1;
    return true;
}

bool hop_part(const dq_plan *p, int32_t w, int32_t step, SchedPart &sp) {
    if (p->n == 1) return false;
    if (p->topo == DQ_RING) {
        if (step < 1 || step >= p->n) return false;
        sp.m = p->n;
        sp.part = ((int64_t)w - step % p->n + p->n) % p->n;
        sp.two_children = false;
        return true;
    }
    if (step < 1 || step > p->L) return false;
    sp.m = (int64_t)1 << step;
    sp.part = (int64_t)w >> (p->L - step);
    sp.two_children = step < p->L;
    return true;
}

int32_t event_of(const dq_plan *p, int32_t w, int32_t step) {
    if (p->topo == DQ_BUTTERFLY && p->n > 1) return (step - 1) * p->n + w;
    return w;
}

// Philox tag and 16-bit stagger of the quantisations a launch makes:
//   correlated:  tag 0 for every event, staggered by the worker's rank of n;
//   independent: tag 1 + event, no stagger;
//   stratified:  a fresh tag per schedule level and a stagger among the
//                workers that quantise the same coordinates at that level --
//                ring step t: tag 1 + t, no stagger (one worker per part and
//                step); butterfly compress: tag 1, k = w mod n/2 of n/2;
//                butterfly hop of level s: tag 1 + s, k = w mod 2^(L-s) of
//                2^(L-s); n = 1: tag 1.  Stagger floor(k 65536 / P).
void fill_rng(const dq_plan *p, int32_t w, int32_t step, bool is_compress, CodecArgs &a) {
    a.key0 = (uint32_t)(p->seed & 0xFFFFFFFFu);
    a.key1 = (uint32_t)(p->seed >> 32);
    a.round = p->round;
    if (p->rounding == DQ_ROUND_STRATIFIED) {
        uint32_t P = 1u, k = 0u;
        if (p->n == 1) {
            a.tag = 1u;
        } else if (p->topo == DQ_RING) {
            a.tag = 1u + (uint32_t)step;
        } else if (is_compress) {
            a.tag = 1u;
            P = (uint32_t)(p->n / 2);
            k = (uint32_t)w % P;
        } else {
            a.tag = 1u + (uint32_t)step;
            P = 1u << (p->L - step);
            k = (uint32_t)w % P;
        }
        a.stagger = (uint32_t)(((uint64_t)k * 65536u) / P);
    } else if (p->rounding == DQ_ROUND_CORRELATED) {
        a.tag = 0u;
        a.stagger = (uint32_t)(((uint64_t)w * 65536u) / (uint64_t)p->n);
    } else {
        a.tag = (uint32_t)(1 + event_of(p, w, step));
        a.stagger = 0u;
    }
}

void fill_common(dq_plan *p, CodecArgs &a) {
    std::memset(&a, 0, sizeof(a));
    a.tab = reinterpret_cast<const DeviceTables *>(p->ws + p->lay.tables);
    a.perm = i32_at(p, p->lay.perm);
    a.mu_stream = f32_at(p, p->lay.mu_stream);
    a.n_workers_f = (float)p->n;
    if (p->qmax == 16) {
        a.L16 = f32_at(p, p->lay.tables16);
        a.W16 = a.L16 + 65536;
        a.LW16 = reinterpret_cast<const Pair *>(a.L16 + 2 * 65536);
    }
    a.eps = (float)p->eps;
}

// bytes of one super-group in a region at the widest class: codes, scale
// unit, group codes
size_t sg_region_bytes(const dq_plan *p) { return (size_t)(32 * p->qmax + 4 + 16); }

// a part of the smallest m the schedule uses must stay below 4 GB (32-bit
// region offsets in the kernels)
bool region_fits(int64_t n_coords, int32_t n, int32_t topology, size_t per_sg) {
    const int64_t m_min = n == 1 ? 1 : (topology == DQ_RING ? n : 2);
    return (n_coords / kSG / m_min + 3) * (int64_t)per_sg + 256 < ((int64_t)1 << 32);
}

int64_t max_part_sg(const dq_plan *p, int64_t m) { return p->J / m + 3; }

int local_of_kind(int32_t kind) {
    if (kind == DQ_BF16) return kLocalBF16;
    if (kind == DQ_F32) return kLocalF32;
    if (kind == DQ_PACKED) return kLocalPacked;
    if (kind == DQ_F32_PARTIAL) return kLocalPartial;
    return -1;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace

namespace {

struct ArenaPlan {
    std::vector<size_t> off;  // slot offsets
    size_t total = 0;
};

// ring: 2n slots of m = n; butterfly: per worker one compress slot (m = 2),
// two child slots per level below the last, one slot for the last level;
// n == 1: one slot of m = 1.
ArenaPlan arena_plan(const dq_plan *p) {
    ArenaPlan ap;
    auto add = [&](int64_t m) {
        ap.off.push_back(ap.total);
        ap.total += dq_region_bytes_max(p, m);
    };
    if (p->n == 1) {
        add(1);
    } else if (p->topo == DQ_RING) {
        for (int i = 0; i < 2 * p->n; i++) add(p->n);
    } else {
        for (int w = 0; w < p->n; w++) {
            add(2);
            for (int s = 1; s <= p->L; s++) {
                if (s < p->L) {
                    const int64_t m = (int64_t)1 << (s + 1);
                    const int keep = (w >> (p->L - s - 1)) & 1;
                    for (int h = 0; h < 2; h++) {
                        if (p->own == DQ_OWN_F32 && h == keep) {
                            ap.off.push_back(ap.total);
                            ap.total += dq_partial_bytes_max(p, m);
                        } else {
                            add(m);
                        }
                    }
                } else {
                    add(p->n);
                }
            }
        }
    }
    return ap;
}

}  // namespace

extern "C" {

const char *dq_status_string(int32_t s) {
    switch (s) {
        case DQ_OK: return "ok";
        case DQ_EINVAL: return "invalid argument";
        case DQ_EBUDGET: return "bit budget below 2 or NaN";
        case DQ_ESTATE: return "call out of stage order";
        case DQ_EWORKSPACE: return "workspace missing, too small or misaligned";
        case DQ_ENULL: return "null pointer";
        case DQ_EHIP: return "HIP runtime error";
        case DQ_ENONFINITE: return "non-finite gradient value";
        default: return "unknown status";
    }
}

int32_t dq_version(void) { return 1; }

dq_status dq_plan_create(int64_t n_coords, int32_t n_workers, int32_t topology, float avg_bits,
                         dq_plan **out) {
    if (!out) return DQ_ENULL;
    *out = nullptr;
    if (n_coords <= 0 || n_coords % kSG != 0 || n_workers < 1 || n_workers > 65536)
        return DQ_EINVAL;
    if (n_coords / kSG > (int64_t)0x7FFFFFFF - 4) return DQ_EINVAL;
    if (topology != DQ_RING && topology != DQ_BUTTERFLY) return DQ_EINVAL;
    int32_t L = 0;
    while ((1 << L) < n_workers) L++;
    if (topology == DQ_BUTTERFLY && (1 << L) != n_workers) return DQ_EINVAL;
    if (!(avg_bits >= 2.0f)) return DQ_EBUDGET;
    // codec kernels address a region with 32-bit offsets: the largest region
    // (a part of the smallest m the schedule uses) must stay below 4 GB
    if (!region_fits(n_coords, n_workers, topology, 256 + 4 + 16)) return DQ_EINVAL;
    dq_plan *p = new (std::nothrow) dq_plan();
    if (!p) return DQ_EINVAL;
    p->d = n_coords;
    p->J = n_coords / kSG;
    p->n = n_workers;
    p->topo = topology;
    p->L = L;
    p->budget = avg_bits;
    // floor(B J); the widths sum to at most 8 J, so any B >= 8 (including
    // +inf) is the budget 8 J and the product stays in range
    p->budget_bits = (long long)std::floor(std::min((double)avg_bits, 8.0) * (double)p->J);
    p->nblk = (p->J + kReorderSGPerBlock - 1) / kReorderSGPerBlock;
    compute_layout(p);
    *out = p;
    return DQ_OK;
}

void dq_plan_destroy(dq_plan *p) {
    if (!p) return;
    for (auto &L : p->launches) {
        if (L.e0) (void)hipEventDestroy(L.e0);
        if (L.e1) (void)hipEventDestroy(L.e1);
    }
    for (auto e : p->pool) (void)hipEventDestroy(e);
    if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
    if (p->join_ev) (void)hipEventDestroy(p->join_ev);
    if (p->aux) (void)hipStreamDestroy(p->aux);
    delete p;
}

dq_status dq_plan_set_u64(dq_plan *p, int32_t option, uint64_t v) {
    if (!p) return DQ_ENULL;
    switch (option) {
        case DQ_OPT_SEED: p->seed = v; return DQ_OK;
        case DQ_OPT_ROUND:
            if (v > 0xFFFFFFFFull) return DQ_EINVAL;
            p->round = (uint32_t)v;
            return DQ_OK;
        case DQ_OPT_ROUNDING:
            if (v != DQ_ROUND_CORRELATED && v != DQ_ROUND_INDEPENDENT && v != DQ_ROUND_STRATIFIED)
                return DQ_EINVAL;
            p->rounding = (int32_t)v;
            return DQ_OK;
        case DQ_OPT_TIMING:
            if (v > 1) return DQ_EINVAL;
            p->timing = v == 1;
            return DQ_OK;
        case DQ_OPT_TIMING_KINDS:
            if (v == 0 || v >= (1ull << DQ_K_COUNT)) return DQ_EINVAL;
            p->timing_kinds = (uint32_t)v;
            return DQ_OK;
        case DQ_OPT_OWN:
            if (v != DQ_OWN_PACKED && v != DQ_OWN_F32) return DQ_EINVAL;
            p->own = (int32_t)v;
            return DQ_OK;
        case DQ_OPT_ALLOC:
            if (v != DQ_ALLOC_THRESHOLD && v != DQ_ALLOC_MEAN_CORRECTED && v != DQ_ALLOC_UNIFORM)
                return DQ_EINVAL;
            p->alloc = (int32_t)v;
            return DQ_OK;
        case DQ_OPT_MAX_WIDTH: {
            if (v != 8 && v != 16) return DQ_EINVAL;
            if (v == 16 && !region_fits(p->d, p->n, p->topo, 512 + 4 + 16)) return DQ_EINVAL;
            p->qmax = (int32_t)v;
            p->budget_bits = (long long)std::floor(std::min((double)p->budget, (double)p->qmax) * (double)p->J);
            compute_layout(p);
            // the workspace size changed: bind again before the next round
            p->ws = nullptr;
            p->ws_bytes = 0;
            p->stats_done = 0;
            p->allocated = p->reordered = false;
            p->tables_dirty = true;
            return DQ_OK;
        }
        case DQ_OPT_STREAMS:
            if (v != 1 && v != 2) return DQ_EINVAL;
            if (v == 2) {
                // each resource once, so that a retry after a failure completes the set;
                // the stream has the default priority and does not sync with the null stream
                if (!p->aux && hipStreamCreateWithFlags(&p->aux, hipStreamNonBlocking) != hipSuccess) {
                    p->aux = nullptr;
                    return DQ_EHIP;
                }
                if (!p->fork_ev && hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming) != hipSuccess) {
                    p->fork_ev = nullptr;
                    return DQ_EHIP;
                }
                if (!p->join_ev && hipEventCreateWithFlags(&p->join_ev, hipEventDisableTiming) != hipSuccess) {
                    p->join_ev = nullptr;
                    return DQ_EHIP;
                }
            }
            p->streams = (int32_t)v;
            return DQ_OK;
        default: return DQ_EINVAL;
    }
}

dq_status dq_plan_set_f64(dq_plan *p, int32_t option, double v) {
    if (!p) return DQ_ENULL;
    if (option != DQ_OPT_EPS) return DQ_EINVAL;
    // (0, 1], and every bucket of the interval search may hold at most one
    // level boundary for this shape
    if (!(v > 0.0 && v <= 1.0) || !level_shape_ok(v)) return DQ_EINVAL;
    p->eps = v;
    p->tables_dirty = true;
    return DQ_OK;
}

size_t dq_workspace_bytes(const dq_plan *p) { return p ? p->lay.total : 0; }

dq_status dq_plan_bind(dq_plan *p, void *ws, size_t bytes) {
    if (!p || !ws) return DQ_ENULL;
    if (bytes < p->lay.total || !aligned(ws, kAlign)) return DQ_EWORKSPACE;
    p->ws = static_cast<uint8_t *>(ws);
    p->tables_dirty = true;
    p->ws_bytes = bytes;
    p->stats_done = 0;
    p->allocated = p->reordered = false;
    return DQ_OK;
}

dq_status dq_workspace_layout(const dq_plan *p, dq_layout *out) {
    if (!p || !out) return DQ_ENULL;
    *out = p->lay;
    return DQ_OK;
}

size_t dq_partial_bytes_max(const dq_plan *p, int64_t m) {
    if (!p || m < 1 || m > p->n || (p->n % m) != 0) return 0;
    return align_up((size_t)max_part_sg(p, m) * kSG * sizeof(float), kAlign);
}

size_t dq_region_bytes_max(const dq_plan *p, int64_t m) {
    if (!p || m < 1 || m > p->n || (p->n % m) != 0) return 0;
    const int64_t N = max_part_sg(p, m);
    return align_up((size_t)N * sg_region_bytes(p) + 16, kAlign);
}

int64_t dq_final_part(const dq_plan *p, int32_t w) {
    if (!p || w < 0 || w >= p->n) return -1;
    if (p->n == 1) return 0;
    if (p->topo == DQ_RING) return (w + 1) % p->n;
    return w;
}

dq_status dq_stats(dq_plan *p, int32_t w, const void *grad, int32_t kind, void *stream) {
    if (!p || !grad) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (w < 0 || w >= p->n || (kind != DQ_BF16 && kind != DQ_F32) || !aligned(grad, 16))
        return DQ_EINVAL;
    if (w == 0) {
        p->stats_done = 0;
        p->allocated = p->reordered = false;
    }
    if (w != p->stats_done) return DQ_ESTATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (w == 0) {
        hipError_t e = launch_zero(reinterpret_cast<uint32_t *>(&ctrl_of(p)->nonfinite), 1, s);
        // the first round after a bind or a new level shape builds the tables
        // on the device, ahead of every codec launch on this stream
        if (e == hipSuccess && p->tables_dirty)
            e = launch_build_tables(reinterpret_cast<DeviceTables *>(p->ws + p->lay.tables), p->eps, s);
        if (e == hipSuccess && p->tables_dirty && p->qmax == 16) {
            float *L16 = f32_at(p, p->lay.tables16);
            e = launch_build_tables16(L16, L16 + 65536, reinterpret_cast<Pair *>(L16 + 2 * 65536), p->eps, s);
        }
        if (e != hipSuccess) return DQ_EHIP;
        p->tables_dirty = false;
    }
    StatsArgs a;
    a.grad = grad;
    a.J = p->J;
    a.sum = f32_at(p, p->lay.sum);
    a.sumsq = f32_at(p, p->lay.sumsq);
    a.first = w == 0;
    a.nonfinite = &ctrl_of(p)->nonfinite;
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_STATS, 0, 0, s, L);
    if (e == hipSuccess) e = launch_stats(a, kind == DQ_F32, s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    if (e != hipSuccess) return DQ_EHIP;
    p->stats_done++;
    return DQ_OK;
}

dq_status dq_allocate(dq_plan *p, void *stream) {
    if (!p) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (p->stats_done != p->n) return DQ_ESTATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    AllocArgs a;
    a.sumsq = f32_at(p, p->lay.sumsq);
    a.J = p->J;
    a.budget = p->budget_bits;
    a.ctrl = ctrl_of(p);
    a.widths = p->ws + p->lay.widths;
    a.blkcnt = blkcnt_of(p);
    a.nblk = p->nblk;
    a.sum = f32_at(p, p->lay.sum);
    a.denom = (float)(256 * p->n);
    a.mode = p->alloc;
    a.wide = p->qmax == 16;
    // uniform: the widest class whose width fits the budget
    a.uniform_k = (a.wide && p->budget >= 16.0f) ? 3 : (p->budget >= 8.0f ? 2 : (p->budget >= 4.0f ? 1 : 0));
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_ALLOCATE, 0, 0, s, L);
    // histograms, class counts, prefix and flag start at zero (a fill kernel,
    // graph-safe); nonfinite is kept (it belongs to the stats of this round)
    const int64_t nzero = (int64_t)(offsetof(Ctrl, rho_bits) / 4);
    if (e == hipSuccess) e = launch_zero(reinterpret_cast<uint32_t *>(a.ctrl), nzero, s);
    if (p->alloc != DQ_ALLOC_UNIFORM)
        for (int pass = 0; pass < kRadixPasses && e == hipSuccess; pass++) e = launch_alloc_pass(a, pass, s);
    if (e == hipSuccess) e = launch_alloc_final(a, s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    if (e != hipSuccess) return DQ_EHIP;
    p->allocated = true;
    p->reordered = false;
    return DQ_OK;
}

dq_status dq_reorder(dq_plan *p, void *stream) {
    if (!p) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (!p->allocated) return DQ_ESTATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ReorderArgs a;
    a.widths = p->ws + p->lay.widths;
    a.sum = f32_at(p, p->lay.sum);
    a.denom = (float)(256 * p->n);
    a.J = p->J;
    a.ctrl = ctrl_of(p);
    a.blkcnt = blkcnt_of(p);
    a.nblk = p->nblk;
    a.perm = i32_at(p, p->lay.perm);
    a.inv = i32_at(p, p->lay.inv);
    a.mu_stream = f32_at(p, p->lay.mu_stream);
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_REORDER, 0, 0, s, L);
    if (e == hipSuccess) e = launch_reorder(a, s);
    if (e == hipSuccess) e = launch_part_table(ctrl_of(p)->class_counts, p->n, p->topo, parts_of(p), s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    if (e != hipSuccess) return DQ_EHIP;
    p->reordered = true;
    return DQ_OK;
}

dq_status dq_compress(dq_plan *p, int32_t w, int32_t step, const void *grad, int32_t kind,
                      void *out, void *stream) {
    if (!p || !grad || !out) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (!p->reordered) return DQ_ESTATE;
    SchedPart sp;
    if (w < 0 || w >= p->n || (kind != DQ_BF16 && kind != DQ_F32) || !compress_part(p, w, step, sp))
        return DQ_EINVAL;
    if (!aligned(grad, 16) || !aligned(out, 16)) return DQ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    CodecArgs a;
    fill_common(p, a);
    fill_rng(p, w, step, true, a);
    a.part_out = a.part_in = part_entry(p, sp.m, sp.part);
    a.grad = grad;
    a.out = static_cast<uint8_t *>(out);
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_COMPRESS, sp.m, sp.part, s, L);
    if (e == hipSuccess) e = launch_codec(a, kCompress, local_of_kind(kind), max_part_sg(p, sp.m), p->qmax == 16, s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    return hip_status(e);
}

namespace {

// dq_hop, and dq_hop_finalize when final_out is set (the schedule's last step)
dq_status hop_impl(dq_plan *p, int32_t w, int32_t step, const void *in, const void *local,
                   int32_t local_kind, void *out0, void *out1, float *final_out, void *stream) {
    if (!p || !in || !local || !out0) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (!p->reordered) return DQ_ESTATE;
    SchedPart sp;
    if (w < 0 || w >= p->n || !hop_part(p, w, step, sp)) return DQ_EINVAL;
    // butterfly levels >= 2 take the worker's own kept child: packed, or fp32
    // partial sums under DQ_OWN_F32
    const bool own32 = p->topo == DQ_BUTTERFLY && p->own == DQ_OWN_F32;
    const bool want_own = p->topo == DQ_BUTTERFLY && step >= 2;
    const int32_t own_kind = own32 ? DQ_F32_PARTIAL : DQ_PACKED;
    if (want_own != (local_kind == own_kind)) return DQ_EINVAL;
    if (!want_own && local_kind != DQ_BF16 && local_kind != DQ_F32) return DQ_EINVAL;
    if (sp.two_children && !out1) return DQ_ENULL;
    if (!aligned(in, 16) || !aligned(local, 16) || !aligned(out0, 16) ||
        (sp.two_children && !aligned(out1, 16)))
        return DQ_EINVAL;
    // the fused final step: only where the hop's part is a final part
    if (final_out && (sp.two_children || sp.m != p->n || (p->topo == DQ_RING && step != p->n - 1) ||
                      !aligned(final_out, 16)))
        return DQ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    CodecArgs a;
    fill_common(p, a);
    fill_rng(p, w, step, false, a);
    a.part_in = part_entry(p, sp.m, sp.part);
    a.region_in = static_cast<const uint8_t *>(in);
    if (local_kind == DQ_PACKED) a.region_own = static_cast<const uint8_t *>(local);
    else if (local_kind == DQ_F32_PARTIAL) a.partial_in = static_cast<const float *>(local);
    else a.grad = local;
    const int kindk = final_out ? DQ_K_HOP_FINAL : (want_own ? DQ_K_HOP_PACKED : DQ_K_HOP_GRAD);
    // the child this worker keeps for the next level (own-fp32: written as fp32)
    const int keep = (own32 && sp.two_children) ? (w >> (p->L - step - 1)) & 1 : -1;
    hipError_t e = hipSuccess;
    if (sp.two_children && keep < 0) {
        // both children in one launch (the kernel splits its blocks between
        // them), timed as the parent part they make up together
        a.part_out = part_entry(p, 2 * sp.m, 2 * sp.part);
        a.part_out2 = part_entry(p, 2 * sp.m, 2 * sp.part + 1);
        a.out = static_cast<uint8_t *>(out0);
        a.out2 = static_cast<uint8_t *>(out1);
        Launch L;
        e = timed_begin(p, kindk, sp.m, sp.part, s, L);
        if (e == hipSuccess)
            e = launch_codec(a, kHop, local_of_kind(local_kind), max_part_sg(p, 2 * sp.m), p->qmax == 16, s);
        if (e == hipSuccess) e = timed_end(p, L, s);
        return hip_status(e);
    }
    // one launch per output region: the part itself, or (own-fp32 variant,
    // whose kept child takes another mode) each of its two children
    const int nout = sp.two_children ? 2 : 1;
    for (int h = 0; h < nout && e == hipSuccess; h++) {
        const int64_t m_out = sp.two_children ? 2 * sp.m : sp.m;
        const int64_t c_out = sp.two_children ? 2 * sp.part + h : sp.part;
        void *dst = h == 0 ? out0 : out1;
        a.part_out = part_entry(p, m_out, c_out);
        a.out = h == keep ? nullptr : static_cast<uint8_t *>(dst);
        a.partial_out = h == keep ? static_cast<float *>(dst) : nullptr;
        a.out_f32 = final_out;
        const int mode = h == keep ? kPartial : (final_out ? kHopFinal : kHop);
        Launch L;
        e = timed_begin(p, kindk, m_out, c_out, s, L);
        if (e == hipSuccess)
            e = launch_codec(a, mode, local_of_kind(local_kind), max_part_sg(p, m_out), p->qmax == 16, s);
        if (e == hipSuccess) e = timed_end(p, L, s);
    }
    return hip_status(e);
}

}  // namespace

dq_status dq_hop(dq_plan *p, int32_t w, int32_t step, const void *in, const void *local,
                 int32_t local_kind, void *out0, void *out1, void *stream) {
    return hop_impl(p, w, step, in, local, local_kind, out0, out1, nullptr, stream);
}

dq_status dq_hop_finalize(dq_plan *p, int32_t w, int32_t step, const void *in, const void *local,
                          int32_t local_kind, void *region_out, float *out, void *stream) {
    if (!out) return DQ_ENULL;
    return hop_impl(p, w, step, in, local, local_kind, region_out, nullptr, out, stream);
}

dq_status dq_finalize(dq_plan *p, int64_t part, const void *region, float *out, void *stream) {
    if (!p || !region || !out) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (!p->reordered) return DQ_ESTATE;
    if (part < 0 || part >= p->n) return DQ_EINVAL;
    if (!aligned(region, 16) || !aligned(out, 16)) return DQ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    CodecArgs a;
    fill_common(p, a);
    a.part_out = a.part_in = part_entry(p, p->n, part);
    a.region_in = static_cast<const uint8_t *>(region);
    a.out_f32 = out;
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_FINALIZE, p->n, part, s, L);
    if (e == hipSuccess) e = launch_codec(a, kFinalize, kLocalNone, max_part_sg(p, p->n), p->qmax == 16, s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    return hip_status(e);
}

// ---- whole round -----------------------------------------------------------


size_t dq_arena_bytes(const dq_plan *p) { return p ? arena_plan(p).total : 0; }

dq_status dq_allreduce(dq_plan *p, const void *const *grads, int32_t kind, void *arena,
                       size_t arena_bytes, float *out, void *stream) {
    if (!p || !grads || !arena || !out) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    const ArenaPlan ap = arena_plan(p);
    if (arena_bytes < ap.total || !aligned(arena, kAlign)) return DQ_EWORKSPACE;
    uint8_t *A = static_cast<uint8_t *>(arena);
    dq_status st;
    for (int w = 0; w < p->n; w++)
        if ((st = dq_stats(p, w, grads[w], kind, stream)) != DQ_OK) return st;
    if ((st = dq_allocate(p, stream)) != DQ_OK) return st;
    if ((st = dq_reorder(p, stream)) != DQ_OK) return st;
    const int n = p->n;
    if (n == 1) {
        if ((st = dq_compress(p, 0, 0, grads[0], kind, A + ap.off[0], stream)) != DQ_OK) return st;
        return dq_finalize(p, 0, A + ap.off[0], out, stream);
    }
    // Within one schedule step the workers' launches are independent.  With two
    // streams the odd workers' launches go to the plan's second stream, forked
    // from and joined back into the caller's stream around every step, so one
    // launch's tail overlaps the next launch's start.
    hipStream_t main_s = static_cast<hipStream_t>(stream);
    const bool two = p->streams == 2;
    auto fork = [&]() -> dq_status {
        if (!two) return DQ_OK;
        if (hipEventRecord(p->fork_ev, main_s) != hipSuccess) return DQ_EHIP;
        return hipStreamWaitEvent(p->aux, p->fork_ev, 0) == hipSuccess ? DQ_OK : DQ_EHIP;
    };
    auto join = [&]() -> dq_status {
        if (!two) return DQ_OK;
        if (hipEventRecord(p->join_ev, p->aux) != hipSuccess) return DQ_EHIP;
        return hipStreamWaitEvent(main_s, p->join_ev, 0) == hipSuccess ? DQ_OK : DQ_EHIP;
    };
    auto sw = [&](int w) -> void * { return two && (w & 1) ? static_cast<void *>(p->aux) : stream; };
    if (p->topo == DQ_RING) {
        auto slot = [&](int w, int t) { return A + ap.off[(size_t)(t & 1) * n + w]; };
        if ((st = fork()) != DQ_OK) return st;
        for (int w = 0; w < n; w++)
            if ((st = dq_compress(p, w, 0, grads[w], kind, slot(w, 0), sw(w))) != DQ_OK) return st;
        if ((st = join()) != DQ_OK) return st;
        // the last step's hops also write the decoded sum (no separate finalize)
        for (int t = 1; t < n; t++) {
            if ((st = fork()) != DQ_OK) return st;
            for (int w = 0; w < n; w++) {
                const void *in = slot((w - 1 + n) % n, t - 1);
                st = t < n - 1 ? dq_hop(p, w, t, in, grads[w], kind, slot(w, t), nullptr, sw(w))
                               : dq_hop_finalize(p, w, t, in, grads[w], kind, slot(w, t), out, sw(w));
                if (st != DQ_OK) return st;
            }
            if ((st = join()) != DQ_OK) return st;
        }
        return DQ_OK;
    }
    const int L = p->L;
    const size_t per_w = 1 + (size_t)(2 * (L - 1) + 1);
    auto cmp = [&](int w) { return A + ap.off[w * per_w]; };
    auto lvl = [&](int w, int s, int h) { return A + ap.off[w * per_w + 1 + 2 * (s - 1) + h]; };
    if ((st = fork()) != DQ_OK) return st;
    for (int w = 0; w < n; w++)
        if ((st = dq_compress(p, w, 1, grads[w], kind, cmp(w), sw(w))) != DQ_OK) return st;
    if ((st = join()) != DQ_OK) return st;
    for (int s = 1; s <= L; s++) {
        if ((st = fork()) != DQ_OK) return st;
        for (int w = 0; w < n; w++) {
            const int partner = w ^ (n >> s);
            const int keep = (w >> (L - s)) & 1;
            const void *in = s == 1 ? (const void *)cmp(partner) : (const void *)lvl(partner, s - 1, keep);
            const void *local = s == 1 ? grads[w] : (const void *)lvl(w, s - 1, keep);
            const int32_t lk = s == 1 ? kind : (p->own == DQ_OWN_F32 ? DQ_F32_PARTIAL : DQ_PACKED);
            st = s < L ? dq_hop(p, w, s, in, local, lk, lvl(w, s, 0), lvl(w, s, 1), sw(w))
                       : dq_hop_finalize(p, w, s, in, local, lk, lvl(w, s, 0), out, sw(w));
            if (st != DQ_OK) return st;
        }
        if ((st = join()) != DQ_OK) return st;
    }
    return DQ_OK;
}

size_t dq_noalloc_max_bytes(void) { return kScratchBytes; }

dq_status dq_allreduce_noalloc(dq_plan *p, const void *const *grads, int32_t kind, float *out,
                               void *stream) {
    if (!p || !grads || !out) return DQ_ENULL;
    const size_t ws = align_up(p->lay.total, kAlign);
    const size_t arena = arena_plan(p).total;
    if (ws + arena > kScratchBytes) return DQ_EWORKSPACE;
    void *base = nullptr;
    if (scratch_address(&base) != hipSuccess || !base) return DQ_EHIP;
    // the plan's state moves into the scratch (a bind: tables are rebuilt by
    // this round's first dq_stats, every stage clears what it accumulates);
    // launch timing would create events, so it is off for this call
    dq_status st = dq_plan_bind(p, base, ws);
    if (st != DQ_OK) return st;
    const bool timing = p->timing;
    p->timing = false;
    st = dq_allreduce(p, grads, kind, static_cast<uint8_t *>(base) + ws, arena, out, stream);
    p->timing = timing;
    return st;
}

// ---- inspection --------------------------------------------------------------

dq_status dq_check_reciprocal(uint32_t lo, uint32_t count, unsigned long long *d_mismatches, void *stream) {
    if (!d_mismatches) return DQ_ENULL;
    if ((uint64_t)lo + count > 0x100000000ull) return DQ_EINVAL;
    if (count == 0) return DQ_OK;
    return hip_status(launch_check_recip(lo, count, d_mismatches, static_cast<hipStream_t>(stream)));
}

dq_status dq_check_round_half_up(uint32_t lo, uint32_t count, unsigned long long *d_mismatches,
                                 void *stream) {
    if (!d_mismatches) return DQ_ENULL;
    if ((uint64_t)lo + count > 0x100000000ull) return DQ_EINVAL;
    if (count == 0) return DQ_OK;
    return hip_status(launch_check_rpi(lo, count, d_mismatches, static_cast<hipStream_t>(stream)));
}

dq_status dq_probe_stream(const void *src, size_t src_bytes, void *dst, size_t dst_bytes,
                          int32_t reads_per_write, void *stream) {
    if (!src || !dst) return DQ_ENULL;
    const int32_t R = reads_per_write;
    if (R != 0 && R != 1 && R != 2 && R != 4 && R != 8) return DQ_EINVAL;
    const size_t tile = 1024 * (size_t)(R == 0 ? 1 : R);
    if (src_bytes == 0 || src_bytes % tile != 0 || !aligned(src, 16) || !aligned(dst, 16))
        return DQ_EINVAL;
    const size_t need = R == 0 ? (size_t)probe_stream_sink_bytes() : src_bytes / (size_t)R;
    if (dst_bytes < need) return DQ_EINVAL;
    return hip_status(launch_probe_stream(src, (int64_t)(src_bytes / tile), R, dst,
                                          static_cast<hipStream_t>(stream)));
}

dq_status dq_get_info(dq_plan *p, dq_info *out, void *stream) {
    if (!p || !out) return DQ_ENULL;
    if (!p->ws) return DQ_EWORKSPACE;
    if (!p->allocated) return DQ_ESTATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Ctrl c;
    if (hipMemcpyAsync(&c, ctrl_of(p), sizeof(Ctrl), hipMemcpyDeviceToHost, s) != hipSuccess)
        return DQ_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DQ_EHIP;
    std::memset(out, 0, sizeof(*out));
    out->rho_bits = c.rho_bits;
    std::memcpy(&out->rho, &c.rho_bits, 4);
    const bool wide = p->qmax == 16;
    out->t12 = (wide ? 21845.0f : 85.0f) * out->rho;
    out->t24 = (wide ? 139808.0f : 544.0f) * out->rho;
    out->t48 = (wide ? 4210688.0f : 16384.0f) * out->rho;
    out->t816 = wide ? 2147483648.0f * out->rho : INFINITY;
    out->budget_bits = p->budget_bits;
    int64_t used = 0;
    for (int k = 0; k < kClasses; k++) {
        const int64_t ck = (int64_t)c.class_counts[k];
        if (k < 3) out->class_counts[k] = ck;
        p->host_counts[k] = ck;
        used += ck * (2 << k);
    }
    out->class_count16 = (int64_t)c.class_counts[3];
    out->used_bits = used;
    out->achieved_bits = (double)used / (double)p->J;
    out->nonfinite = c.nonfinite ? 1 : 0;
    return out->nonfinite ? DQ_ENONFINITE : DQ_OK;
}

dq_status dq_timing_read(dq_plan *p, dq_timing *out) {
    if (!p || !out) return DQ_ENULL;
    // exact per-part super-group counts need the class counts of this round
    Ctrl c;
    std::memset(&c, 0, sizeof(c));
    if (p->ws && p->allocated && !p->launches.empty()) {
        if (hipEventSynchronize(p->launches.back().e1) != hipSuccess) return DQ_EHIP;
        if (hipMemcpy(&c, ctrl_of(p), sizeof(Ctrl), hipMemcpyDeviceToHost) != hipSuccess)
            return DQ_EHIP;
    }
    for (auto &L : p->launches) {
        float ms = 0.0f;
        if (hipEventSynchronize(L.e1) != hipSuccess) return DQ_EHIP;
        if (hipEventElapsedTime(&ms, L.e0, L.e1) != hipSuccess) return DQ_EHIP;
        p->acc.ms[L.kind] += ms;
        p->acc.launches[L.kind] += 1;
        int64_t sg = 0;
        if (L.m == 0) {
            sg = p->J;
        } else {
            for (int k = 0; k < kClasses; k++) {
                const int64_t Ck = (int64_t)c.class_counts[k];
                sg += (L.part + 1) * Ck / L.m - L.part * Ck / L.m;
            }
        }
        p->acc.coords[L.kind] += sg * kSG;
        p->pool.push_back(L.e0);
        p->pool.push_back(L.e1);
    }
    p->launches.clear();
    *out = p->acc;
    std::memset(&p->acc, 0, sizeof(p->acc));
    return DQ_OK;
}

}  // extern "C"

// ---- MX reference codecs in the same schedule (quality report) ----------------

namespace {

// part c of m of the ORIGINAL order: coordinates [lo, lo + n)
void mx_part(const dq_plan *p, int64_t m, int64_t c, int64_t &lo, int64_t &n) {
    lo = c * p->J / m * kSG;
    n = (c + 1) * p->J / m * kSG - lo;
}

size_t mx_region_max(const dq_plan *p, int64_t m) {
    const size_t coords = (size_t)(p->J / m + 1) * kSG;
    return align_up(coords + coords / 32, kAlign);
}

dq_status mx_launch(dq_plan *p, int fmt, int mode, int local, const void *grad, const uint8_t *in,
                    const uint8_t *own, int64_t in_m, int64_t in_c, uint8_t *out, float *out_f32,
                    int64_t m, int64_t c, hipStream_t s) {
    MxArgs a;
    std::memset(&a, 0, sizeof(a));
    a.grad = grad;
    a.in = in;
    a.own = own;
    mx_part(p, in_m, in_c, a.in_lo, a.in_n);
    a.out = out;
    a.out_f32 = out_f32;
    mx_part(p, m, c, a.lo, a.n);
    a.mode = mode;
    Launch L;
    hipError_t e = timed_begin(p, DQ_K_MXFP8, 0, 0, s, L);
    if (e == hipSuccess && a.n > 0) e = launch_mx(a, fmt, local, s);
    if (e == hipSuccess) e = timed_end(p, L, s);
    return hip_status(e);
}

}  // namespace

extern "C" {

size_t dq_mxfp8_arena_bytes(const dq_plan *p) {
    if (!p) return 0;
    if (p->n == 1) return mx_region_max(p, 1);
    if (p->topo == DQ_RING) return 2 * (size_t)p->n * mx_region_max(p, p->n);
    size_t per_w = mx_region_max(p, 2);
    for (int s = 1; s <= p->L; s++) per_w += mx_region_max(p, (int64_t)1 << s);
    return (size_t)p->n * per_w;
}

size_t dq_mx_arena_bytes(const dq_plan *p) { return dq_mxfp8_arena_bytes(p); }

dq_status dq_mx_allreduce(dq_plan *p, int32_t format, const void *const *grads, int32_t kind, void *arena,
                          size_t arena_bytes, float *out, void *stream) {
    if (!p || !grads || !arena || !out) return DQ_ENULL;
    if (format < DQ_MX_FP8_E4M3 || format > DQ_MX_FP4_E2M1) return DQ_EINVAL;
    const int f = format;
    if (kind != DQ_BF16 && kind != DQ_F32) return DQ_EINVAL;
    if (arena_bytes < dq_mxfp8_arena_bytes(p) || !aligned(arena, kAlign)) return DQ_EWORKSPACE;
    for (int w = 0; w < p->n; w++)
        if (!grads[w] || !aligned(grads[w], 16)) return DQ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *A = static_cast<uint8_t *>(arena);
    const int n = p->n, lk = local_of_kind(kind);
    dq_status st;
    if (n == 1) {
        if ((st = mx_launch(p, f, kCompress, lk, grads[0], nullptr, nullptr, 1, 0, A, nullptr, 1, 0, s)))
            return st;
        return mx_launch(p, f, kFinalize, kLocalNone, nullptr, A, nullptr, 1, 0, nullptr, out, 1, 0, s);
    }
    if (p->topo == DQ_RING) {
        const size_t R = mx_region_max(p, n);
        auto slot = [&](int w, int t) { return A + ((size_t)(t & 1) * n + w) * R; };
        for (int w = 0; w < n; w++)
            if ((st = mx_launch(p, f, kCompress, lk, grads[w], nullptr, nullptr, n, w, slot(w, 0), nullptr,
                                n, w, s)))
                return st;
        for (int t = 1; t < n; t++)
            for (int w = 0; w < n; w++) {
                const int64_t c = ((int64_t)w - t % n + n) % n;
                if ((st = mx_launch(p, f, kHop, lk, grads[w], slot((w - 1 + n) % n, t - 1), nullptr, n, c,
                                    slot(w, t), nullptr, n, c, s)))
                    return st;
            }
        for (int w = 0; w < n; w++)
            if ((st = mx_launch(p, f, kFinalize, kLocalNone, nullptr, slot(w, n - 1), nullptr, n, (w + 1) % n,
                                nullptr, out, n, (w + 1) % n, s)))
                return st;
        return DQ_OK;
    }
    const int L = p->L;
    std::vector<size_t> off;    // per worker: compress slot, then one slot per level
    size_t total = 0;
    for (int w = 0; w < n; w++) {
        off.push_back(total);
        total += mx_region_max(p, 2);
        for (int l = 1; l <= L; l++) {
            off.push_back(total);
            total += mx_region_max(p, (int64_t)1 << l);
        }
    }
    auto slot = [&](int w, int l) { return A + off[(size_t)w * (L + 1) + l]; };   // l = 0: compress
    for (int w = 0; w < n; w++) {
        const int64_t c = ((int64_t)w >> (L - 1)) ^ 1;
        if ((st = mx_launch(p, f, kCompress, lk, grads[w], nullptr, nullptr, 2, c, slot(w, 0), nullptr, 2, c, s)))
            return st;
    }
    for (int l = 1; l <= L; l++)
        for (int w = 0; w < n; w++) {
            const int partner = w ^ (n >> l);
            const int64_t m = (int64_t)1 << l, c = (int64_t)w >> (L - l);
            if (l == 1) {
                if ((st = mx_launch(p, f, kHop, lk, grads[w], slot(partner, 0), nullptr, m, c, slot(w, 1),
                                    nullptr, m, c, s)))
                    return st;
            } else {
                // partner's and own level l-1 regions cover part c >> 1 of m / 2
                if ((st = mx_launch(p, f, kHop, kLocalPacked, nullptr, slot(partner, l - 1), slot(w, l - 1),
                                    m / 2, c >> 1, slot(w, l), nullptr, m, c, s)))
                    return st;
            }
        }
    for (int w = 0; w < n; w++)
        if ((st = mx_launch(p, f, kFinalize, kLocalNone, nullptr, slot(w, L), nullptr, n, w, nullptr, out, n, w, s)))
            return st;
    return DQ_OK;
}

dq_status dq_mxfp8_allreduce(dq_plan *p, const void *const *grads, int32_t kind, void *arena,
                             size_t arena_bytes, float *out, void *stream) {
    return dq_mx_allreduce(p, DQ_MX_FP8_E4M3, grads, kind, arena, arena_bytes, out, stream);
}

}  // extern "C"
