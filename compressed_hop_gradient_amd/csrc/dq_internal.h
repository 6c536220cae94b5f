// dq_internal.h -- declarations shared by the C ABI (dq_api.cpp) and the HIP
// kernels (dq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int kSG = 256;          // coordinates per super-group
constexpr int kGroup = 16;        // coordinates per group (one lane owns one group)
constexpr int kGroupsPerSG = 16;
constexpr int kSGPerBlock = 16;   // finalize: 4 waves x 4 super-groups
constexpr int kReorderSGPerBlock = 1024;  // allocation/reorder: 256 threads x 4
// The scalar rho is found by an exact radix search on its fp32 bit pattern:
// pass p fixes the bits above kRadixShift[p] by testing up to 256 candidates.
constexpr int kRadixPasses = 4;
constexpr int kRadixCand = 256;

// control block at the head of the workspace's control area
struct Ctrl {
    unsigned int hist4[kRadixCand + 1];       // per-pass histograms (see k_alloc_count)
    unsigned int hist8[kRadixCand + 1];
    unsigned int hist16[kRadixCand + 1];      // (the 16-bit class)
    unsigned long long class_counts[4];       // super-groups at 2, 4, 8 (and 16) bits
    uint32_t prefix;                          // bits of rho fixed so far
    uint32_t done;                            // 1 once rho is known
    uint32_t rho_bits;
    int32_t nonfinite;
};

// kPartial: a hop whose output (the child a worker keeps, own-fp32 variant)
// is the fp32 partial sum itself instead of a packed region.
// kHopFinal: the last hop of a schedule; writes its region and also the
// decoded final sum of its part (what finalize would compute from it).
enum Mode { kCompress = 0, kHop = 1, kFinalize = 2, kPartial = 3, kHopFinal = 4 };

// Width classes: 2, 4, 8 bits, and 16 when a plan takes the 16-bit class
// (DQ_OPT_MAX_WIDTH); without it the fourth class is empty everywhere.
constexpr int kClasses = 4;

// Layout of one part (m, c) of the bitwidth-sorted stream and of its region;
// computed once per round on the device (k_part_table) for every part the
// schedule uses.
struct PartInfo {
    int64_t lo[kClasses];     // first stream position of each class in the part
    int64_t cnt[kClasses];    // super-groups of each class
    int64_t pre[kClasses];    // part-local index of each class's first super-group
    int64_t N;                // super-groups in the part
    int64_t offc[kClasses];   // region byte offset of each class's codes
    int64_t offs;      // region byte offset of the fp32 scale units
    int64_t offg;      // region byte offset of the UINT8 group codes
    int64_t bytes;     // region size
};
// kLocalPartial: the worker's own fp32 partial sums, 256 floats per
// super-group in the input part's order
enum Local { kLocalNone = 0, kLocalBF16 = 1, kLocalF32 = 2, kLocalPacked = 3, kLocalPartial = 4 };

// arguments of one codec launch (compress / hop / finalize).  A launch covers
// the super-groups of one output part (m_out, part_out); the input regions
// (incoming and own packed) hold the part (m_in, part_in) that contains it
// (the same part, or its parent when a hop writes the two children).
struct DeviceTables;
struct Pair;

struct CodecArgs {
    const DeviceTables *tab;                 // level and bucket tables (plan workspace)
    const PartInfo *part_out;                // device part table entries
    const PartInfo *part_in;
    const int32_t *perm;
    const float *mu_stream;
    const void *grad;                        // local gradient (bf16 / f32)
    const uint8_t *region_in;                // incoming region (hop, finalize)
    const uint8_t *region_own;               // own packed region (butterfly level >= 2)
    const float *partial_in;                 // own fp32 partial sums (own-fp32 variant)
    float *partial_out;                      // kPartial output: fp32 partial sums of the part
    uint8_t *out;                            // output region of (m_out, part_out)
    // a hop that writes both children of its part in one launch: the second
    // child's part entry and region (null: one output); blocks [0, split)
    // write the first child, the others the second
    const PartInfo *part_out2;
    uint8_t *out2;
    uint32_t split;
    float *out_f32;                          // finalize output, original order
    float n_workers_f;                       // finalize: fl(n * mu)
    uint32_t key0, key1, round, tag, stagger;
    // the 16-bit class: its 65,536 levels and weights (workspace), and the
    // level shape for the first guess of the interval search
    const float *L16, *W16;
    const Pair *LW16;             // (L16[r], W16[r]) pairs
    float eps;
};

struct StatsArgs {
    const void *grad;
    int64_t J;
    float *sum, *sumsq;
    int32_t first;
    int32_t *nonfinite;
};

enum AllocMode { kAllocThreshold = 0, kAllocMeanCorrected = 1, kAllocUniform = 2 };

struct AllocArgs {
    const float *sumsq;
    const float *sum;   // mean-corrected key: mu = fl(sum / denom)
    float denom;        // fl(256 n)
    int32_t mode;       // AllocMode
    int32_t uniform_k;  // class of every super-group under kAllocUniform
    int32_t wide;       // 1: widths {2,4,8,16} (thresholds 139808, 4210688, 2^31 rho)
    int64_t J;
    long long budget;   // floor(B * J)
    Ctrl *ctrl;
    uint8_t *widths;
    int32_t *blkcnt;    // [kClasses][nblk]
    int64_t nblk;
};

struct ReorderArgs {
    const uint8_t *widths;
    const float *sum;
    float denom;        // fl(256 n)
    int64_t J;
    const Ctrl *ctrl;
    int32_t *blkcnt;    // [kClasses][nblk] counts in, offsets out (scan)
    int64_t nblk;
    int32_t *perm, *inv;
    float *mu_stream;
};

// MX reference codecs (quality report only).  Regions hold one element code
// byte per coordinate of the part, then one E8M0 scale byte per 32 coordinates.
enum MxFormat { kMxE4M3 = 0, kMxE3M2 = 1, kMxE2M3 = 2, kMxE2M1 = 3 };
struct MxArgs {
    const void *grad;          // local gradient (original order), or nullptr
    int32_t grad_f32;
    const uint8_t *in;         // incoming region (hop / finalize), part [in_lo, in_lo + in_n)
    const uint8_t *own;        // own region (butterfly level >= 2), same part as `in`
    int64_t in_lo, in_n;
    uint8_t *out;              // output region, part [lo, lo + n)
    float *out_f32;            // finalize output (original order)
    int64_t lo, n;
    int32_t mode;              // kCompress / kHop / kFinalize
};

// launchers (dq_kernels.hip); each returns the hipError_t of its launch
hipError_t launch_zero(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_build_tables(DeviceTables *t, double eps, hipStream_t s);
hipError_t launch_stats(const StatsArgs &a, int f32, hipStream_t s);
hipError_t launch_alloc_pass(const AllocArgs &a, int pass, hipStream_t s);
hipError_t launch_alloc_final(const AllocArgs &a, hipStream_t s);
hipError_t launch_reorder(const ReorderArgs &a, hipStream_t s);
// wide: the plan has the 16-bit class (kernels with its code path)
hipError_t launch_codec(const CodecArgs &a, int mode, int local, int64_t max_sg, bool wide, hipStream_t s);
// the 16-bit class's level and weight tables (65,536 each) for level shape eps
hipError_t launch_build_tables16(float *L16, float *W16, Pair *LW16, double eps, hipStream_t s);
// part table for the schedule of n workers: ring entry c = part c of n;
// butterfly entry (m - 2) + c = part c of m for m = 2, 4, .., n; n = 1: one entry
int32_t part_table_entries(int32_t n, int32_t topology);
int32_t part_table_index(int32_t n, int32_t topology, int64_t m, int64_t c);
hipError_t launch_part_table(const unsigned long long *class_counts, int32_t n, int32_t topology,
                             PartInfo *table, hipStream_t s);
hipError_t launch_mx(const MxArgs &a, int fmt, int local, hipStream_t s);
hipError_t launch_check_recip(uint32_t lo, uint32_t n, unsigned long long *count, hipStream_t s);
hipError_t launch_check_rpi(uint32_t lo, uint32_t n, unsigned long long *count, hipStream_t s);
// static device scratch (dq_allreduce_noalloc): its device address on the
// current device (looked up once per device)
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
hipError_t scratch_address(void **ptr);
// streaming probe: `tiles` tiles of reads_per_write x 1 KB read (0: read only)
hipError_t launch_probe_stream(const void *src, int64_t tiles, int reads_per_write, void *dst, hipStream_t s);
int64_t probe_stream_sink_bytes();

}  // namespace dq
