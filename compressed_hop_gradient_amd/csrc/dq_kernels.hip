// dq_kernels.hip -- HIP kernels of the DynamiQ hot path for gfx950 (CDNA4).
//
// Everything here is HBM-streaming integer/fp32 work: no stage is a dense
// contraction, so nothing uses MFMA.  Kernels are written for 64-lane
// wavefronts:
//   * stats: 16 lanes per super-group (SG), each lane two 128-bit loads of 8
//     bf16 (partials l and l + 16); 8 sequential adds per partial, then the
//     tree over the 32 partials (one in-lane step, four DPP row shifts); one
//     resident block per CU parks its results in LDS and writes the running
//     sums in one burst after its share has been read;
//   * codec (compress / hop / fused last hop / finalize): one 16-lane DPP row
//     per SG, one lane per group of 16 coordinates, so group scales are
//     per-lane scalars and the SG maximum is a 4-step DPP row reduction;
//     128-bit loads of codes and of the local bf16 gradient; level tables
//     copied into LDS once per block from an image kept in the workspace;
//   * allocation: integer counts only (order-free), a 4-pass radix search on
//     the fp32 bit pattern of the scalar with no host round trip;
//   * reorder: per-block counts, one scan block, stable per-block scatter.
//
// Numerics follow the readings shared with the CPU oracle: fp32, round to
// nearest even, no contraction (built with -ffp-contract=off), correctly
// rounded division.
#include "dq_internal.h"
#include "dq_tables.h"

namespace dq {

// Streaming 16-byte loads (read once, no reuse): non-temporal, so they do not
// displace other data from the caches (about 4% on the stats pass).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load_u4(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 stream_load_f4(const void *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

static int grid_for(int64_t items, int64_t per_block, int64_t cap);
static int64_t device_cus();


// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                      0xF, 0xF, false));
}

// x from another lane of the row; 0 where no lane is read (never, for the
// in-row permutations used here).  0 is the identity of an unsigned max, which
// lets the compiler fold the move into the max as a DPP operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// maximum over the 16 lanes of a DPP row (all lanes get the result).  The
// inputs are magnitudes (non-negative floats), whose order is their bit
// patterns' integer order, so an integer max serves and folds into DPP.
__device__ __forceinline__ float row_max16(float x) {
    uint32_t u = __float_as_uint(x);
    u = max(u, dpp_mov_u<0xB1>(u));   // quad_perm [1,0,3,2]
    u = max(u, dpp_mov_u<0x4E>(u));   // quad_perm [2,3,0,1]
    u = max(u, dpp_mov_u<0x141>(u));  // row_half_mirror
    u = max(u, dpp_mov_u<0x140>(u));  // row_mirror
    return __uint_as_float(u);
}

// Philox4x32 with 10 rounds (Salmon et al., SC'11): per round two 32x32->64
// products of the even words; high halves xored with the odd words and the key;
// words permuted; key advanced by the Weyl constants between rounds.  Each
// product is one 64-bit multiply (v_mad_u64_u32) and each three-way xor one
// v_bitop3_b32 (truth table 0x96), 1.8x faster on gfx950 than separate
// high/low multiplies and two-input xors.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ void philox4x32_10(uint32_t &x0, uint32_t &x1, uint32_t &x2,
                                              uint32_t &x3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
            // keep the round keys as two scalar registers bumped per round
            // (scalar adds, off the vector pipe): left to itself the compiler
            // holds all twenty round keys for the whole kernel, which pushes
            // the codec kernels past the SGPR file and spills into VGPR lanes
            // read back with v_readlane inside the loop
            asm volatile("" : "+s"(k0), "+s"(k1));
        }
        const uint64_t pa = (uint64_t)0xD2511F53u * x0;
        const uint64_t pb = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t y0 = xor3((uint32_t)(pb >> 32), x1, k0);
        const uint32_t y2 = xor3((uint32_t)(pa >> 32), x3, k1);
        x0 = y0;
        x1 = (uint32_t)pb;
        x2 = y2;
        x3 = (uint32_t)pa;
    }
}

// Scale unit of a super-group: fl(A/255), raised to the next float while
// fl(255 s) < A.  One raise always suffices: over every non-negative finite
// fp32 A, fl(255 s) < A after one raise never happens (exhaustive CPU check),
// so the loop of the definition is a single guarded step.
__device__ __forceinline__ float scale_unit(float A) {
    // fl(A / 255) by a product and two FMAs: equal to the correctly rounded
    // quotient for every non-negative finite A (exhaustive CPU check)
    constexpr float R = 1.0f / 255.0f;
    const float y = A * R;
    const float rem = __builtin_fmaf(-y, 255.0f, A);
    float s = __builtin_fmaf(rem, R, y);
    if (255.0f * s < A) s = __uint_as_float(__float_as_uint(s) + 1u);
    return s;
}

// fl(1/x), correctly rounded.  For x in [2^-126, 2^126) one Newton step on the
// hardware reciprocal, e = fma(-x, r, 1) and fma(e, r, r), gives exactly the
// IEEE quotient (checked on the hardware for every fp32 in the range by
// dq_check_reciprocal); outside it, and only in the lanes that need it, the
// IEEE division.
__device__ __forceinline__ float recip_rn(float x) {
    float y;
    if (__builtin_expect(x >= 1.1754943508222875e-38f && x < 8.507059173023462e37f, 1)) {
        const float r = __builtin_amdgcn_rcpf(x);
        const float e = __builtin_fmaf(-x, r, 1.0f);
        y = __builtin_fmaf(e, r, r);
    } else {
        y = 1.0f / x;
    }
    return y;
}

// floor(x + 0.5) as an integer, exactly, for every finite fp32 x: the
// hardware's round-half-up conversion (values beyond the int range saturate,
// and so does NaN, by its sign bit; checked over every bit pattern by
// dq_check_round_half_up).  The rounding decision d + 0.5 <= P of a 16-bit
// dither d then reads d < round_half_up(P): one conversion and one integer
// compare, where the float form needs a conversion, an add and a compare.
// P is finite for every finite input (an overflowing 1/sigma is handled
// before the search); a NaN P comes only from non-finite gradients, which
// the statistics flag, and still gives a code inside the class.
__device__ __forceinline__ int round_half_up(float x) {
    int n;
    asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(n) : "v"(x));
    return n;
}

// Smallest c in [0, 255] with fl(c * s) >= a (exists because fl(255 s) >= A >= a).
// For a normal s the estimate ceil(a * rcp(s)) (rcp within 1 ulp) is within one
// of the answer, so one checked step down or up settles it; subnormal s (scale
// units below 2^-126) take the general search.
__device__ __forceinline__ int group_code(float a, float s) {
    if (s == 0.0f) return 0;
    if (s < 1.1754943508222875e-38f) {
        int c = 0;
        while (c < 255 && (float)c * s < a) c++;
        return c;
    }
    int c = (int)ceilf(fminf(a * __builtin_amdgcn_rcpf(s), 255.0f));
    c = min(max(c, 0), 255);
    const bool down = c > 0 && (float)(c - 1) * s >= a;
    const bool up = c < 255 && (float)c * s < a;
    return down ? c - 1 : (up ? c + 1 : c);
}

// Interval search over NL = 16 or 256 levels: r = largest r <= NL-2 with
// L[r] <= v.  The linear bucket NB/2 + rne(v M) of v, M = NB/2 - 1, holds at
// most one level boundary, so its table entry est is r or r - 1; one compare
// with the next level settles it, and the pair (L[r], W[r]) is read at r.
// The bucket is one FMA on the subnormal grid, where a float's bits are its
// value in units of 2^-149: fl(v (M 2^-149) + (NB/2) 2^-149) rounds
// v M + NB/2 to an integer (ties to even) and its bits are that integer, the
// byte offset of the entry.  The encoder's |v| <= 1 + 2^-22 (1/sigma rounded
// once, |y| <= sigma) keeps it in [1, NB - 1]; the FMA's clamp to [0, 1]
// turns the NaN of a non-finite gradient into bucket 0, so no input reads
// outside the table.
template <int NL>
__device__ __forceinline__ uint32_t search_levels(float v, const uint8_t *est_tab, const float *cl,
                                                  const Pair *lw, float &Lr, float &Wr) {
    constexpr int NB = bucket_count(NL);
    constexpr float kM = __builtin_bit_cast(float, (uint32_t)(NB / 2 - 1));
    constexpr float kHalf = __builtin_bit_cast(float, (uint32_t)(NB / 2));
    const float x = __builtin_amdgcn_fmed3f(__builtin_fmaf(v, kM, kHalf), 0.0f, 1.0f);
    const uint32_t est = est_tab[__float_as_uint(x)];
    uint32_t r = est + (v >= cl[est + 1] ? 1u : 0u);
    // keep r opaque: the code is then formed as r + (round up), one carry-add,
    // rather than re-derived from est and both comparisons
    asm("" : "+v"(r));
    const Pair p = lw[r];
    Lr = p.l;
    Wr = p.w;
    return r;
}

// 16-bit search over the 65,536 levels in the workspace: r = the largest
// r <= 65534 with L[r] <= v (v already clamped to [-1, 1], so L[0] = -1 <= v).
// First guess r0 from the closed form of the levels, |v| = t (eps + (1 - eps) t)
// and u = (2 r + 1 - Q) / (Q - 1), i.e. r = floor((u + 1) (Q - 1) / 2), with
// the hardware square root and a reciprocal (off by at most one level in
// practice).  Then, without a loop: with r0 clamped to [1, 65533], the pairs
// r0 - 1, r0, r0 + 1 and the level r0 + 2 (independent loads) decide
// r = r0 - 1 + [v >= L[r0]] + [v >= L[r0 + 1]] whenever L[r0 - 1] <= v <
// L[r0 + 2] (or r0 + 2 is the last level, which is no boundary); otherwise a
// bisection over all levels.
__device__ __forceinline__ uint32_t search_levels16(float v, const float *L, const Pair *LW, float eps,
                                                    float &Lr, float &Wr) {
    const float av = fabsf(v), ce = 1.0f - eps;
    const float t = ce > 0.0f
        ? (__builtin_amdgcn_sqrtf(eps * eps + 4.0f * ce * av) - eps) * __builtin_amdgcn_rcpf(2.0f * ce)
        : av;
    const float u = v < 0.0f ? -t : t;
    int r0 = (int)floorf((u + 1.0f) * 32767.5f);
    r0 = min(max(r0, 1), 65533);
    // The window's answer and its test are formed without a branch, so that
    // all four loads are needed up front and go out together (one memory
    // round trip); with a short-circuit test the compiler sank them into
    // the branches and waited for each in turn.
    const Pair p0 = LW[r0 - 1], p1 = LW[r0], p2 = LW[r0 + 1];
    const float l3 = L[r0 + 2];
    const int k = (v >= p1.l ? 1 : 0) + (v >= p2.l ? 1 : 0);
    float Lc = k == 0 ? p0.l : (k == 1 ? p1.l : p2.l);
    float Wc = k == 0 ? p0.w : (k == 1 ? p1.w : p2.w);
    int r = r0 - 1 + k;
    const bool in_window = (p0.l <= v) & ((v < l3) | (r0 == 65533));
    if (__builtin_expect(!in_window, 0)) {
        int lo = 0, hi = 65534;
        while (lo < hi) {
            const int mid = lo + (hi - lo + 1) / 2;
            if (L[mid] <= v) lo = mid;
            else hi = mid - 1;
        }
        r = lo;
        Lc = LW[lo].l;
        Wc = LW[lo].w;
    }
    Lr = Lc;
    Wr = Wc;
    return (uint32_t)r;
}

// 2-bit search: two compares against the inner levels c1 = L[1], c2 = L[2]
__device__ __forceinline__ uint32_t search_levels2(float v, float c1, float c2, const Pair *lw,
                                                   float &Lr, float &Wr) {
    uint32_t r = (v >= c1 ? 1u : 0u) + (v >= c2 ? 1u : 0u);
    asm("" : "+v"(r));
    const Pair p = lw[r];
    Lr = p.l;
    Wr = p.w;
    return r;
}

// ---------------------------------------------------------------------------
// parts and regions
// ---------------------------------------------------------------------------

__device__ __forceinline__ void part_info(const unsigned long long *C, int64_t m, int64_t c,
                                          PartInfo &p) {
    int64_t base = 0, off = 0;
    p.N = 0;
#pragma unroll
    for (int k = 0; k < kClasses; k++) {
        const int64_t Ck = (int64_t)C[k];
        const int64_t a = c * Ck / m, b = (c + 1) * Ck / m;
        p.lo[k] = base + a;
        p.cnt[k] = b - a;
        p.pre[k] = p.N;
        p.N += b - a;
        base += Ck;
    }
#pragma unroll
    for (int k = 0; k < kClasses; k++) {
        p.offc[k] = off;
        off += p.cnt[k] * 32 * (2 << k);
    }
    p.offs = off;
    off += 4 * p.N;
    off = (off + 15) & ~int64_t(15);
    p.offg = off;
    off += 16 * p.N;
    p.bytes = off;
}


// level of a code; the 16-bit class reads its 65,536 levels from the
// workspace (L2-resident), the others from the block's LDS tables
template <int B>
__device__ __forceinline__ float level_of(const SharedTables &T, const float *L16, uint32_t code) {
    if constexpr (B == 2) return T.dec2[code];
    else if constexpr (B == 4) return T.dec4[code];
    else if constexpr (B == 8) return T.dec8[code];
    else return L16[code];
}

// x[i] = fl(sigma * L[code i]) for the 16 codes of one group.  2- and 4-bit
// codes are looked up a byte at a time (four or two levels per LDS read).
template <int B>
__device__ __forceinline__ void decode_codes(const uint32_t (&w)[B / 2], float sigma, const SharedTables &T,
                                             const float *L16, float (&x)[16]) {
    if constexpr (B == 2) {
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const f32x4_t l = *reinterpret_cast<const f32x4_t *>(T.quad2[(w[0] >> (8 * k)) & 0xFFu]);
            x[4 * k] = sigma * l.x;
            x[4 * k + 1] = sigma * l.y;
            x[4 * k + 2] = sigma * l.z;
            x[4 * k + 3] = sigma * l.w;
        }
    } else if constexpr (B == 4) {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float2 l = *reinterpret_cast<const float2 *>(T.pair4[(w[k >> 2] >> (8 * (k & 3))) & 0xFFu]);
            x[2 * k] = sigma * l.x;
            x[2 * k + 1] = sigma * l.y;
        }
    } else if constexpr (B == 8) {
#pragma unroll
        for (int i = 0; i < 16; i++) x[i] = sigma * T.dec8[(w[i >> 2] >> (8 * (i & 3))) & 0xFFu];
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) x[i] = sigma * L16[(w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu];
    }
}

// load / store the 2B bytes of one group's codes (B = bits per code)
template <int B>
__device__ __forceinline__ void load_codes(const uint8_t *p, uint32_t (&w)[B / 2]) {
    if constexpr (B == 16) {
        const uint4 v0 = reinterpret_cast<const uint4 *>(p)[0], v1 = reinterpret_cast<const uint4 *>(p)[1];
        w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
        w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    } else if constexpr (B == 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (B == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

template <int B>
__device__ __forceinline__ void store_codes(uint8_t *p, const uint32_t (&w)[B / 2]) {
    if constexpr (B == 16) {
        reinterpret_cast<uint4 *>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4 *>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else if constexpr (B == 8) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (B == 4) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        *reinterpret_cast<uint32_t *>(p) = w[0];
    }
}

// The stream positions and part-local offsets of a part's classes as 32-bit
// values (a part holds fewer than 2^31 super-groups), so that a launch keeps
// a dozen scalar registers of layout instead of the whole 64-bit PartInfo.
struct PartU32 {
    uint32_t lo[kClasses];    // first stream position of each class
    uint32_t pre[kClasses];   // part-local index of each class's first super-group
};

__device__ __forceinline__ PartU32 part_u32(const PartInfo &P) {
    PartU32 q;
#pragma unroll
    for (int k = 0; k < kClasses; k++) {
        q.lo[k] = (uint32_t)P.lo[k];
        q.pre[k] = (uint32_t)P.pre[k];
    }
    return q;
}

// Region pointers of one part, split by class (uniform over a launch).  Offsets
// added to them are 32-bit: the host keeps every region below 4 GB.
struct RegionBase {
    const uint8_t *codes[kClasses];   // codes of class k
    const uint8_t *s;          // fp32 scale units
    const uint8_t *g;          // UINT8 group codes
};

__device__ __forceinline__ RegionBase region_base(const uint8_t *r, const PartInfo &P) {
    RegionBase b;
    for (int k = 0; k < kClasses; k++) b.codes[k] = r + P.offc[k];
    b.s = r + P.offs;
    b.g = r + P.offg;
    return b;
}

// decode the group (lane g) of the super-group at part-local index t and
// class-local index idx of class K (B = bits per code)
template <int B, int K>
__device__ __forceinline__ void decode_group(const RegionBase &R, uint32_t t, uint32_t idx, int g,
                                             const SharedTables &T, const float *L16, float (&x)[16]) {
    uint32_t w[B / 2];
    load_codes<B>(R.codes[K] + (idx * (32u * B) + (uint32_t)g * (2u * B)), w);
    const float s = *reinterpret_cast<const float *>(R.s + 4u * t);
    const uint32_t c = R.g[16u * t + (uint32_t)g];
    const float sigma = (float)c * s;
    decode_codes<B>(w, sigma, T, L16, x);
}

// ---------------------------------------------------------------------------
// codec kernel: compress / hop / finalize on one part
// ---------------------------------------------------------------------------

// One super-group per 16-lane row, one group of 16 coordinates per lane.
// Q = bits per code of the super-group's class, K = the class index.
// Po = output part, Pi = input part (the same part or its parent); In / Own /
// Out are their regions.  t is the part-local index in the output part.
// Whether a kernel fetches its rows' next super-group's j and mean one
// iteration ahead, so that the gather of the local gradient at j waits for an
// LDS read instead of a global load.  The value is parked in LDS rather than
// carried in a register: vector-memory completions count in issue order, and
// a loop-carried load would make every iteration wait for the previous one's
// stores.  Measured: compress 6% faster; the hop kernels no faster (their
// incoming-region loads cover the latency) and some of them would spill.
template <int MODE, int LOCAL>
constexpr bool codec_ahead() { return LOCAL == kLocalBF16 && MODE == kCompress; }

template <int Q, int MODE, int LOCAL>
__device__ __forceinline__ void codec_sg(const CodecArgs &a, const PartU32 &Po, const PartU32 &Pi,
                                         const RegionBase &In, const RegionBase &Own,
                                         const RegionBase &Out, uint32_t t, uint32_t j, float mu,
                                         uint32_t pos_next, uint32_t *slot_j, float *slot_mu, int g,
                                         const SharedTables &T, float *stage_row) {
    constexpr int K = Q == 2 ? 0 : (Q == 4 ? 1 : (Q == 8 ? 2 : 3));
    const uint32_t idx = t - (uint32_t)Po.pre[K];        // index in the class, output part
    const uint32_t pos = (uint32_t)Po.lo[K] + idx;       // stream position
    const uint32_t idx_in = pos - (uint32_t)Pi.lo[K];    // index in the class, input part
    const uint32_t t_in = (uint32_t)Pi.pre[K] + idx_in;
    if constexpr (!codec_ahead<MODE, LOCAL>()) {
        j = (uint32_t)a.perm[pos];                       // original super-group
        mu = a.mu_stream[pos];
    }
    float y[16];

    if constexpr (MODE != kCompress) decode_group<Q, K>(In, t_in, idx_in, g, T, a.L16, y);

    if constexpr (LOCAL == kLocalBF16) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(a.grad) + ((uint64_t)j * kSG + (uint32_t)g * kGroup));
        const uint4 h0 = src[0], h1 = src[1];
        const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float e0 = bf16_lo(hw[i]) - mu, e1 = bf16_hi(hw[i]) - mu;
            if constexpr (MODE == kHop || MODE == kPartial || MODE == kHopFinal) {
                y[2 * i] = y[2 * i] + e0;
                y[2 * i + 1] = y[2 * i + 1] + e1;
            } else {
                y[2 * i] = e0;
                y[2 * i + 1] = e1;
            }
        }
    } else if constexpr (LOCAL == kLocalF32) {
        const float4 *src = reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.grad) + ((uint64_t)j * kSG + (uint32_t)g * kGroup));
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float4 f = src[v];
            const float e[4] = {f.x - mu, f.y - mu, f.z - mu, f.w - mu};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if constexpr (MODE == kHop || MODE == kPartial || MODE == kHopFinal) y[4 * v + i] = y[4 * v + i] + e[i];
                else y[4 * v + i] = e[i];
            }
        }
    } else if constexpr (LOCAL == kLocalPacked) {
        float own[16];
        decode_group<Q, K>(Own, t_in, idx_in, g, T, a.L16, own);
#pragma unroll
        for (int i = 0; i < 16; i++) y[i] = y[i] + own[i];
    } else if constexpr (LOCAL == kLocalPartial) {
        const float4 *src = reinterpret_cast<const float4 *>(a.partial_in + ((uint64_t)t_in * kSG + (uint32_t)g * kGroup));
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float4 f = src[v];
            y[4 * v] = y[4 * v] + f.x;
            y[4 * v + 1] = y[4 * v + 1] + f.y;
            y[4 * v + 2] = y[4 * v + 2] + f.z;
            y[4 * v + 3] = y[4 * v + 3] + f.w;
        }
    }

    // the next iteration's original index and mean, issued after this
    // super-group's loads and parked in LDS at the end
    uint32_t j_next = 0u;
    float mu_next = 0.0f;
    const bool ahead = codec_ahead<MODE, LOCAL>() && pos_next != 0xFFFFFFFFu;
    if (ahead) {
        j_next = (uint32_t)a.perm[pos_next];
        mu_next = a.mu_stream[pos_next];
    }
    auto park = [&]() {
        if (ahead && g == 0) {
            *slot_j = j_next;
            *slot_mu = mu_next;
        }
    };

    if constexpr (MODE == kPartial) {
        // the kept child of the own-fp32 variant: store y, no quantisation
        float4 *dst = reinterpret_cast<float4 *>(a.partial_out + ((uint64_t)t * kSG + (uint32_t)g * kGroup));
#pragma unroll
        for (int v = 0; v < 4; v++) dst[v] = make_float4(y[4 * v], y[4 * v + 1], y[4 * v + 2], y[4 * v + 3]);
        park();
        return;
    } else {

    // ---- encode ----
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(y[i]));
    const float A = row_max16(amax);
    const float s = scale_unit(A);
    const int c = group_code(amax, s);
    const float sigma = (float)c * s;
    float inv = sigma == 0.0f ? 0.0f : recip_rn(sigma);
    // 1/sigma overflows only for sigma below 2^-128 (a subnormal scale unit):
    // there v = y * inf would be +-inf, or NaN where y = 0.  Such a group takes
    // the definition literally, v = 0 where y = 0 and clamp(y * inv) elsewhere,
    // with the values put in place of y and inv = 1 for the loop below.
    if (__builtin_expect(!(inv <= 3.4028234663852886e38f), 0)) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float v = y[i] == 0.0f ? 0.0f : y[i] * inv;
            y[i] = v < -1.0f ? -1.0f : (v > 1.0f ? 1.0f : v);
        }
        inv = 1.0f;
    }
    float c1 = 0.0f, c2 = 0.0f;
    if constexpr (Q == 2) {
        c1 = T.dec2[1];
        c2 = T.dec2[2];
    }

    typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
    const ushort2_t stag = {(unsigned short)a.stagger, (unsigned short)a.stagger};
    uint32_t w[Q / 2];
#pragma unroll
    for (int i = 0; i < Q / 2; i++) w[i] = 0u;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        // 8 dithers of coordinates 8h..8h+7 of this group from one Philox call
        uint32_t x0 = 2u * g + h, x1 = j, x2 = a.round, x3 = a.tag;
        philox4x32_10(x0, x1, x2, x3, a.key0, a.key1);
        // add the worker's stagger to both 16-bit halves (mod 65536)
        uint32_t d[4] = {x0, x1, x2, x3};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            ushort2_t hv = __builtin_bit_cast(ushort2_t, d[q]);
            hv = hv + stag;
            d[q] = __builtin_bit_cast(uint32_t, hv);
        }
#pragma unroll
        for (int ii = 0; ii < 8; ii++) {
            const int i = 8 * h + ii;
            // The definition clamps v to [-1, 1].  With a finite 1/sigma,
            // |y| <= sigma makes v exceed 1 in magnitude by at most 2 ulps,
            // and there every step below gives the clamped value's code: the
            // bucket key and the capped interval (r = 2^q - 2 above +1, r = 0
            // below -1) are the same, P(+1) >= 65535.99 >= any d + 0.5 so
            // rounding up stays certain, and P < 0 below -1 keeps rounding
            // down certain.  The clamp is therefore left out (an overflowing
            // 1/sigma has been dealt with above).
            float v = y[i] * inv;
            float Lr, Wr;
            uint32_t r;
            if constexpr (Q == 2) r = search_levels2(v, c1, c2, T.lw2, Lr, Wr);
            else if constexpr (Q == 4) r = search_levels<16>(v, T.b4, T.cl4, T.lw4, Lr, Wr);
            else if constexpr (Q == 8) r = search_levels<256>(v, T.b8, T.cl8, T.lw8, Lr, Wr);
            else {
                // the clamp of the definition, kept for the 16-bit class
                v = v < -1.0f ? -1.0f : (v > 1.0f ? 1.0f : v);
                r = search_levels16(v, a.L16, a.LW16, a.eps, Lr, Wr);
            }
            // round up iff d + 0.5 <= P, i.e. d < floor(P + 0.5)
            const float P = (v - Lr) * Wr;
            const uint32_t dd = (ii & 1) ? (d[ii >> 1] >> 16) : (d[ii >> 1] & 0xFFFFu);
            const uint32_t code = r + ((int)dd < round_half_up(P) ? 1u : 0u);
            // pack as one shift-and-or per code, in coordinate order (kept
            // as a chain: the compiler's own tree of shifts and ORs takes
            // more instructions)
            if ((i * Q) % 32 == 0) w[(i * Q) / 32] = code;
            else w[(i * Q) / 32] |= code << ((i * Q) % 32);
            asm("" : "+v"(w[(i * Q) / 32]));
        }
    }

    uint8_t *out_codes = const_cast<uint8_t *>(Out.codes[K]);
    store_codes<Q>(out_codes + (idx * (32u * Q) + (uint32_t)g * (2u * Q)), w);
    const_cast<uint8_t *>(Out.g)[16u * t + (uint32_t)g] = (uint8_t)c;
    if (g == 0) *reinterpret_cast<float *>(const_cast<uint8_t *>(Out.s) + 4u * t) = s;

    if constexpr (MODE == kHopFinal) {
        // the decoded final sum of these coordinates, as finalize computes it
        // from the region just written: fl(fl(c s) L[code]) + fl(n mu).  The
        // row's 1 KB goes through LDS so that every store instruction writes
        // 256 contiguous bytes of the super-group (lane g: floats 64v + 4g).
        const float add = a.n_workers_f * mu;
        f32x4_t *stage = reinterpret_cast<f32x4_t *>(stage_row);
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float x[4];
#pragma unroll
            for (int ii = 0; ii < 4; ii++) {
                const int i = 4 * v + ii;
                const uint32_t code = (w[(i * Q) / 32] >> ((i * Q) % 32)) & ((1u << Q) - 1u);
                x[ii] = sigma * level_of<Q>(T, a.L16, code) + add;
            }
            stage[4 * g + v] = f32x4_t{x[0], x[1], x[2], x[3]};
        }
        // the row lives in one wave: a wavefront-scope fence orders the LDS
        // writes above before the other lanes' reads below
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        f32x4_t *dst = reinterpret_cast<f32x4_t *>(a.out_f32 + (uint64_t)j * kSG);
#pragma unroll
        for (int v = 0; v < 4; v++) __builtin_nontemporal_store(stage[16 * v + g], dst + 16 * v + g);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    park();
    }   // MODE != kPartial
}

// Block layout of each codec kernel, one super-group per 16-lane row.  The
// kernels with a bf16 local run 256-thread blocks (compress 8 per CU, the hop 7,
// the fused last hop 4 as its output staging and the tables allow: 33.5 KB of
// LDS per block); the others 512-thread blocks, 3 per CU.  Measured per kernel: with the packed local the larger
// blocks are 4.6% faster, with the bf16 local the smaller ones 1-4%.
// The instances with the 16-bit class (WIDE) hold six resident waves per
// SIMD (80 VGPRs), the fused last hop four (128): at the default kernels' seven
// or eight waves the wider codes and the 65,536-level search spill to scratch.
template <int MODE, int LOCAL, bool WIDE = false>
struct CodecShape {
    static constexpr bool kSmall = LOCAL == kLocalBF16 && MODE != kPartial;
    static constexpr int threads = kSmall ? 256 : 512;
    static constexpr int sg_per_block = threads / 16;
    static constexpr int blocks_per_cu = WIDE ? (kSmall ? (MODE == kHopFinal ? 4 : 6) : (MODE == kHopFinal ? 2 : 3))
                                              : (kSmall ? (MODE == kCompress ? 8 : (MODE == kHopFinal ? 4 : 7)) : 3);
    static constexpr int waves_per_simd = blocks_per_cu * threads / 256;   // 4 SIMDs per CU
};

// WIDE: the plan has the 16-bit class (a fourth class after the 8-bit one);
// the default kernels are built without its code path.
template <int MODE, int LOCAL, bool WIDE>
__global__ __launch_bounds__((CodecShape<MODE, LOCAL, WIDE>::threads))
__attribute__((amdgpu_waves_per_eu(CodecShape<MODE, LOCAL, WIDE>::waves_per_simd)))
void k_codec(CodecArgs a) {
    using Shape = CodecShape<MODE, LOCAL, WIDE>;
    constexpr int kThreads = Shape::threads, kSGPerBlock = Shape::sg_per_block;
    __shared__ SharedTables T;
    {
        // the block's copy of the tables: the workspace keeps their LDS image
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(&a.tab->lds);
        u32x4_t *dst = reinterpret_cast<u32x4_t *>(&T);
        for (int i = threadIdx.x; i < (int)(sizeof(SharedTables) / 16); i += blockDim.x) dst[i] = src[i];
    }
    __syncthreads();
    // A hop that writes both children of its part runs as one launch, so that
    // the two share one tail: blocks [0, split) write the first child and the
    // others the second.  The choice is per block, so the layouts stay in
    // scalar registers; a launch with one output has split = gridDim.x.
    const bool second = blockIdx.x >= a.split;
    const uint32_t blk = second ? blockIdx.x - a.split : blockIdx.x;
    const uint32_t nblk = second ? gridDim.x - a.split : a.split;
    // part layouts: uniform loads from the per-round part table
    const PartInfo Po = *(second ? a.part_out2 : a.part_out), Pi = *a.part_in;
    const RegionBase In = region_base(a.region_in, Pi), Own = region_base(a.region_own, Pi);
    const RegionBase Out = region_base(second ? a.out2 : a.out, Po);
    const PartU32 po = part_u32(Po), pi = part_u32(Pi);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, row = lane >> 4;
    const uint32_t N = (uint32_t)Po.N, pre1 = (uint32_t)Po.pre[1], pre2 = (uint32_t)Po.pre[2];
    const uint32_t pre3 = WIDE ? (uint32_t)Po.pre[3] : N;
    // the fused final hop stages each row's decoded super-group here
    constexpr int kStageRows = MODE == kHopFinal ? kThreads / 16 : 1;
    __shared__ __align__(16) float stage[kStageRows][kSG];
    float *stage_row = stage[MODE == kHopFinal ? threadIdx.x / 16 : 0];
    // per row: the original index and mean of the row's next super-group,
    // fetched during the current one (see codec_sg)
    __shared__ uint32_t next_j[kThreads / 16];
    __shared__ float next_mu[kThreads / 16];
    uint32_t *slot_j = &next_j[threadIdx.x / 16];
    float *slot_mu = &next_mu[threadIdx.x / 16];
    // (selects, not an index into Po's arrays: a runtime index would put the
    // part layout in scratch memory)
    const uint32_t lo0 = (uint32_t)Po.lo[0], lo1 = (uint32_t)Po.lo[1], lo2 = (uint32_t)Po.lo[2];
    const uint32_t lo3 = WIDE ? (uint32_t)Po.lo[3] : 0u;
    auto pos_of = [&](uint32_t tt) -> uint32_t {
        return tt < pre1 ? lo0 + tt
                         : (tt < pre2 ? lo1 + (tt - pre1) : (tt < pre3 ? lo2 + (tt - pre2) : lo3 + (tt - pre3)));
    };
    const uint32_t stride = nblk * kSGPerBlock;
    constexpr bool kAhead = codec_ahead<MODE, LOCAL>();
    if (kAhead) {
        const uint32_t t0 = blk * kSGPerBlock + wave * 4 + row;
        if (t0 < N && g == 0) {
            const uint32_t p0 = pos_of(t0);
            *slot_j = (uint32_t)a.perm[p0];
            *slot_mu = a.mu_stream[p0];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    for (uint32_t base = blk * kSGPerBlock; base < N; base += stride) {
        const uint32_t t = base + wave * 4 + row;
        if (t >= N) continue;
        uint32_t j = 0u;
        float mu = 0.0f;
        uint32_t pn = 0xFFFFFFFFu;
        if (kAhead) {
            // written by this row at the end of its previous super-group (or
            // before the loop): same wave, same address, program order
            j = *slot_j;
            mu = *slot_mu;
            if (t + stride < N) pn = pos_of(t + stride);
        }
        if (t < pre1) codec_sg<2, MODE, LOCAL>(a, po, pi, In, Own, Out, t, j, mu, pn, slot_j, slot_mu, g, T, stage_row);
        else if (t < pre2) codec_sg<4, MODE, LOCAL>(a, po, pi, In, Own, Out, t, j, mu, pn, slot_j, slot_mu, g, T, stage_row);
        else if (t < pre3) codec_sg<8, MODE, LOCAL>(a, po, pi, In, Own, Out, t, j, mu, pn, slot_j, slot_mu, g, T, stage_row);
        else if constexpr (WIDE)
            codec_sg<16, MODE, LOCAL>(a, po, pi, In, Own, Out, t, j, mu, pn, slot_j, slot_mu, g, T, stage_row);
    }
}

// ---------------------------------------------------------------------------
// finalize: decode the final region, add back n * mean, restore the order.
// Lane g of a row holds coordinates 64v + 4g .. 64v + 4g + 3 (v = 0..3) of the
// row's super-group, i.e. 4-coordinate pieces of groups 4v + g/4, so each
// store instruction writes 256 contiguous bytes per row.
// ---------------------------------------------------------------------------

template <int Q>
__device__ __forceinline__ void finalize_sg(const CodecArgs &a, const PartInfo &P, int64_t t,
                                            int g, const SharedTables &T) {
    constexpr int K = Q == 2 ? 0 : (Q == 4 ? 1 : (Q == 8 ? 2 : 3));
    const int64_t idx = t - P.pre[K];
    const int64_t pos = P.lo[K] + idx;
    const int64_t j = a.perm[pos];
    const uint8_t *reg = a.region_in;
    const float s = *reinterpret_cast<const float *>(reg + P.offs + 4 * t);
    const uint4 cg4 = *reinterpret_cast<const uint4 *>(reg + P.offg + 16 * t);
    const uint32_t cgw[4] = {cg4.x, cg4.y, cg4.z, cg4.w};
    const float add = a.n_workers_f * a.mu_stream[pos];
    const uint8_t *codes = reg + P.offc[K] + idx * (32 * Q);
    float4 *out = reinterpret_cast<float4 *>(a.out_f32 + j * kSG);
    const uint32_t shift = 8u * (uint32_t)(g >> 2);
#pragma unroll
    for (int v = 0; v < 4; v++) {
        // group 4v + g/4: its UINT8 code is byte g/4 of word v of the 16 codes
        const uint32_t c = (cgw[v] >> shift) & 0xFFu;
        const float sigma = (float)c * s;
        const int c0 = 64 * v + 4 * g;                  // first coordinate of the piece
        uint64_t w;
        if constexpr (Q == 16) w = *reinterpret_cast<const unsigned long long *>(codes + 2 * c0);
        else if constexpr (Q == 8) w = *reinterpret_cast<const uint32_t *>(codes + c0);
        else if constexpr (Q == 4) w = *reinterpret_cast<const uint16_t *>(codes + c0 / 2);
        else w = codes[c0 / 4];
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t code = (uint32_t)(w >> (i * Q)) & ((1u << Q) - 1u);
            x[i] = sigma * level_of<Q>(T, a.L16, code) + add;
        }
        // the output is written once and not read back here: non-temporal
        const f32x4_t xv = {x[0], x[1], x[2], x[3]};
        __builtin_nontemporal_store(xv, reinterpret_cast<f32x4_t *>(&out[16 * v + g]));
    }
}

template <bool WIDE>
__global__ __launch_bounds__(256) void k_finalize(CodecArgs a) {
    __shared__ __align__(16) SharedTables T;
    const LevelTables &lev = a.tab->lev;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) T.dec8[i] = lev.L8[i];
    if (threadIdx.x < 16) T.dec4[threadIdx.x] = lev.L4[threadIdx.x];
    if (threadIdx.x < 4) T.dec2[threadIdx.x] = lev.L2[threadIdx.x];
    __syncthreads();
    const PartInfo P = *a.part_in;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 15, row = lane >> 4;
    for (int64_t base = (int64_t)blockIdx.x * kSGPerBlock; base < P.N;
         base += (int64_t)gridDim.x * kSGPerBlock) {
        const int64_t t = base + wave * 4 + row;
        if (t >= P.N) continue;
        if (t < P.pre[1]) finalize_sg<2>(a, P, t, g, T);
        else if (t < P.pre[2]) finalize_sg<4>(a, P, t, g, T);
        else if (!WIDE || t < P.pre[3]) finalize_sg<8>(a, P, t, g, T);
        else if constexpr (WIDE) finalize_sg<16>(a, P, t, g, T);
    }
}

// ---------------------------------------------------------------------------
// part table (once per round, after the class counts are known)
// ---------------------------------------------------------------------------

__host__ __device__ inline int32_t part_entries(int32_t n, int32_t topology) {
    if (n == 1) return 1;
    return topology == 0 ? n : 2 * n - 2;
}

__global__ void k_part_table(const unsigned long long *C, int32_t n, int32_t topology,
                             PartInfo *table) {
    const int32_t e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= part_entries(n, topology)) return;
    int64_t m = 1, c = 0;
    if (n > 1 && topology == 0) {
        m = n;
        c = e;
    } else if (n > 1) {
        m = 2;
        while (e >= (2 * m - 2)) m *= 2;   // entries of m start at m - 2
        c = e - (m - 2);
    }
    PartInfo p;
    part_info(C, m, c, p);
    table[e] = p;
}

int32_t part_table_entries(int32_t n, int32_t topology) { return part_entries(n, topology); }

int32_t part_table_index(int32_t n, int32_t topology, int64_t m, int64_t c) {
    if (n == 1) return 0;
    if (topology == 0) return (int32_t)c;
    return (int32_t)(m - 2 + c);
}

hipError_t launch_part_table(const unsigned long long *class_counts, int32_t n, int32_t topology,
                             PartInfo *table, hipStream_t s) {
    const int32_t e = part_entries(n, topology);
    hipLaunchKernelGGL(k_part_table, dim3((e + 63) / 64), dim3(64), 0, s, class_counts, n, topology,
                       table);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// statistics
// ---------------------------------------------------------------------------

// Lane l of a 16-lane DPP row holds the partials k = l and k = l + 16 of one
// super-group (8 sequential adds each).  The tree step P_k <- P_k + P_{k+delta}
// is then in-lane for delta = 16 and a DPP row shift (lane i reads lane i +
// delta) for delta = 8, 4, 2, 1; lanes past the ones that matter compute values
// nobody reads.  The result is in lane 0 of the row.
template <int CTRL>
__device__ __forceinline__ float dpp_shl(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float tree16(float x) {
    x = x + dpp_shl<0x108>(x);   // row_shl:8
    x = x + dpp_shl<0x104>(x);   // row_shl:4
    x = x + dpp_shl<0x102>(x);   // row_shl:2
    x = x + dpp_shl<0x101>(x);   // row_shl:1
    return x;
}

// the raw bytes of partial k of super-group j (elements 8k .. 8k+7): one
// 16-byte load of bf16, two of fp32; converted only when summed, so that the
// loads of a whole iteration fit in registers
template <int F32> struct Partial;
template <> struct Partial<0> {
    uint4 h;
    __device__ __forceinline__ void load(const void *grad, int64_t j, int k) {
        h = stream_load_u4(static_cast<const uint16_t *>(grad) + j * kSG + k * 8);
    }
    __device__ __forceinline__ void clear() { h = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void values(float (&e)[8]) const {
        e[0] = bf16_lo(h.x); e[1] = bf16_hi(h.x); e[2] = bf16_lo(h.y); e[3] = bf16_hi(h.y);
        e[4] = bf16_lo(h.z); e[5] = bf16_hi(h.z); e[6] = bf16_lo(h.w); e[7] = bf16_hi(h.w);
    }
};
template <> struct Partial<1> {
    float4 f0, f1;
    __device__ __forceinline__ void load(const void *grad, int64_t j, int k) {
        const float *src = static_cast<const float *>(grad) + j * kSG + k * 8;
        f0 = stream_load_f4(src);
        f1 = stream_load_f4(src + 4);
    }
    __device__ __forceinline__ void clear() { f0 = f1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
    __device__ __forceinline__ void values(float (&e)[8]) const {
        e[0] = f0.x; e[1] = f0.y; e[2] = f0.z; e[3] = f0.w;
        e[4] = f1.x; e[5] = f1.y; e[6] = f1.z; e[7] = f1.w;
    }
};

template <int F32>
__device__ __forceinline__ void partial_sums(const Partial<F32> &p, float &s, float &q) {
    float e[8];
    p.values(e);
    s = e[0];
    q = e[0] * e[0];
#pragma unroll
    for (int i = 1; i < 8; i++) {
        s = s + e[i];
        const float sq = e[i] * e[i];
        q = q + sq;
    }
}

// One resident 1024-thread block per CU owns a contiguous range of at most
// kStatsChunk super-groups.  A wave takes 4 rows x iterations super-groups per
// step (all their loads in flight before any arithmetic); each row's leader
// parks its sums in LDS.  Only when the whole range has been read does the
// block read the earlier workers' running sums, add, and store the new ones,
// in one coalesced burst: writes interleaved with the read stream make the
// memory turn around and cost far more than their bytes.
constexpr int kStatsThreads = 1024;
constexpr int kStatsChunk = 15360;                   // 120 KB of LDS per block
template <int F32>
constexpr int stats_iters() { return F32 ? 4 : 8; }  // fp32 partials take twice the registers

template <int F32>
__global__ __launch_bounds__(kStatsThreads) void k_stats(StatsArgs a, int64_t chunk) {
    constexpr int kIter = stats_iters<F32>();
    constexpr int kPerWave = 4 * kIter, kPerBlock = (kStatsThreads / 64) * kPerWave;
    const int row = (threadIdx.x >> 4) & 3, wave = threadIdx.x >> 6, l = threadIdx.x & 15;
    __shared__ float park[2][kStatsChunk];
    for (int64_t c0 = (int64_t)blockIdx.x * chunk; c0 < a.J; c0 += (int64_t)gridDim.x * chunk) {
        const int64_t c1 = c0 + chunk < a.J ? c0 + chunk : a.J;
        for (int64_t base = c0; base < c1; base += kPerBlock) {
            const int64_t wbase = base + wave * kPerWave;
            Partial<F32> p0[kIter], p1[kIter];
#pragma unroll
            for (int u = 0; u < kIter; u++) {
                const int64_t j = wbase + u * 4 + row;
                if (j < c1) {
                    p0[u].load(a.grad, j, l);
                    p1[u].load(a.grad, j, l + 16);
                } else {
                    p0[u].clear();
                    p1[u].clear();
                }
            }
#pragma unroll
            for (int u = 0; u < kIter; u++) {
                float sa, qa, sb, qb;
                partial_sums(p0[u], sa, qa);
                partial_sums(p1[u], sb, qb);
                const float s = tree16(sa + sb), q = tree16(qa + qb);
                const int64_t j = wbase + u * 4 + row;
                if (l == 0 && j < c1) {
                    park[0][j - c0] = s;
                    park[1][j - c0] = q;
                }
            }
        }
        __syncthreads();
        // the fold with the earlier workers' running sums: all of this
        // thread's loads are issued before any is used (one memory round
        // trip rather than one per element), then the adds and stores
        constexpr int kTail = (kStatsChunk + kStatsThreads - 1) / kStatsThreads;
        float ps[kTail], pq[kTail];
        if (!a.first) {
#pragma unroll
            for (int k = 0; k < kTail; k++) {
                const int64_t j = c0 + threadIdx.x + (int64_t)k * kStatsThreads;
                ps[k] = j < c1 ? a.sum[j] : 0.0f;
                pq[k] = j < c1 ? a.sumsq[j] : 0.0f;
            }
        }
        bool bad = false;
#pragma unroll
        for (int k = 0; k < kTail; k++) {
            const int64_t j = c0 + threadIdx.x + (int64_t)k * kStatsThreads;
            if (j < c1) {
                const float s = park[0][j - c0], q = park[1][j - c0];
                const float S = a.first ? s : ps[k] + s, F = a.first ? q : pq[k] + q;
                __builtin_nontemporal_store(S, a.sum + j);
                __builtin_nontemporal_store(F, a.sumsq + j);
                bad |= !(__builtin_isfinite(S) && __builtin_isfinite(F));
            }
        }
        if (bad) atomicOr(a.nonfinite, 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// allocation: bisection on the fp32 bit pattern of rho, integer counts
// ---------------------------------------------------------------------------

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v) {
    __shared__ unsigned long long part[4];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    unsigned long long t = 0;
    if (threadIdx.x == 0) t = part[0] + part[1] + part[2] + part[3];
    return t;
}

// Radix search for rho: the smallest x in [0, 0x7F800000] (fp32 bit patterns
// of rho >= 0, up to +inf) with  sum_j q_j(x) <= budget,  a non-increasing
// count.  Pass p tests the candidates x_c = prefix + (c << shift_p); the first
// passing candidate c* leaves prefix + ((c* - 1) << shift_p) as the largest
// known failing value, and the last pass (shift 0) returns x_{c*} itself.
// Same result as any exact search of the monotone predicate.
__device__ __forceinline__ int radix_shift(int pass) { return pass == 0 ? 23 : (pass == 1 ? 15 : (pass == 2 ? 7 : 0)); }
__device__ __forceinline__ int radix_ncand(int pass) { return pass == 3 ? 128 : 256; }

// The value the thresholds compare: F_j, or under the mean-corrected variant
// the squared norm of the mean-subtracted values, F_j - fl(256 n) mu_j^2 with
// each product and difference rounded once and negative results set to 0.
__device__ __forceinline__ float alloc_key(const AllocArgs &a, float F, float sum) {
    if (a.mode != kAllocMeanCorrected) return F;
    const float mu = sum / a.denom;
    const float m2 = mu * mu;
    const float t = a.denom * m2;
    const float g = F - t;
    return g < 0.0f ? 0.0f : g;
}

// Threshold multipliers T = fl(K rho): widths {2,4,8} K24 = 544, K48 = 16384;
// with the 16-bit class the chain is scaled by 257 so that T48 / T816 =
// 257 / 2^17 stays exact: K24 = 139808, K48 = 4210688, K816 = 2^31.
__device__ __forceinline__ float k24(int wide) { return wide ? 139808.0f : 544.0f; }
__device__ __forceinline__ float k48(int wide) { return wide ? 4210688.0f : 16384.0f; }
constexpr float kK816 = 2147483648.0f;

// number of entries of the non-decreasing t[0..n) that are <= F
__device__ __forceinline__ uint32_t count_le(const float *t, int n, float F) {
    uint32_t lo = 0, len = (uint32_t)n;
    while (len > 0) {
        const uint32_t half = len >> 1;
        if (t[lo + half] <= F) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    return lo;
}

// For every F_j: i4 = #{c : fl(544 x_c) <= F_j}, i8 = #{c : fl(16384 x_c) <= F_j};
// histograms of i4 and i8 give, by suffix sums, how many super-groups reach
// 4 and 8 bits at each candidate.
__global__ __launch_bounds__(256) void k_alloc_count(AllocArgs a, int pass) {
    Ctrl *c = a.ctrl;
    if (c->done) return;
    __shared__ float t4[kRadixCand], t8[kRadixCand], t16[kRadixCand];
    __shared__ unsigned int h4[kRadixCand + 1], h8[kRadixCand + 1], h16[kRadixCand + 1];
    const int n = radix_ncand(pass), shift = radix_shift(pass);
    const uint32_t prefix = c->prefix;
    for (int i = threadIdx.x; i < kRadixCand + 1; i += blockDim.x) {
        h4[i] = 0u;
        h8[i] = 0u;
        h16[i] = 0u;
    }
    if (threadIdx.x < n) {
        const float rho = __uint_as_float(prefix + ((uint32_t)threadIdx.x << shift));
        t4[threadIdx.x] = k24(a.wide) * rho;
        t8[threadIdx.x] = k48(a.wide) * rho;
        t16[threadIdx.x] = kK816 * rho;
    }
    __syncthreads();
    // count 0 adds to no suffix sum and is skipped; count n (F at or above
    // every candidate threshold) is kept in a register
    const float lo4 = t4[0], hi4 = t4[n - 1], lo8 = t8[0], hi8 = t8[n - 1];
    const float lo16 = t16[0], hi16 = t16[n - 1];
    uint32_t top4 = 0u, top8 = 0u, top16 = 0u;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < a.J;
         j += (int64_t)gridDim.x * blockDim.x) {
        const float F = alloc_key(a, a.sumsq[j], a.mode == kAllocMeanCorrected ? a.sum[j] : 0.0f);
        if (F >= hi4) top4++;
        else if (F >= lo4) atomicAdd(&h4[count_le(t4, n, F)], 1u);
        if (F >= hi8) top8++;
        else if (F >= lo8) atomicAdd(&h8[count_le(t8, n, F)], 1u);
        if (a.wide) {
            if (F >= hi16) top16++;
            else if (F >= lo16) atomicAdd(&h16[count_le(t16, n, F)], 1u);
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        top4 += __shfl_xor(top4, d, 64);
        top8 += __shfl_xor(top8, d, 64);
        top16 += __shfl_xor(top16, d, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        if (top4) atomicAdd(&h4[n], top4);
        if (top8) atomicAdd(&h8[n], top8);
        if (top16) atomicAdd(&h16[n], top16);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n + 1; i += blockDim.x) {
        if (h4[i]) atomicAdd(&c->hist4[i], h4[i]);
        if (h8[i]) atomicAdd(&c->hist8[i], h8[i]);
        if (h16[i]) atomicAdd(&c->hist16[i], h16[i]);
    }
}

// One block of 256: total bits at each candidate from suffix sums of the
// histograms, first passing candidate, next prefix (or rho); then clears the
// histograms for the next pass.
__global__ __launch_bounds__(256) void k_alloc_decide(AllocArgs a, int pass) {
    Ctrl *c = a.ctrl;
    if (c->done) return;
    __shared__ unsigned long long s4[kRadixCand], s8[kRadixCand], s16[kRadixCand];
    __shared__ int first;
    const int n = radix_ncand(pass), shift = radix_shift(pass);
    const int t = threadIdx.x;
    // s[t] starts as hist[t + 1]; after the scan s[t] = #{j : i_j > t}
    s4[t] = t < n ? c->hist4[t + 1] : 0ull;
    s8[t] = t < n ? c->hist8[t + 1] : 0ull;
    s16[t] = t < n ? c->hist16[t + 1] : 0ull;
    if (t == 0) first = n;
    __syncthreads();
    for (int d = 1; d < kRadixCand; d <<= 1) {
        const unsigned long long v4 = t + d < kRadixCand ? s4[t + d] : 0ull;
        const unsigned long long v8 = t + d < kRadixCand ? s8[t + d] : 0ull;
        const unsigned long long v16 = t + d < kRadixCand ? s16[t + d] : 0ull;
        __syncthreads();
        s4[t] += v4;
        s8[t] += v8;
        s16[t] += v16;
        __syncthreads();
    }
    if (t < n) {
        // 2 bits each, +2 at 4 bits, +4 more at 8, +8 more at 16
        const long long total = 2 * (long long)a.J + 2 * (long long)s4[t] + 4 * (long long)s8[t] +
                                8 * (long long)s16[t];
        if (total <= a.budget) atomicMin(&first, t);
    }
    __syncthreads();
    if (t == 0) {
        const int cs = first;
        const uint32_t prefix = c->prefix;
        if (cs == 0) {              // only at pass 0 (later passes start at a failing value): rho = 0
            c->rho_bits = prefix;
            c->done = 1u;
        } else if (cs == n && pass == 0) {
            // not even rho = +inf (the last candidate) meets the budget: only
            // keys of +inf (overflowed squared norms, which the statistics
            // flag) keep a width above 2 there.  The search range ends at
            // +inf, and so does rho; the next passes would step past it.
            c->rho_bits = 0x7F800000u;
            c->done = 1u;
        } else if (pass == kRadixPasses - 1) {
            c->rho_bits = prefix + ((uint32_t)cs << shift);
            c->done = 1u;
        } else {
            c->prefix = prefix + ((uint32_t)(cs - 1) << shift);
        }
    }
    for (int i = t; i < kRadixCand + 1; i += blockDim.x) {
        c->hist4[i] = 0u;
        c->hist8[i] = 0u;
        c->hist16[i] = 0u;
    }
}

// widths, per-block class counts for the reorder, global class counts
__global__ __launch_bounds__(256) void k_alloc_final(AllocArgs a) {
    Ctrl *c = a.ctrl;
    const bool uniform = a.mode == kAllocUniform, centred = a.mode == kAllocMeanCorrected;
    // the uniform variant has no scalar (block 0 stores NaN below, nobody reads it)
    const uint32_t rb = uniform ? 0u : c->rho_bits;
    const float rho = __uint_as_float(rb);
    const float t4 = k24(a.wide) * rho, t8 = k48(a.wide) * rho;
    // without the 16-bit class no key reaches class 3, not even F = +inf (a
    // squared norm that overflowed): the class-3 test is skipped, not given
    // an infinite threshold that +inf would meet
    const bool wide = a.wide;
    const float t16 = kK816 * rho;
    uint32_t cnt[kClasses] = {0u, 0u, 0u, 0u};
    const int64_t j0 = (int64_t)blockIdx.x * kReorderSGPerBlock + threadIdx.x * 4;
    if (j0 + 4 <= a.J) {
        // the arrays are 256-byte aligned in the workspace and j0 is a multiple of 4
        const float4 F4 = *reinterpret_cast<const float4 *>(a.sumsq + j0);
        float4 S4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (centred) S4 = *reinterpret_cast<const float4 *>(a.sum + j0);
        const float F[4] = {F4.x, F4.y, F4.z, F4.w}, S[4] = {S4.x, S4.y, S4.z, S4.w};
        uint32_t w = 0u;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float G = alloc_key(a, F[i], S[i]);
            const int k = uniform ? a.uniform_k : ((wide && G >= t16) ? 3 : (G >= t8 ? 2 : (G >= t4 ? 1 : 0)));
            w |= (2u << k) << (8 * i);
            cnt[k]++;
        }
        *reinterpret_cast<uint32_t *>(a.widths + j0) = w;
    } else {
        for (int64_t j = j0; j < a.J; j++) {
            const float G = alloc_key(a, a.sumsq[j], centred ? a.sum[j] : 0.0f);
            const int k = uniform ? a.uniform_k : ((wide && G >= t16) ? 3 : (G >= t8 ? 2 : (G >= t4 ? 1 : 0)));
            a.widths[j] = (uint8_t)(2 << k);
            cnt[k]++;
        }
    }
    if (uniform && blockIdx.x == 0 && threadIdx.x == 0) c->rho_bits = 0x7FC00000u;
    // pack four counts (each <= 1024) into 16-bit fields and reduce
    unsigned long long v = (unsigned long long)cnt[0] | ((unsigned long long)cnt[1] << 16) |
                           ((unsigned long long)cnt[2] << 32) | ((unsigned long long)cnt[3] << 48);
    const unsigned long long tot = block_sum_u64(v);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < kClasses; k++)
            a.blkcnt[k * a.nblk + blockIdx.x] = (int32_t)((tot >> (16 * k)) & 0xFFFFu);
    }
}

// Class totals from the per-block counts (one block; no contended atomics).
__global__ __launch_bounds__(1024) void k_alloc_totals(AllocArgs a) {
    __shared__ unsigned long long part[16][kClasses];
    unsigned long long s[kClasses] = {0ull, 0ull, 0ull, 0ull};
    for (int64_t b = threadIdx.x; b < a.nblk; b += blockDim.x) {
#pragma unroll
        for (int k = 0; k < kClasses; k++) s[k] += (unsigned long long)a.blkcnt[k * a.nblk + b];
    }
#pragma unroll
    for (int k = 0; k < kClasses; k++) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s[k] += __shfl_xor(s[k], d, 64);
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < kClasses; k++) part[threadIdx.x >> 6][k] = s[k];
    }
    __syncthreads();
    if (threadIdx.x < kClasses) {
        unsigned long long t = 0ull;
        for (int w = 0; w < (int)(blockDim.x >> 6); w++) t += part[w][threadIdx.x];
        a.ctrl->class_counts[threadIdx.x] = t;
    }
}

__global__ __launch_bounds__(1024) void k_reorder_scan(ReorderArgs a) {
    __shared__ int64_t sh[1024];
    const int64_t nb = a.nblk;
    const int64_t per = (nb + 1023) / 1024;
    const int64_t b0 = threadIdx.x * per, b1 = min(nb, b0 + per);
    int64_t base = 0;
    for (int k = 0; k < kClasses; k++) {
        int64_t mine = 0;
        for (int64_t b = b0; b < b1; b++) mine += a.blkcnt[k * nb + b];
        sh[threadIdx.x] = mine;
        __syncthreads();
        // Hillis-Steele inclusive scan over 1024 threads
        for (int d = 1; d < 1024; d <<= 1) {
            const int64_t add = threadIdx.x >= d ? sh[threadIdx.x - d] : 0;
            __syncthreads();
            sh[threadIdx.x] += add;
            __syncthreads();
        }
        int64_t run = base + sh[threadIdx.x] - mine;
        for (int64_t b = b0; b < b1; b++) {
            const int32_t cb = a.blkcnt[k * nb + b];
            a.blkcnt[k * nb + b] = (int32_t)run;
            run += cb;
        }
        base += (int64_t)a.ctrl->class_counts[k];
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_reorder_scatter(ReorderArgs a) {
    __shared__ unsigned long long wtot[4];
    const int64_t j0 = (int64_t)blockIdx.x * kReorderSGPerBlock + threadIdx.x * 4;
    int k_of[4];
    uint32_t cnt[kClasses] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t j = j0 + i;
        k_of[i] = -1;
        if (j < a.J) {
            const uint8_t q = a.widths[j];
            k_of[i] = q == 2 ? 0 : (q == 4 ? 1 : (q == 8 ? 2 : 3));
            cnt[k_of[i]]++;
        }
    }
    const unsigned long long mine = (unsigned long long)cnt[0] | ((unsigned long long)cnt[1] << 16) |
                                    ((unsigned long long)cnt[2] << 32) | ((unsigned long long)cnt[3] << 48);
    // inclusive scan inside the wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long inc = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    unsigned long long before = 0;
    for (int w = 0; w < wave; w++) before += wtot[w];
    unsigned long long excl = before + inc - mine;
    int32_t pos[kClasses];
#pragma unroll
    for (int k = 0; k < kClasses; k++)
        pos[k] = a.blkcnt[k * a.nblk + blockIdx.x] + (int32_t)((excl >> (16 * k)) & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (k_of[i] < 0) continue;
        const int64_t j = j0 + i;
        const int32_t p = pos[k_of[i]]++;
        a.perm[p] = (int32_t)j;
        a.inv[j] = p;
        a.mu_stream[p] = a.sum[j] / a.denom;
    }
}

// ---------------------------------------------------------------------------
// MXFP8 reference (OCP Microscaling v1.0: 32-element blocks, E8M0 scale
// 2^(floor(log2 max|x|) - 8) clamped to [2^-127, 2^127], E4M3 elements rounded
// to nearest even and saturated at 448).  Measurement path for the quality
// report; one thread per 8 coordinates, a DPP quad per 32-element block.
// ---------------------------------------------------------------------------

// Compares recip_rn with the IEEE quotient 1/x for the fp32 bit patterns
// [lo, lo + n); counts the mismatches.
__global__ __launch_bounds__(256) void k_check_recip(uint32_t lo, uint32_t n, unsigned long long *count) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    bool bad = false;
    if (i < n) {
        const float x = __uint_as_float(lo + i);
        bad = __float_as_uint(recip_rn(x)) != __float_as_uint(1.0f / x);
    }
    const unsigned long long m = __ballot(bad);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd(count, (unsigned long long)__popcll(m));
}

// round_half_up against the exact floor(x + 0.5) (in double, where x + 0.5
// is exact) for the bit patterns lo .. lo + n - 1, with the conversion's
// saturation beyond the int range; NaN saturates by its sign bit
__global__ __launch_bounds__(256) void k_check_rpi(uint32_t lo, uint32_t n, unsigned long long *count) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    bool bad = false;
    if (i < n) {
        const float x = __uint_as_float(lo + i);
        int want;
        if (x != x) {
            want = (lo + i) >> 31 ? (-2147483647 - 1) : 2147483647;
        } else {
            const double f = floor((double)x + 0.5);
            want = f >= 2147483647.0 ? 2147483647 : (f <= -2147483648.0 ? (-2147483647 - 1) : (int)f);
        }
        bad = round_half_up(x) != want;
    }
    const unsigned long long m = __ballot(bad);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd(count, (unsigned long long)__popcll(m));
}

__device__ __forceinline__ int floor_log2(float a) {   // a > 0
    const uint32_t b = __float_as_uint(a);
    const int e = (int)(b >> 23);
    if (e != 0) return e - 127;
    return (31 - __clz(b)) - 149;                      // subnormal
}

// MX element formats (OCP Microscaling v1.0): mantissa bits, exponent of the
// smallest normal and of the largest normal, largest finite value, sign bit,
// and the code of the largest finite value.  Codes are stored one per byte.
template <int FMT> struct MxElem;
template <> struct MxElem<kMxE4M3> {
    static constexpr int kM = 3, kEmin = -6, kEmax = 8, kSign = 7;
    static constexpr float kMax = 448.0f;
};
template <> struct MxElem<kMxE3M2> {
    static constexpr int kM = 2, kEmin = -2, kEmax = 4, kSign = 5;
    static constexpr float kMax = 28.0f;
};
template <> struct MxElem<kMxE2M3> {
    static constexpr int kM = 3, kEmin = 0, kEmax = 2, kSign = 5;
    static constexpr float kMax = 7.5f;
};
template <> struct MxElem<kMxE2M1> {
    static constexpr int kM = 1, kEmin = 0, kEmax = 2, kSign = 3;
    static constexpr float kMax = 6.0f;
};

// magnitude code of a value a on the element grid: ((ex - emin) << M) + q
// with ex = max(floor(log2 a), emin) and q = a 2^(M - ex) rounded to nearest
// even (a carry into the next binade is the next code)
template <int FMT>
__host__ __device__ constexpr uint32_t mx_max_code() {
    using F = MxElem<FMT>;
    return (uint32_t)(((F::kEmax - F::kEmin) << F::kM) +
                      (int)(F::kMax / (float)(1 << F::kEmax) * (float)(1 << F::kM)));
}
static_assert(mx_max_code<kMxE4M3>() == 0x7Eu && mx_max_code<kMxE3M2>() == 0x1Fu &&
              mx_max_code<kMxE2M3>() == 0x1Fu && mx_max_code<kMxE2M1>() == 0x7u, "MX max codes");

// element code of v (v already divided by the block scale)
template <int FMT>
__device__ __forceinline__ uint32_t mx_encode(float v) {
    using F = MxElem<FMT>;
    const float a = fabsf(v);
    if (a == 0.0f) return 0u;
    const uint32_t sign = (__float_as_uint(v) >> 31) << F::kSign;
    if (a >= F::kMax) return sign | mx_max_code<FMT>();
    const int ex = max(floor_log2(a), F::kEmin);
    const uint32_t q = (uint32_t)rintf(a * ldexpf(1.0f, F::kM - ex));   // exact scaling, nearest even
    return sign | ((uint32_t)((ex - F::kEmin) << F::kM) + q);
}

template <int FMT>
__device__ __forceinline__ float mx_decode(uint32_t code, int se) {
    using F = MxElem<FMT>;
    const uint32_t mag = code & ((1u << F::kSign) - 1u), E = mag >> F::kM, M = mag & ((1u << F::kM) - 1u);
    const float m = (float)(E ? (1u << F::kM) + M : M);
    float v = ldexpf(m, (int)(E ? E : 1u) + F::kEmin - 1 - F::kM + se);
    return ((code >> F::kSign) & 1u) ? -v : v;
}

template <int FMT, int MODE, int LOCAL>
__global__ __launch_bounds__(256) void k_mx(MxArgs a) {
    using F = MxElem<FMT>;
    const int64_t nthreads = a.n / 8;
    const int64_t in_codes = a.in_n, out_codes = a.n;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nthreads;
         t += (int64_t)gridDim.x * blockDim.x) {
        // a.n is a multiple of 256, so the 4 threads of a quad pass or fail this test together
        const int64_t i0 = a.lo + 8 * t;                 // first coordinate (original order)
        float y[8];
        if constexpr (MODE != kCompress) {
            const int64_t r = i0 - a.in_lo;
            const uint2 cw = *reinterpret_cast<const uint2 *>(a.in + r);
            const int se = (int)a.in[in_codes + r / 32] - 127;
            for (int i = 0; i < 8; i++) y[i] = mx_decode<FMT>(((i < 4 ? cw.x : cw.y) >> (8 * (i & 3))) & 0xFFu, se);
        }
        if constexpr (MODE == kFinalize) {
            float4 *o = reinterpret_cast<float4 *>(a.out_f32 + i0);
            o[0] = make_float4(y[0], y[1], y[2], y[3]);
            o[1] = make_float4(y[4], y[5], y[6], y[7]);
            continue;
        } else {
            float e[8];
            if constexpr (LOCAL == kLocalBF16) {
                const uint4 h = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.grad) + i0);
                const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                for (int i = 0; i < 4; i++) { e[2 * i] = bf16_lo(hw[i]); e[2 * i + 1] = bf16_hi(hw[i]); }
            } else if constexpr (LOCAL == kLocalF32) {
                const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.grad) + i0);
                const float4 f0 = src[0], f1 = src[1];
                e[0] = f0.x; e[1] = f0.y; e[2] = f0.z; e[3] = f0.w;
                e[4] = f1.x; e[5] = f1.y; e[6] = f1.z; e[7] = f1.w;
            } else {
                const int64_t r = i0 - a.in_lo;
                const uint2 cw = *reinterpret_cast<const uint2 *>(a.own + r);
                const int se = (int)a.own[in_codes + r / 32] - 127;
                for (int i = 0; i < 8; i++) e[i] = mx_decode<FMT>(((i < 4 ? cw.x : cw.y) >> (8 * (i & 3))) & 0xFFu, se);
            }
            for (int i = 0; i < 8; i++) y[i] = (MODE == kHop) ? y[i] + e[i] : e[i];
        }
        float amax = 0.0f;
        for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(y[i]));
        amax = fmaxf(amax, dpp_mov<0xB1>(amax));
        amax = fmaxf(amax, dpp_mov<0x4E>(amax));
        int se = -127;
        if (amax > 0.0f) se = min(max(floor_log2(amax) - F::kEmax, -127), 127);
        uint32_t w0 = 0u, w1 = 0u;
        for (int i = 0; i < 8; i++) {
            const uint32_t c = mx_encode<FMT>(ldexpf(y[i], -se));
            if (i < 4) w0 |= c << (8 * i);
            else w1 |= c << (8 * (i - 4));
        }
        const int64_t r = i0 - a.lo;
        *reinterpret_cast<uint2 *>(a.out + r) = make_uint2(w0, w1);
        if ((threadIdx.x & 3) == 0) a.out[out_codes + r / 32] = (uint8_t)(se + 127);
    }
}

template <int FMT>
static hipError_t launch_mx_fmt(const MxArgs &a, int local, dim3 grid, dim3 block, hipStream_t s) {
    if (a.mode == kCompress && local == kLocalBF16) hipLaunchKernelGGL((k_mx<FMT, kCompress, kLocalBF16>), grid, block, 0, s, a);
    else if (a.mode == kCompress && local == kLocalF32) hipLaunchKernelGGL((k_mx<FMT, kCompress, kLocalF32>), grid, block, 0, s, a);
    else if (a.mode == kHop && local == kLocalBF16) hipLaunchKernelGGL((k_mx<FMT, kHop, kLocalBF16>), grid, block, 0, s, a);
    else if (a.mode == kHop && local == kLocalF32) hipLaunchKernelGGL((k_mx<FMT, kHop, kLocalF32>), grid, block, 0, s, a);
    else if (a.mode == kHop && local == kLocalPacked) hipLaunchKernelGGL((k_mx<FMT, kHop, kLocalPacked>), grid, block, 0, s, a);
    else if (a.mode == kFinalize) hipLaunchKernelGGL((k_mx<FMT, kFinalize, kLocalNone>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mx(const MxArgs &a, int fmt, int local, hipStream_t s) {
    const dim3 grid(grid_for(a.n / 8, 256, 4096)), block(256);
    switch (fmt) {
        case kMxE4M3: return launch_mx_fmt<kMxE4M3>(a, local, grid, block, s);
        case kMxE3M2: return launch_mx_fmt<kMxE3M2>(a, local, grid, block, s);
        case kMxE2M3: return launch_mx_fmt<kMxE2M3>(a, local, grid, block, s);
        case kMxE2M1: return launch_mx_fmt<kMxE2M1>(a, local, grid, block, s);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// streaming probe: the HBM rate a kernel with a given read:write mix reaches.
// A wave moves tiles of R x 64 sixteen-byte words: load k of a tile reads
// words k*64 .. k*64 + 63 (one contiguous kilobyte per instruction), and the
// xor of the R words a lane read is stored as one 16-byte word of the tile's
// contiguous kilobyte of output.  R = 0 reads only: every lane folds all it
// read and stores one word at the end of the grid-stride loop, so no write
// is interleaved with the read stream.  Plain loads and stores, as in the
// codec kernels.
// ---------------------------------------------------------------------------

constexpr int kProbeBlocks = 2048;     // 256 CUs x 8 resident blocks of 256 threads

template <int R>
__global__ __launch_bounds__(256) void k_probe_stream(const uint4 *src, int64_t tiles, uint4 *dst) {
    constexpr int kR = R == 0 ? 1 : R;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t t = wave; t < tiles; t += waves) {
        const uint4 *p = src + t * (64 * kR) + lane;
        uint4 v[kR];
#pragma unroll
        for (int k = 0; k < kR; k++) v[k] = p[64 * k];
        uint4 x = v[0];
#pragma unroll
        for (int k = 1; k < kR; k++) x = make_uint4(x.x ^ v[k].x, x.y ^ v[k].y, x.z ^ v[k].z, x.w ^ v[k].w);
        if constexpr (R == 0) acc = make_uint4(acc.x ^ x.x, acc.y ^ x.y, acc.z ^ x.z, acc.w ^ x.w);
        else dst[t * 64 + lane] = x;
    }
    if constexpr (R == 0) dst[wave * 64 + lane] = acc;
}

int64_t probe_stream_sink_bytes() { return (int64_t)kProbeBlocks * 256 * 16; }

hipError_t launch_probe_stream(const void *src, int64_t tiles, int reads_per_write, void *dst, hipStream_t s) {
    const dim3 grid(kProbeBlocks), block(256);
    const uint4 *in = static_cast<const uint4 *>(src);
    uint4 *out = static_cast<uint4 *>(dst);
    switch (reads_per_write) {
        case 0: hipLaunchKernelGGL(k_probe_stream<0>, grid, block, 0, s, in, tiles, out); break;
        case 1: hipLaunchKernelGGL(k_probe_stream<1>, grid, block, 0, s, in, tiles, out); break;
        case 2: hipLaunchKernelGGL(k_probe_stream<2>, grid, block, 0, s, in, tiles, out); break;
        case 4: hipLaunchKernelGGL(k_probe_stream<4>, grid, block, 0, s, in, tiles, out); break;
        case 8: hipLaunchKernelGGL(k_probe_stream<8>, grid, block, 0, s, in, tiles, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// utility
// ---------------------------------------------------------------------------

// Level, compare-level, (L, W) and bucket tables of the level shape eps, from
// the same constexpr definitions the compile-time checks use (fp64, rounded
// once to fp32); bucket entry k = the number of interior levels L[1..NL-2]
// whose bucket lies below k, by binary search (their buckets increase).
template <int NL>
__device__ int est_of(int k, double eps) {
    int lo = 0, hi = NL - 2;           // the count lies in [0, NL - 2]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bucket_of<NL>(level_f(mid, NL, eps)) < k) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_build_tables(DeviceTables *t, double eps) {
    LevelTables &v = t->lev;
    for (int r = threadIdx.x; r < 256; r += blockDim.x) {
        v.L8[r] = level_f(r, 256, eps);
        v.CL8[r] = compare_level(r, 256, eps);
        if (r < 255) v.LW8[r] = Pair{level_f(r, 256, eps), weight_f(r, 256, eps)};
        if (r < 16) {
            v.L4[r] = level_f(r, 16, eps);
            v.CL4[r] = compare_level(r, 16, eps);
        }
        if (r < 15) v.LW4[r] = Pair{level_f(r, 16, eps), weight_f(r, 16, eps)};
        if (r < 4) v.L2[r] = level_f(r, 4, eps);
        if (r < 3) v.W2[r] = weight_f(r, 4, eps);
    }
    for (int k = threadIdx.x; k < bucket_count(256); k += blockDim.x) {
        t->b8.est[k] = (unsigned char)est_of<256>(k, eps);
        if (k < bucket_count(16)) t->b4.est[k] = (unsigned char)est_of<16>(k, eps);
    }
    // the LDS image, from the tables just written (visible to the whole block
    // after the barrier)
    __syncthreads();
    SharedTables &S = t->lds;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) {
        S.dec8[i] = v.L8[i];
        S.cl8[i] = v.CL8[i];
        if (i < 255) S.lw8[i] = v.LW8[i];
        if (i < 16) {
            S.dec4[i] = v.L4[i];
            S.cl4[i] = v.CL4[i];
        }
        if (i < 15) S.lw4[i] = v.LW4[i];
        if (i < 4) S.dec2[i] = v.L2[i];
        if (i < 3) S.lw2[i] = Pair{v.L2[i], v.W2[i]};
    }
    for (int i = threadIdx.x; i < bucket_count(256); i += blockDim.x) {
        S.b8[i] = t->b8.est[i];
        if (i < bucket_count(16)) S.b4[i] = t->b4.est[i];
    }
    for (int b = threadIdx.x; b < 256; b += blockDim.x) {
#pragma unroll
        for (int k = 0; k < 4; k++) S.quad2[b][k] = v.L2[(b >> (2 * k)) & 3];
        S.pair4[b][0] = v.L4[b & 15];
        S.pair4[b][1] = v.L4[b >> 4];
    }
}

// the 16-bit class: L[r] and W[r] = fl32(65536 / (L[r+1] - L[r])) for
// r < 65,536, from the same fp64 definitions as the narrower classes (W[65535]
// is unused and set to 0)
__global__ __launch_bounds__(256) void k_build_tables16(float *L16, float *W16, Pair *LW16, double eps) {
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < 65536; r += gridDim.x * blockDim.x) {
        const float l = level_f(r, 65536, eps), w = r < 65535 ? weight_f(r, 65536, eps) : 0.0f;
        L16[r] = l;
        W16[r] = w;
        LW16[r] = Pair{l, w};
    }
}

hipError_t launch_build_tables16(float *L16, float *W16, Pair *LW16, double eps, hipStream_t s) {
    hipLaunchKernelGGL(k_build_tables16, dim3(256), dim3(256), 0, s, L16, W16, LW16, eps);
    return hipGetLastError();
}

hipError_t launch_build_tables(DeviceTables *t, double eps, hipStream_t s) {
    hipLaunchKernelGGL(k_build_tables, dim3(1), dim3(256), 0, s, t, eps);
    return hipGetLastError();
}

__global__ void k_zero_u32(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// static scratch for callers that cannot allocate (dq_allreduce_noalloc): the
// plan workspace and the region arena of one round, in a device array every
// GPU the library runs on holds until the process ends.  Host code uses the
// array only through the device address hipGetSymbolAddress returns, taken
// once per device with that device current.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **ptr) {
    static void *addr[kScratchDevices];
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    if (!addr[dev]) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t items, int64_t per_block, int64_t cap) {
    int64_t b = (items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

constexpr int64_t kStreamGrid = 2048;  // 256 CUs x 8 blocks

hipError_t launch_zero(uint32_t *p, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_u32, dim3(grid_for(n, 256, 1024)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_check_recip(uint32_t lo, uint32_t n, unsigned long long *count, hipStream_t s) {
    constexpr uint32_t kChunk = 1u << 28;   // bit patterns per launch
    for (uint32_t done = 0; done < n;) {
        const uint32_t k = n - done < kChunk ? n - done : kChunk;
        hipLaunchKernelGGL(k_check_recip, dim3((k + 255) / 256), dim3(256), 0, s, lo + done, k, count);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += k;
    }
    return hipSuccess;
}

hipError_t launch_check_rpi(uint32_t lo, uint32_t n, unsigned long long *count, hipStream_t s) {
    constexpr uint32_t kChunk = 1u << 28;   // bit patterns per launch
    for (uint32_t done = 0; done < n;) {
        const uint32_t k = n - done < kChunk ? n - done : kChunk;
        hipLaunchKernelGGL(k_check_rpi, dim3((k + 255) / 256), dim3(256), 0, s, lo + done, k, count);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += k;
    }
    return hipSuccess;
}

hipError_t launch_stats(const StatsArgs &a, int f32, hipStream_t s) {
    // one block per CU; the super-groups are cut into rounds x CUs even shares
    // of at most kStatsChunk, with the fewest rounds that allows, so that every
    // block does the same number of equal shares
    const int64_t cus = device_cus();
    const int64_t rounds = (a.J + cus * kStatsChunk - 1) / (cus * kStatsChunk);
    int64_t chunk = (a.J + rounds * cus - 1) / (rounds * cus);
    if (chunk < 1) chunk = 1;
    const dim3 grid(grid_for(a.J, chunk, cus));
    if (f32) hipLaunchKernelGGL(k_stats<1>, grid, dim3(kStatsThreads), 0, s, a, chunk);
    else hipLaunchKernelGGL(k_stats<0>, grid, dim3(kStatsThreads), 0, s, a, chunk);
    return hipGetLastError();
}

hipError_t launch_alloc_pass(const AllocArgs &a, int pass, hipStream_t s) {
    hipLaunchKernelGGL(k_alloc_count, dim3(grid_for(a.J, 256, 1024)), dim3(256), 0, s, a, pass);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_alloc_decide, dim3(1), dim3(256), 0, s, a, pass);
    return hipGetLastError();
}

hipError_t launch_alloc_final(const AllocArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_alloc_final, dim3((unsigned)a.nblk), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_alloc_totals, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_reorder(const ReorderArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_reorder_scan, dim3(1), dim3(1024), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_reorder_scatter, dim3((unsigned)a.nblk), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Compute units of the current device, cached per device.
constexpr int kMaxDevices = 64;
static int64_t device_cus() {
    static int cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    if (cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    cache[dev] = cus;
    return cus;
}

// Grid of a codec launch over n super-groups: whole "waves" of the kernel's
// resident blocks (a partial last wave leaves CUs idle at the end): one wave
// while that gives each block fewer than about 18 grid-stride iterations, else
// two.  Measured on launches of 1.6e5 to 2e6 super-groups (BERT-, LLaMA- and
// Gemma-shaped parts): one wave up to 3e5, two from 4.9e5 on, 3-9% faster
// than a fixed grid at the small end.
static dim3 codec_grid(int64_t n, int64_t blocks_per_cu, int64_t sg_per_block) {
    const int64_t wave = device_cus() * blocks_per_cu;
    int64_t waves = (n + wave * sg_per_block * 6) / (wave * sg_per_block * 12);
    waves = waves < 1 ? 1 : (waves > 2 ? 2 : waves);
    return dim3(grid_for(n, sg_per_block, wave * waves));
}

// With a second output (both children of a hop's part) the grid holds each
// child's own grid, one after the other, and split marks the boundary.
template <int MODE, int LOCAL, bool WIDE>
static hipError_t launch_codec_w(const CodecArgs &a, int64_t max_sg, hipStream_t s) {
    using Shape = CodecShape<MODE, LOCAL, WIDE>;
    const dim3 one = codec_grid(max_sg, Shape::blocks_per_cu, Shape::sg_per_block);
    CodecArgs b = a;
    b.split = one.x;
    const dim3 grid(a.out2 ? 2 * one.x : one.x);
    hipLaunchKernelGGL((k_codec<MODE, LOCAL, WIDE>), grid, dim3(Shape::threads), 0, s, b);
    return hipGetLastError();
}

template <int MODE, int LOCAL>
static hipError_t launch_codec_t(const CodecArgs &a, int64_t max_sg, bool wide, hipStream_t s) {
    return wide ? launch_codec_w<MODE, LOCAL, true>(a, max_sg, s) : launch_codec_w<MODE, LOCAL, false>(a, max_sg, s);
}

hipError_t launch_codec(const CodecArgs &a, int mode, int local, int64_t max_sg, bool w, hipStream_t s) {
    if (mode == kCompress && local == kLocalBF16) return launch_codec_t<kCompress, kLocalBF16>(a, max_sg, w, s);
    if (mode == kCompress && local == kLocalF32) return launch_codec_t<kCompress, kLocalF32>(a, max_sg, w, s);
    if (mode == kHop && local == kLocalBF16) return launch_codec_t<kHop, kLocalBF16>(a, max_sg, w, s);
    if (mode == kHop && local == kLocalF32) return launch_codec_t<kHop, kLocalF32>(a, max_sg, w, s);
    if (mode == kHop && local == kLocalPacked) return launch_codec_t<kHop, kLocalPacked>(a, max_sg, w, s);
    if (mode == kHop && local == kLocalPartial) return launch_codec_t<kHop, kLocalPartial>(a, max_sg, w, s);
    if (mode == kPartial && local == kLocalBF16) return launch_codec_t<kPartial, kLocalBF16>(a, max_sg, w, s);
    if (mode == kPartial && local == kLocalF32) return launch_codec_t<kPartial, kLocalF32>(a, max_sg, w, s);
    if (mode == kPartial && local == kLocalPartial) return launch_codec_t<kPartial, kLocalPartial>(a, max_sg, w, s);
    if (mode == kHopFinal && local == kLocalBF16) return launch_codec_t<kHopFinal, kLocalBF16>(a, max_sg, w, s);
    if (mode == kHopFinal && local == kLocalF32) return launch_codec_t<kHopFinal, kLocalF32>(a, max_sg, w, s);
    if (mode == kHopFinal && local == kLocalPacked) return launch_codec_t<kHopFinal, kLocalPacked>(a, max_sg, w, s);
    if (mode == kHopFinal && local == kLocalPartial) return launch_codec_t<kHopFinal, kLocalPartial>(a, max_sg, w, s);
    if (mode == kFinalize) {
        // finalize streams at memory speed: 8 blocks per CU
        const dim3 grid(grid_for(max_sg, kSGPerBlock, device_cus() * 8));
        if (w) hipLaunchKernelGGL(k_finalize<true>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_finalize<false>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace dq
