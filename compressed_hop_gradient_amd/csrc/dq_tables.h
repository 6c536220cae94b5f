// dq_tables.h -- non-uniform level tables and the bucket index of the
// interval search; constexpr functions used at compile time (the default
// shape, checked by static_assert) and on the host at plan set-up (any shape).
//
// DynamiQ places more quantisation levels near zero (scribe notes, "Key idea
// and contribution"); the pith.science ledger names the level set
// Q = {f(eps, r)} without giving f or eps.  Reading used here: 2^q symmetric
// levels on the grid u_r = (2r + 1 - 2^q) / (2^q - 1), level
// sign(u) * phi(|u|) with phi(t) = t * (eps + (1 - eps) t), eps = 1/2 unless
// the plan sets another value in (0, 1], evaluated in double precision and
// rounded once to float.  W[r] = 65536 / (L[r+1] - L[r]) (double, rounded
// once) turns the position inside an interval into a 16-bit dither threshold
// with a single multiply.
//
// The encoder's interval search uses CL[r] = L[r] for r <= 2^q - 2 and
// CL[2^q - 1] = +inf (so the search never steps past the last interval), and
// the pairs LW[r] = (L[r], W[r]) of the interval it lands in.
#pragma once

namespace dq {

struct Pair { float l, w; };

struct LevelTables {
    float L2[4], L4[16], L8[256];
    float W2[3];
    float CL4[16], CL8[256];
    Pair LW4[15], LW8[255];
};

constexpr double kDefaultEps = 0.5;

constexpr double level_value(int r, int Q, double eps) {
    double u = double(2 * r + 1 - Q) / double(Q - 1);
    double t = u < 0 ? -u : u;
    double ph = t * (eps + (1.0 - eps) * t);
    return u < 0 ? -ph : ph;
}

constexpr float level_f(int r, int Q, double eps) { return float(level_value(r, Q, eps)); }

constexpr float weight_f(int r, int Q, double eps) {
    return float(65536.0 / (double(level_f(r + 1, Q, eps)) - double(level_f(r, Q, eps))));
}

constexpr float compare_level(int r, int Q, double eps) {
    return r <= Q - 2 ? level_f(r, Q, eps) : __builtin_huge_valf();
}

constexpr LevelTables make_tables(double eps) {
    LevelTables t{};
    for (int r = 0; r < 4; r++) t.L2[r] = level_f(r, 4, eps);
    for (int r = 0; r < 16; r++) t.L4[r] = level_f(r, 16, eps);
    for (int r = 0; r < 256; r++) t.L8[r] = level_f(r, 256, eps);
    for (int r = 0; r < 3; r++) t.W2[r] = weight_f(r, 4, eps);
    for (int r = 0; r < 16; r++) t.CL4[r] = compare_level(r, 16, eps);
    for (int r = 0; r < 256; r++) t.CL8[r] = compare_level(r, 256, eps);
    for (int r = 0; r < 15; r++) t.LW4[r] = Pair{level_f(r, 16, eps), weight_f(r, 16, eps)};
    for (int r = 0; r < 255; r++) t.LW8[r] = Pair{level_f(r, 256, eps), weight_f(r, 256, eps)};
    return t;
}

constexpr LevelTables kLevelTables = make_tables(kDefaultEps);

// ---------------------------------------------------------------------------
// Bucket index for the interval search, linear in v.  Class NL (16 or 256
// levels) has NB buckets; bucket(v) = NB/2 + rne(v M) with M = NB/2 - 1 and
// rne the round-to-nearest-even to an integer, so every |v| <= 1 + 2^-13
// falls in [1, NB - 1].  The kernels compute it in one instruction: x =
// fl(fma(v, M 2^-149, (NB/2) 2^-149)) lies on the subnormal grid, where the
// bits of a float count units of 2^-149, so the bits of x are bucket(v); the
// FMA's clamp to [0, 1] sends NaN to bucket 0.  bucket() is non-decreasing in
// v; when the interior levels
// L[1] < ... < L[NL-2] fall in strictly increasing buckets (checked for the
// plan's level shape), the entry est[k] = #{interior levels in buckets < k}
// is r(v) or r(v) - 1 for every v in bucket k, and one compare with
// CL[est + 1] (CL[NL - 1] = +inf) decides.
// ---------------------------------------------------------------------------

constexpr int bucket_count(int NL) { return NL == 256 ? 8192 : 1024; }

// rne(v * M) for |v| < 2 and 0 < M < 2^13, in exact integer arithmetic on the
// bits of v (the product m M of the 24-bit significand fits 37 bits)
constexpr long long rne_times(float v, int M) {
    const unsigned b = __builtin_bit_cast(unsigned, v);
    const int e = (int)((b >> 23) & 0xFFu);
    const unsigned long long m = (unsigned long long)(b & 0x7FFFFFu) | (e ? 0x800000ull : 0ull);
    const unsigned long long p = m * (unsigned long long)M;
    const int s = 150 - (e ? e : 1);                   // value = p 2^-s
    long long q = 0;
    if (s <= 0) {
        q = (long long)(p << -s);
    } else if (s < 64) {
        const unsigned long long fl = p >> s, rem = p & ((1ull << s) - 1ull), half = 1ull << (s - 1);
        q = (long long)(fl + ((rem > half || (rem == half && (fl & 1ull))) ? 1ull : 0ull));
    }
    return (b >> 31) ? -q : q;
}

template <int NL>
constexpr int bucket_of(float v) {
    constexpr int NB = bucket_count(NL);
    return NB / 2 + (int)rne_times(v, NB / 2 - 1);
}

template <int NL>
struct BucketTable {
    unsigned char est[bucket_count(NL)];
};

// est[k] = number of interior levels L[1..NL-2] whose bucket is below k, by a
// sweep over the buckets
template <int NL>
constexpr BucketTable<NL> make_buckets(double eps) {
    BucketTable<NL> t{};
    int r = 0;
    for (int k = 0; k < bucket_count(NL); k++) {
        while (r + 1 <= NL - 2 && bucket_of<NL>(level_f(r + 1, NL, eps)) < k) r++;
        t.est[k] = (unsigned char)r;
    }
    return t;
}

// the interior levels fall in strictly increasing buckets (at most one level
// boundary per bucket)
template <int NL>
constexpr bool buckets_hold_one_boundary(double eps) {
    for (int r = 1; r + 1 <= NL - 2; r++)
        if (bucket_of<NL>(level_f(r, NL, eps)) >= bucket_of<NL>(level_f(r + 1, NL, eps))) return false;
    return true;
}

// Everything the codec kernels read from their tables; one copy per plan in
// the workspace (built on the host for the plan's level shape).
// The tables as a codec block holds them in LDS: decode levels, compare
// levels, (L, W) pairs and bucket entries of each class.  The workspace keeps
// a byte image of it so that a block loads its copy with 16-byte reads.
struct alignas(16) SharedTables {
    // decode of a whole code byte: four 2-bit codes, two 4-bit codes
    // (code k of the byte sits at bits q k, LSB first)
    float quad2[256][4];
    float pair4[256][2];
    float dec2[4];
    Pair lw2[3];
    float dec4[16];
    float dec8[256];
    float cl4[16];
    float cl8[256];
    Pair lw4[15];
    Pair lw8[255];
    unsigned char b4[bucket_count(16)];
    unsigned char b8[bucket_count(256)];
};
static_assert(sizeof(SharedTables) % 16 == 0, "the image is copied in 16-byte pieces");

struct DeviceTables {
    LevelTables lev;
    BucketTable<256> b8;
    BucketTable<16> b4;
    SharedTables lds;      // the same tables in the LDS layout (filled by the device)
};

constexpr bool level_shape_ok(double eps) {
    return eps > 0.0 && eps <= 1.0 && buckets_hold_one_boundary<16>(eps) &&
           buckets_hold_one_boundary<256>(eps);
}

constexpr DeviceTables make_device_tables(double eps) {
    return DeviceTables{make_tables(eps), make_buckets<256>(eps), make_buckets<16>(eps), SharedTables{}};
}

static_assert(level_shape_ok(kDefaultEps), "default level shape: one boundary per bucket");  // needs -fconstexpr-steps
static_assert(level_shape_ok(1.0), "uniform grid: one boundary per bucket");

// spot checks of the closed form at compile time (default shape)
static_assert(kLevelTables.L2[0] == -1.0f && kLevelTables.L2[3] == 1.0f, "endpoints");
static_assert(kLevelTables.L2[2] == float(2.0 / 9.0), "phi(1/3) = 2/9");
static_assert(kLevelTables.L8[255] == 1.0f && kLevelTables.L8[128] == -kLevelTables.L8[127], "symmetry");

}  // namespace dq
