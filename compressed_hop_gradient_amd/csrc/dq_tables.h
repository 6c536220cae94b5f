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
// Bucket index for the interval search.  The key of v is 7 mantissa bits and
// the exponent of |v| (fp32 bits >> 16), offset so that key 0 holds every
// |v| < 2^-12 and key kKeyMax holds |v| = 1.  Each bucket is at most 2^-7
// wide relative to its start; for every level shape the plan accepts, each
// bucket contains at most one level boundary (checked when the tables are
// built), so the table gives r or r - 1 and one compare with the next level
// decides.  Entry 2k serves v >= 0 in bucket k, entry 2k + 1 serves v < 0.
// ---------------------------------------------------------------------------

constexpr int kKeyBase = 0x3980;              // fp32 bits of 2^-12, >> 16
constexpr int kKeyMax = 0x3F80 - kKeyBase;    // key of 1.0
// The kernels take the key from fp32 bits 29..16 (bit 30 is clear for every
// |v| < 2), so a key never exceeds 0x3FFF - kKeyBase and needs no upper
// clamp.  Keys above kKeyMax hold |v| > 1 + 2^-7, which finite inputs never
// produce (|v| exceeds 1 by at most two ulps); they repeat the entries of
// |v| = 1.  Non-finite inputs (flagged by the stats) land somewhere in the
// table and give meaningless but in-bounds codes.
constexpr int kKeys = 0x4000 - kKeyBase;

constexpr float key_lo(int k) {
    return k == 0 ? 0.0f : (k >= kKeyMax ? 1.0f : __builtin_bit_cast(float, (unsigned)(k + kKeyBase) << 16));
}
constexpr float key_hi(int k) {
    return k >= kKeyMax ? 1.0f : __builtin_bit_cast(float, (unsigned)(k + 1 + kKeyBase) << 16);
}

template <int NL>
struct BucketTable {
    unsigned char est[2 * kKeys];
};

// est for v >= 0 in bucket k: largest r <= NL-2 with L[r] <= key_lo(k);
// est for v < 0: largest r <= NL-2 with L[r] <= -key_hi(k).  Both by sweeps.
template <int NL>
constexpr BucketTable<NL> make_buckets(double eps) {
    BucketTable<NL> t{};
    int r = 0;
    for (int k = 0; k < kKeys; k++) {
        const float lo = key_lo(k);
        while (r + 1 <= NL - 2 && level_f(r + 1, NL, eps) <= lo) r++;
        t.est[2 * k] = (unsigned char)r;
    }
    r = 0;
    for (int k = kKeys - 1; k >= 0; k--) {
        const float nh = -key_hi(k);
        while (r + 1 <= NL - 2 && level_f(r + 1, NL, eps) <= nh) r++;
        t.est[2 * k + 1] = (unsigned char)r;
    }
    return t;
}

// at most one level boundary inside every bucket (sweeps over the levels)
template <int NL>
constexpr bool buckets_hold_one_boundary(double eps) {
    // positive side: levels in (key_lo(k), key_hi(k))
    int r = 0;
    for (int k = 0; k < kKeys; k++) {
        const float lo = key_lo(k), hi = key_hi(k);
        while (r < NL && level_f(r, NL, eps) <= lo) r++;
        int c = 0;
        for (int q = r; q < NL && level_f(q, NL, eps) < hi; q++) c++;
        if (c > 1) return false;
    }
    // negative side: levels in (-key_hi(k), -key_lo(k)], by a sweep from the
    // most negative level up (buckets k = kKeys-1 .. 0 cover increasing v)
    r = 0;
    for (int k = kKeys - 1; k >= 0; k--) {
        const float a = -key_hi(k), b = -key_lo(k);
        while (r < NL && level_f(r, NL, eps) <= a) r++;
        int c = 0;
        for (int q = r; q < NL && level_f(q, NL, eps) <= b; q++) c++;
        if (c > 1) return false;
    }
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
    unsigned char b4[2 * kKeys];
    unsigned char b8[2 * kKeys];
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
