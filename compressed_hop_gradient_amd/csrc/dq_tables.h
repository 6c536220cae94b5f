// dq_tables.h -- non-uniform level tables, built at compile time.
//
// DynamiQ places more quantisation levels near zero (scribe notes, "Key idea
// and contribution"); the pith.science ledger names the level set
// Q = {f(eps, r)} without giving f or eps.  Reading used here: 2^q symmetric
// levels on the grid u_r = (2r + 1 - 2^q) / (2^q - 1), level
// sign(u) * phi(|u|) with phi(t) = t * (1/2 + t/2) (eps = 1/2), evaluated in
// double precision and rounded once to float.  W[r] = 65536 / (L[r+1] - L[r])
// (double, rounded once) turns the position inside an interval into a 16-bit
// dither threshold with a single multiply.
//
// The search rows serve the interval search of the encoder: row r holds
// (L[r], L[r+1], W[r], W[r+1]); in the last row (r = 2^q - 2) the "next level"
// is +inf so the search never steps past the last interval.
#pragma once

namespace dq {

struct Row4 { float l0, l1, w0, w1; };

struct LevelTables {
    float L2[4], L4[16], L8[256];
    float W2[3];
    Row4 R4[15];
    Row4 R8[255];
};

constexpr double level_value(int r, int Q) {
    double u = double(2 * r + 1 - Q) / double(Q - 1);
    double t = u < 0 ? -u : u;
    double ph = t * (0.5 + 0.5 * t);
    return u < 0 ? -ph : ph;
}

constexpr float level_f(int r, int Q) { return float(level_value(r, Q)); }

constexpr float weight_f(int r, int Q) {
    return float(65536.0 / (double(level_f(r + 1, Q)) - double(level_f(r, Q))));
}

constexpr Row4 search_row(int r, int Q) {
    return Row4{level_f(r, Q), r + 1 <= Q - 2 ? level_f(r + 1, Q) : __builtin_huge_valf(),
                weight_f(r, Q), r + 1 <= Q - 2 ? weight_f(r + 1, Q) : 0.0f};
}

constexpr LevelTables make_tables() {
    LevelTables t{};
    for (int r = 0; r < 4; r++) t.L2[r] = level_f(r, 4);
    for (int r = 0; r < 16; r++) t.L4[r] = level_f(r, 16);
    for (int r = 0; r < 256; r++) t.L8[r] = level_f(r, 256);
    for (int r = 0; r < 3; r++) t.W2[r] = weight_f(r, 4);
    for (int r = 0; r < 15; r++) t.R4[r] = search_row(r, 16);
    for (int r = 0; r < 255; r++) t.R8[r] = search_row(r, 256);
    return t;
}

constexpr LevelTables kLevelTables = make_tables();

// spot checks of the closed form at compile time
static_assert(kLevelTables.L2[0] == -1.0f && kLevelTables.L2[3] == 1.0f, "endpoints");
static_assert(kLevelTables.L2[2] == float(2.0 / 9.0), "phi(1/3) = 2/9");
static_assert(kLevelTables.L8[255] == 1.0f && kLevelTables.L8[128] == -kLevelTables.L8[127], "symmetry");

}  // namespace dq
