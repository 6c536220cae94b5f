/* The interval search's linear bucket (codec kernels): for class tables of
 * NB = 1024 and 8192 buckets, bucket(v) = NB/2 + rne(v M) with M = NB/2 - 1
 * is computed as the bits of clamp01(fl(fma(v, M 2^-149, (NB/2) 2^-149))):
 * the FMA rounds on the subnormal grid, whose spacing 2^-149 is one unit of
 * the bits, and the result's clamp to [0, 1] sends NaN to +0.
 * Checked here in increasing order of v from -(1 + 1024 ulp) to
 * 1 + 1024 ulp (the encoder's |v| is at most 1 + 2^-22;
 * 1 + 1024 ulp = 1 + 2^-13): every fp32 v with |v| >= 2^-14, where v M can
 * round to a nonzero integer, and every 64th bit pattern below, where
 * |v M| < 1/4 and the key is NB/2.  The bits must equal NB/2 + rint(v M)
 * (v M is exact in double, rint rounds to nearest even), lie in [0, NB), and
 * never decrease.  Prints: values checked, mismatches, decreases,
 * out-of-table keys, and whether every NaN (both signs, quiet and
 * signalling payloads) lands in bucket 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits_of(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
static float float_of(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }

/* the clamp output modifier of the GPU's FMA: NaN -> +0, then [0, 1] */
static float clamp01(float x) { return x != x ? 0.0f : (x < 0.0f ? 0.0f : (x > 1.0f ? 1.0f : x)); }

static uint32_t key(float v, int NB) {
    const float m = float_of((uint32_t)(NB / 2 - 1)), h = float_of((uint32_t)(NB / 2));
    return bits_of(clamp01(fmaf(v, m, h)));
}

/* The sweep in increasing order of v, as four segments of bit patterns:
   negative |v| >= 2^-14 (every pattern, magnitude falling), negative
   |v| < 2^-14 (every 64th), positive |v| < 2^-14 (every 64th), positive
   |v| >= 2^-14 (every pattern). */
static uint32_t g_top, g_b14;
static uint64_t seg_len(int s) {
    return (s == 0 || s == 3) ? (uint64_t)(g_top - g_b14) + 1 : (uint64_t)(g_b14 + 63) / 64;
}
static float sweep_value(uint64_t i) {
    int s = 0;
    while (i >= seg_len(s)) i -= seg_len(s++);
    switch (s) {
    case 0: return float_of(0x80000000u | (uint32_t)(g_top - i));
    case 1: return float_of(0x80000000u | (uint32_t)(g_b14 - 1 - 64 * i));
    case 2: return float_of((uint32_t)(64 * i));
    default: return float_of((uint32_t)(g_b14 + i));
    }
}

int main(void) {
    const int NBs[2] = {1024, 8192};
    g_top = bits_of(1.0f) + 1024;
    g_b14 = bits_of(0x1p-14f);
    const uint64_t total = seg_len(0) + seg_len(1) + seg_len(2) + seg_len(3);
    /* x86 takes a slow assist for every subnormal result: the sweep is cut
       into chunks checked in parallel, each for its own order, and the
       chunks' end keys are compared afterwards */
    enum { kChunks = 256 };
    static uint32_t first[kChunks][2], last[kChunks][2];
    unsigned long long bad = 0, dec = 0, out = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad, dec, out)
    for (int ch = 0; ch < kChunks; ch++) {
        const uint64_t lo = total * ch / kChunks, hi = total * (ch + 1) / kChunks;
        for (uint64_t i = lo; i < hi; i++) {
            const float v = sweep_value(i);
            for (int c = 0; c < 2; c++) {
                const int NB = NBs[c], M = NB / 2 - 1;
                const uint32_t idx = key(v, NB);
                const long long ref = NB / 2 + (long long)rint((double)v * (double)M);
                if ((long long)idx != ref) bad++;
                if (idx >= (uint32_t)NB) out++;
                if (i == lo) first[ch][c] = idx;
                else if (idx < last[ch][c]) dec++;
                last[ch][c] = idx;
            }
        }
    }
    for (int ch = 1; ch < kChunks; ch++)
        for (int c = 0; c < 2; c++)
            if (first[ch][c] < last[ch - 1][c]) dec++;
    int nan_ok = 1;
    const uint32_t nans[6] = {0x7FC00000u, 0xFFC00000u, 0x7F800001u, 0xFF800001u, 0x7FFFFFFFu, 0xFFFFFFFFu};
    for (int i = 0; i < 6; i++)
        for (int c = 0; c < 2; c++)
            if (key(float_of(nans[i]), NBs[c]) != 0u) nan_ok = 0;
    printf("%llu %llu %llu %llu %d\n", (unsigned long long)total, bad, dec, out, nan_ok);
    return 0;
}
