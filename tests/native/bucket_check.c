/* The interval search's linear bucket (codec kernels): for class tables of
 * NB = 1024 and 8192 buckets, bucket(v) = NB/2 + rne(v M) with M = NB/2 - 1
 * is computed as the bits of fl(fma(v, M, 2^23 + NB/2)) masked to NB - 1.
 * Checked here for every fp32 v from -(1 + 16 ulp) to 1 + 16 ulp, in
 * increasing order: the masked bits equal NB/2 + rint(v M) (v M is exact in
 * double, rint rounds to nearest even), and the bucket never decreases.
 * Prints: values checked, mismatches, decreases, and whether NaN and the
 * infinities land inside the table. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits_of(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
static float float_of(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }

int main(void) {
    const int NBs[2] = {1024, 8192};
    unsigned long long checked = 0, bad = 0, dec = 0;
    int prev[2] = {-1, -1};
    const uint32_t one = bits_of(1.0f);
    /* negative values from -(1 + 16 ulp) up to -0, then +0 up to 1 + 16 ulp */
    for (int side = 0; side < 2; side++) {
        for (uint32_t k = 0; k <= one + 16; k++) {
            const uint32_t b = side == 0 ? (0x80000000u | (one + 16 - k)) : k;
            const float v = float_of(b);
            for (int c = 0; c < 2; c++) {
                const int NB = NBs[c], M = NB / 2 - 1;
                const float x = fmaf(v, (float)M, 8388608.0f + (float)(NB / 2));
                const int idx = (int)(bits_of(x) & (uint32_t)(NB - 1));
                const int ref = NB / 2 + (int)rint((double)v * (double)M);
                if (idx != ref) bad++;
                if (idx < prev[c]) dec++;
                prev[c] = idx;
            }
            checked++;
        }
    }
    int special_ok = 1;
    const float sp[3] = {NAN, INFINITY, -INFINITY};
    for (int i = 0; i < 3; i++)
        for (int c = 0; c < 2; c++) {
            const int NB = NBs[c];
            const float x = fmaf(sp[i], (float)(NB / 2 - 1), 8388608.0f + (float)(NB / 2));
            const uint32_t idx = bits_of(x) & (uint32_t)(NB - 1);
            if (idx >= (uint32_t)NB) special_ok = 0;
        }
    printf("%llu %llu %llu %d\n", checked, bad, dec, special_ok);
    return 0;
}
