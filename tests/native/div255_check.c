/* Checks, for every non-negative finite fp32 A in the given exponent-field
 * ranges, that the correctly rounded quotient fl(A / 255) equals
 *   y = fl(A * R),  r = fma(-y, 255, A),  q = fma(r, R, y),  R = fl(1 / 255),
 * the two-FMA form the codec kernels use for the scale unit, and that one
 * raise of the quotient to the next float always reaches fl(255 s) >= A (the
 * kernels take at most one raise).  Prints the number of values checked, the
 * number whose quotient differs and the number that would need a second raise.
 * usage: div255_check e_lo e_hi [e_lo e_hi ...]  (exponent fields, inclusive) */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(int argc, char **argv) {
    const float R = 1.0f / 255.0f;
    unsigned long long checked = 0, bad = 0, second = 0;
    for (int a = 1; a + 1 < argc; a += 2) {
        const long lo = strtol(argv[a], NULL, 10), hi = strtol(argv[a + 1], NULL, 10);
        for (long e = lo; e <= hi; e++) {
            for (uint32_t m = 0; m < (1u << 23); m++) {
                const float A = from_bits(((uint32_t)e << 23) | m);
                const float y = A * R;
                const float r = fmaf(-y, 255.0f, A);
                const float q = fmaf(r, R, y);
                if (to_bits(q) != to_bits(A / 255.0f)) bad++;
                float s = A / 255.0f;
                if (255.0f * s < A) s = from_bits(to_bits(s) + 1u);
                if (255.0f * s < A) second++;
                checked++;
            }
        }
    }
    printf("%llu %llu %llu\n", checked, bad, second);
    return 0;
}
