// Philox4x32-10 from rocRAND's header-only engine, run on the host: an
// implementation independent of the oracle's.  Reads lines "x y z w k0 k1"
// (decimal counter words and key words) from stdin and prints the four output
// words of each, in hexadecimal.  rocrand_init(seed, subsequence, offset)
// puts offset / 4 into the counter's words x, y and the subsequence into its
// words z, w; the key is (seed low 32 bits, seed high 32 bits).
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
    unsigned long long v[6];
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5]) == 6) {
        const unsigned long long seed = v[4] | (v[5] << 32);
        const unsigned long long subsequence = v[2] | (v[3] << 32);
        const unsigned long long block = v[0] | (v[1] << 32);
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subsequence, 4ull * block, &st);   // 4 * block wraps mod 2^64: the
        unsigned int out[4];                                   // engine keeps offset / 4 only as
        for (int i = 0; i < 4; i++) out[i] = rocrand(&st);     // 64 bits, so block < 2^62 here
        std::printf("%08x %08x %08x %08x\n", out[0], out[1], out[2], out[3]);
    }
    return 0;
}
