/* Exhaustive host check of the sampler's scaling identity: for every fp32
 * z (all 2^32 bit patterns but NaN) and each temperature T given on the
 * command line, fl32(fl64(z) * fl64(1 / T)) must equal the IEEE fp32
 * quotient z / T.  The sampler kernels compute s = z / T by the double
 * product when |z| >= 2^-125 T; this checks every z, the smaller ones too.
 *
 *   gcc -O2 -o scaling_exhaustive tests/scaling_exhaustive.c
 *   ./scaling_exhaustive 0.8 0.7 1.0 6.0
 *
 * Prints one line per temperature; exit status 1 on any mismatch.  Test
 * infrastructure only: nothing in the library uses it. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_to_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(int argc, char **argv)
{
    int failed = 0;
    for (int k = 1; k < argc; ++k) {
        const float T = strtof(argv[k], NULL);
        const double inv = 1.0 / (double)T;
        unsigned long long bad = 0;
        for (uint64_t u = 0; u < (1ull << 32); ++u) {
            const float z = bits_to_float((uint32_t)u);
            if (z != z) continue;
            volatile float quotient = z / T;   /* (volatile: the fp32 division itself) */
            const float product = (float)((double)z * inv);
            if (float_to_bits(quotient) != float_to_bits(product)) {
                if (bad < 5) printf("T=%a z=%a quotient=%a product=%a\n", T, z, (float)quotient, product);
                ++bad;
            }
        }
        printf("T=%g (%a): %llu mismatches over every non-NaN z\n", T, T, bad);
        fflush(stdout);
        failed |= bad != 0;
    }
    return failed;
}
