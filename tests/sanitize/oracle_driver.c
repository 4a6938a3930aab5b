/* oracle_driver.c -- runs the C oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test-only; built by tests/test_sanitize.py with
 * gcc -fsanitize=address,undefined).  Random masks of 1 to 4 axes, densities
 * from all background to none, unit and dyadic spacings: the separable
 * routine must equal the brute force exactly, and every returned feature must
 * attain the minimum.  Exit status 0 when every case agrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/oracle_edt.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* splitmix64 */
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(void) {
    const double dens[] = {0.0, 0.01, 0.1, 0.5, 1.0};
    const double samp[4] = {2.5, 1.0, 0.5, 1.5};
    int bad = 0, cases = 0;
    for (int it = 0; it < 400; ++it) {
        const int ndim = 1 + (int)(next_u64() % 4);
        int64_t shape[4], n = 1;
        for (int k = 0; k < ndim; ++k) {
            shape[k] = 1 + (int64_t)(next_u64() % (ndim >= 3 ? 9 : 40));
            n *= shape[k];
        }
        const double p = dens[it % 5];
        uint8_t* m = (uint8_t*)malloc((size_t)n);
        for (int64_t i = 0; i < n; ++i) m[i] = ((double)(next_u64() >> 11) / 9007199254740992.0) < p ? 0 : 1;
        double* a = (double*)malloc(sizeof(double) * (size_t)n);
        double* b = (double*)malloc(sizeof(double) * (size_t)n);
        int32_t* fa = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n * ndim));
        int32_t* fb = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n * ndim));
        const double* s = (it & 1) ? samp : NULL;
        if (oracle_edt_separable(m, ndim, shape, s, a, fa) || oracle_edt_brute(m, ndim, shape, s, b, fb)) {
            ++bad;
        } else {
            for (int64_t i = 0; i < n; ++i) {
                if (a[i] != b[i]) { ++bad; break; }
                /* the feature attains the minimum */
                int64_t rem = i;
                double d = 0.0;
                for (int k = ndim - 1; k >= 0; --k) {
                    const int64_t c = rem % shape[k];
                    rem /= shape[k];
                    const double t = (double)(c - fa[i * ndim + k]);
                    const double sk = s ? s[k] : 1.0;
                    d += sk * sk * t * t;
                }
                if (d != a[i]) { ++bad; break; }
            }
        }
        ++cases;
        free(m); free(a); free(b); free(fa); free(fb);
    }
    printf("oracle driver: %d cases, %d disagreements\n", cases, bad);
    return bad ? 1 : 0;
}
