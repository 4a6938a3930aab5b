// host_model_driver.cpp -- runs the host model of the envelope kernels
// (tests/host_model/host_model.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer (test-only; built by tests/test_sanitize.py).
// Random lines of candidate values, every chunk layout and reach the kernels
// use, under both metrics (squared Euclidean and chessboard): each owner must
// attain the minimum over all candidates.  Exit status 0 when every line
// agrees.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../host_model/host_model.cpp"

static uint64_t st = 0xD1B54A32D192ED03ull;
static uint64_t next_u64() {   // splitmix64
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main() {
    int bad = 0, lines = 0;
    const int Ls[] = {1, 2, 31, 33, 100, 257, 1000};
    const int Ks[] = {8, 16, 32, 64};
    const int reaches[] = {0, 1, 8};
    for (int L : Ls) {
        for (int K : Ks) {
            for (int reach : reaches) {
                for (int rep = 0; rep < 3; ++rep) {
                    // slots past the line (rep 1) stay empty; spacing 2.5 on rep 1
                    const int G = (L + K - 1) / K + (rep == 1 ? 3 : 0);
                    const double s2l = rep == 1 ? 6.25 : 1.0;
                    std::vector<double> f(L);
                    for (int i = 0; i < L; ++i) {
                        const uint64_t r = next_u64();
                        f[i] = (r % 5 == 0) ? INFINITY : (double)((r >> 8) % (uint64_t)(4 * L * L + 1));
                    }
                    if (rep == 2) for (int i = 0; i < L; ++i) f[i] = 49.0;   // every candidate a member
                    std::vector<int32_t> own(L);
                    if (model_envelope_line(f.data(), L, s2l, K, G, reach, own.data()) != 0) { ++bad; continue; }
                    for (int q = 0; q < L; ++q) {
                        double best = INFINITY;
                        for (int j = 0; j < L; ++j) best = fmin(best, s2l * (double)(q - j) * (q - j) + f[j]);
                        const int o = own[q];
                        const double v = o < 0 ? INFINITY : s2l * (double)(q - o) * (q - o) + f[o];
                        if (v != best) { ++bad; break; }
                    }
                    ++lines;
                }
            }
        }
    }
    // the chessboard metric: g[j] < 0 is no source; owners must attain
    // min_j max(g_j, |q - j|), and the value the model forms must equal it
    for (int L : Ls) {
        for (int K : Ks) {
            for (int reach : reaches) {
                for (int rep = 0; rep < 3; ++rep) {
                    std::vector<int32_t> g(L);
                    for (int i = 0; i < L; ++i) {
                        const uint64_t r = next_u64();
                        g[i] = (r % 5 == 0) ? -1 : (int32_t)((r >> 8) % (uint64_t)(2 * L + 1));
                    }
                    if (rep == 1) for (int i = 0; i < L; ++i) g[i] = (int32_t)((next_u64() >> 8) % 4);
                    if (rep == 2) for (int i = 0; i < L; ++i) g[i] = 7;   // flat bottoms everywhere
                    const int G = (L + K - 1) / K + (rep == 1 ? 3 : 0);
                    std::vector<int32_t> own(L), val(L);
                    if (model_linf_envelope_lines(g.data(), 1, L, K, G, reach, own.data(), val.data()) != 0) {
                        ++bad;
                        continue;
                    }
                    for (int q = 0; q < L; ++q) {
                        int best = -1;
                        for (int j = 0; j < L; ++j) {
                            if (g[j] < 0) continue;
                            const int v = g[j] > abs(q - j) ? g[j] : abs(q - j);
                            if (best < 0 || v < best) best = v;
                        }
                        const int o = own[q];
                        const int v = o < 0 ? -1 : (g[o] > abs(q - o) ? g[o] : abs(q - o));
                        if (v != best || val[q] != best || (o >= 0 && g[o] < 0)) { ++bad; break; }
                    }
                    ++lines;
                }
            }
        }
    }
    printf("host model driver: %d lines, %d disagreements\n", lines, bad);
    return bad ? 1 : 0;
}
