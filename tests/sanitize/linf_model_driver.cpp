// linf_model_driver.cpp -- runs the host model of the chessboard line step
// (tests/host_model/linf_model.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer (test-only; built by tests/test_sanitize.py).
// Random lines of sources: h and the returned source must match the
// definition min_j max(g(j), |q - j|).  Exit status 0 when every line agrees.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../host_model/linf_model.cpp"

static uint64_t st = 0x632BE59BD9B4E019ull;
static uint64_t next_u64() {   // splitmix64
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main() {
    int bad = 0, lines = 0;
    const int Ls[] = {1, 7, 8, 9, 17, 64, 100, 513, 2000};
    const int gmaxs[] = {0, 5, 300, 65534};
    for (int L : Ls) {
        for (int gmax : gmaxs) {
            for (int rep = 0; rep < 6; ++rep) {
                std::vector<int32_t> g(L), h(L), j(L);
                const uint64_t p = 1 + next_u64() % 100;   // percent of sources
                bool any = false;
                for (int i = 0; i < L; ++i) {
                    g[i] = (int)(next_u64() % 100) < (int)p ? (int)(next_u64() % (uint64_t)(gmax + 1)) : -1;
                    any = any || g[i] >= 0;
                }
                if (!any) g[L / 2] = 0;
                if (model_linf_line(g.data(), L, h.data(), j.data()) != 0) { ++bad; continue; }
                for (int q = 0; q < L; ++q) {
                    int best = 1 << 30;
                    for (int k = 0; k < L; ++k) {
                        if (g[k] < 0) continue;
                        const int v = g[k] > abs(q - k) ? g[k] : abs(q - k);
                        if (v < best) best = v;
                    }
                    const int jq = j[q];
                    const bool ok = h[q] == best && jq >= 0 && jq < L && g[jq] >= 0 &&
                                    (g[jq] > abs(q - jq) ? g[jq] : abs(q - jq)) == best;
                    if (!ok) { ++bad; break; }
                }
                ++lines;
            }
        }
    }
    printf("linf model driver: %d lines, %d disagreements\n", lines, bad);
    return bad ? 1 : 0;
}
