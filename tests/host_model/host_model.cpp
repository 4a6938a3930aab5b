// host_model.cpp -- test-only host build of the envelope machinery in
// exact_euclidean_distance_amd/csrc/envelope.h.
//
// Runs, for one line at a time, the same functions the envelope kernels run
// (build_chunk, Chain::junction, first_owned_chunk, walk_chunk) in the same
// phase order as the kernels, with plain arrays in place of LDS, so the CPU
// test-suite can check the algorithm against the definition.  Not part of the
// library.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../exact_euclidean_distance_amd/csrc/envelope.h"

namespace {

template <int K>
struct LineView {
    using Mask = typename edt::MaskOf<K>::T;
    const double* fb;
    Mask* masks;
    double s2l;
    Mask mask(int c) const { return masks[c]; }
    void set_mask(int c, Mask m) { masks[c] = m; }
    double Y(int pos) const { return fb[pos] + s2l * (double)pos * (double)pos; }
};

template <int K>
int run_line(const double* fb, int L, double s2l, int G, int32_t* owner) {
    using Mask = typename edt::MaskOf<K>::T;
    if ((int64_t)G * K < L) return -1;
    std::vector<Mask> masks(G, 0);
    LineView<K> view{fb, masks.data(), s2l};
    // phase 1: local envelopes
    for (int g = 0; g < G; ++g) {
        masks[g] = edt::build_chunk<Mask, K>(
            g, L, [&](int t) { return fb[g * K + t]; }, [](double v) { return isfinite(v) != 0; },
            [&](double v, int p) { return v + s2l * (double)p * (double)p; });
    }
    // phase 2: merge tree, one level at a time
    for (int h = 1; h < G; h <<= 1) {
        for (int g = 0; g < G; ++g) {
            if ((g & (2 * h - 1)) == h) {
                edt::Chain<LineView<K>, Mask, K> ch(view);
                ch.junction(g - h, g, g + h < G ? g + h : G);
            }
        }
    }
    // phase 3: first owned chunk of every member, prefix maximum
    std::vector<unsigned> slot(G, 0u);
    edt::Chain<LineView<K>, Mask, K> ch(view);
    for (int g = 0; g < G; ++g) {
        Mask mm = masks[g];
        int u = ch.last_in(0, g);
        double Yu = u >= 0 ? view.Y(u) : 0.0;
        while (mm) {
            const int v = g * K + edt::low_bit(mm);
            mm &= mm - 1;
            const double Yv = view.Y(v);
            const int sc = edt::first_owned_chunk(u, Yu, v, Yv, s2l, K, G);
            if (sc < G && slot[sc] < (unsigned)(v + 1)) slot[sc] = (unsigned)(v + 1);
            u = v;
            Yu = Yv;
        }
    }
    for (int g = 1; g < G; ++g) if (slot[g] < slot[g - 1]) slot[g] = slot[g - 1];
    // phase 4: walk
    for (int g = 0; g < G; ++g) {
        const int v = (int)slot[g] - 1;
        for (int t = 0; t < K && g * K + t < L; ++t) owner[g * K + t] = -1;
        if (v < 0) continue;
        edt::walk_chunk(g, K, L, v, s2l, [&](int pos) { return ch.next_member(pos, G); },
                        [&](int pos) { return view.Y(pos); },
                        [&](int t, int o) { owner[g * K + t] = o; });
    }
    return 0;
}

}  // namespace

extern "C" int model_envelope_line(const double* fb, int L, double s2l, int K, int G,
                                   int32_t* owner) {
    if (K == 32) return run_line<32>(fb, L, s2l, G, owner);
    if (K == 64) return run_line<64>(fb, L, s2l, G, owner);
    return -1;
}

// Every line of a [nlines][L] array (one call per line).
extern "C" int model_envelope_lines(const double* fb, int64_t nlines, int L, double s2l, int K,
                                    int G, int32_t* owner) {
    for (int64_t i = 0; i < nlines; ++i) {
        const int rc = model_envelope_line(fb + i * L, L, s2l, K, G, owner + i * L);
        if (rc) return rc;
    }
    return 0;
}
