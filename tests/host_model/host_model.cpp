// host_model.cpp -- test-only host build of the envelope machinery in
// exact_euclidean_distance_amd/csrc/envelope.h.
//
// Runs, for one line at a time, the same functions the envelope kernels run
// (chunk_bound, build_chunk, chunk_owner_marks, boundary_dead,
// first_index_beating) in the same
// phase order as the kernels, with plain arrays in place of LDS, so the CPU
// test-suite can check the algorithm against the definition.  Not part of the
// library.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../exact_euclidean_distance_amd/csrc/envelope.h"

namespace {

template <int K>
struct LineView {
    using Mask = typename edt::MaskOf<K>::T;
    const double* fb;
    Mask* masks;
    uint64_t* occ;
    const float* fminc;   // chunk minima of F as float32, rounded up
    double s2l;
    double fmin_lb(int c) const { return (double)fminc[c] * (1.0 - 0x1p-22); }
    int last_nonempty(int lo, int hi) const {
        return edt::occ_last([&](int w) { return occ[w]; }, lo, hi);
    }
    int first_nonempty(int lo, int hi) const {
        return edt::occ_first([&](int w) { return occ[w]; }, lo, hi);
    }
    void mark_empty(int c) { occ[c >> 6] &= ~(uint64_t(1) << (c & 63)); }
    Mask mask(int c) const { return masks[c]; }
    void set_mask(int c, Mask m) { masks[c] = m; }
    double f(int pos) const { return fb[pos]; }
    double Y(int pos) const { return fb[pos] + s2l * (double)pos * (double)pos; }
};

// G chunk slots of K positions (G * K >= L; slots past the line stay empty).
// CAP: members reaching into a chunk from one side before the line falls back
// to whole-line rounds (0: always whole-line rounds).
template <int K, int CAP>
int run_line(const double* fb, int L, double s2l, int G, int32_t* owner) {
    using Mask = typename edt::MaskOf<K>::T;
    if ((int64_t)G * K < L) return -1;
    const int Greal = (L + K - 1) / K;
    std::vector<Mask> masks(G, 0);
    std::vector<uint64_t> occ((G + 63) / 64, 0);
    // phase 0: chunk minima of F, their first minimisers, and the candidate
    // bound U (float32, rounded up)
    std::vector<float> fmin(G, INFINITY);
    LineView<K> view{fb, masks.data(), occ.data(), fmin.data(), s2l};
    std::vector<int> amin(G, -1);
    for (int g = 0; g < Greal; ++g) {
        double mn = INFINITY;
        for (int p = g * K; p < L && p < (g + 1) * K; ++p)
            if (isfinite(fb[p]) && fb[p] < mn) { mn = fb[p]; amin[g] = p; }
        fmin[g] = edt::round_up_float(mn);
    }
    float U = 0.0f;
    for (int g = 0; g < Greal; ++g) {
        const double prev = g > 0 ? (double)fmin[g - 1] : INFINITY;
        const double next = g + 1 < Greal ? (double)fmin[g + 1] : INFINITY;
        const float b = edt::round_up_float(edt::chunk_bound(fmin[g], prev, next, s2l, K));
        if (b > U) U = b;
    }
    // phase 1: local envelopes of the candidates with F <= U that are not
    // dominated by the nearest chunk minimisers on either side
    for (int g = 0; g < G; ++g) {
        const int base = g * K;
        const int n = L - base < K ? L - base : K;
        const int acur = g < Greal ? amin[g] : -1;
        const int aprev = g > 0 && g - 1 < Greal ? amin[g - 1] : -1;
        const int anext = g + 1 < Greal ? amin[g + 1] : -1;
        Mask cand = 0;
        for (int t = 0; t < n; ++t) {
            const int p = base + t;
            if (!isfinite(fb[p]) || !(fb[p] <= (double)U)) continue;
            const int lo = acur >= 0 && acur < p ? acur : aprev;
            const int hi = acur > p ? acur : anext;
            if (lo >= 0 && hi >= 0 && edt::dominated(lo, view.Y(lo), p, view.Y(p), hi, view.Y(hi)))
                continue;
            cand |= Mask(1) << t;
        }
        masks[g] = edt::build_chunk<Mask>(
            base, cand, [&](int t) { return fb[base + t]; },
            [&](double v, int p) { return v + s2l * (double)p * (double)p; });
        // the unrolled sweep over heights held per position must agree
        double Yr[K];
        for (int t = 0; t < K; ++t) Yr[t] = t < n ? view.Y(base + t) : 0.0;
        if (edt::build_chunk_unrolled<K>(base, cand, Yr, [&](int p) { return view.Y(p); }) != masks[g])
            return -2;
        if (masks[g]) occ[g >> 6] |= uint64_t(1) << (g & 63);
    }
    std::vector<int> mark(L, 0);
    // phase 2: owners of each chunk from its own envelope and the members of
    // other chunks that reach into it
    bool ok = CAP > 0;
    if constexpr (CAP > 0) {
        for (int g = 0; g < Greal && ok; ++g) {
            const int base = g * K;
            ok = edt::chunk_owner_marks<K, CAP>(view, g, Greal, L, masks[g],
                                                [&](int t, int o) { mark[base + t] = o + 1; });
        }
    }
    if (!ok) {
        std::fill(mark.begin(), mark.end(), 0);
        // phase 2': whole-line rounds; every chunk is tested against the line
        // as it stands at the start of the round, the removals land together
        for (;;) {
            std::vector<Mask> dead(G, 0);
            bool any = false;
            for (int g = 0; g < G; ++g) {
                dead[g] = edt::boundary_dead<K>(view, g, G, masks[g]);
                any = any || dead[g] != 0;
            }
            if (!any) break;
            for (int g = 0; g < G; ++g) {
                if (!dead[g]) continue;
                masks[g] &= ~dead[g];
                if (!masks[g]) view.mark_empty(g);
            }
        }
        // phase 3': every member v owns [st, en): st where it beats its
        // predecessor, en where its successor takes over; a non-empty interval
        // marks v + 1 at st (one writer per mark)
        std::vector<int> members;
        for (int g = 0; g < G; ++g)
            for (Mask mm = masks[g]; mm; mm &= mm - 1) members.push_back(g * K + edt::low_bit(mm));
        for (size_t i = 0; i < members.size(); ++i) {
            const int v = members[i];
            const double Yv = view.Y(v);
            int st = 0, en = L;
            if (i > 0) {
                const int u = members[i - 1];
                st = edt::first_index_beating(Yv - view.Y(u), 2.0 * s2l * (double)(v - u), L);
            }
            if (i + 1 < members.size()) {
                const int w = members[i + 1];
                en = edt::first_index_beating(view.Y(w) - Yv, 2.0 * s2l * (double)(w - v), L);
            }
            if (st < en) mark[st] = v + 1;
        }
    }
    // phase 4: the owner of q is the latest mark at or before q
    int o = 0;
    for (int q = 0; q < L; ++q) {
        if (mark[q] > o) o = mark[q];
        owner[q] = o - 1;
    }
    return 0;
}

}  // namespace

template <int CAP>
int line_k(const double* fb, int L, double s2l, int K, int G, int32_t* owner) {
    if (K == 8) return run_line<8, CAP>(fb, L, s2l, G, owner);
    if (K == 16) return run_line<16, CAP>(fb, L, s2l, G, owner);
    if (K == 32) return run_line<32, CAP>(fb, L, s2l, G, owner);
    if (K == 64) return run_line<64, (CAP > 0 ? 0 : 0)>(fb, L, s2l, G, owner);
    return -1;
}

extern "C" int model_envelope_line(const double* fb, int L, double s2l, int K, int G, int reach,
                                   int32_t* owner) {
    if (reach == 8) return line_k<8>(fb, L, s2l, K, G, owner);
    if (reach == 1) return line_k<1>(fb, L, s2l, K, G, owner);
    if (reach == 0) return line_k<0>(fb, L, s2l, K, G, owner);
    return -1;
}

// Every line of a [nlines][L] array (one call per line).
extern "C" int model_envelope_lines(const double* fb, int64_t nlines, int L, double s2l, int K,
                                    int G, int reach, int32_t* owner) {
    for (int64_t i = 0; i < nlines; ++i) {
        const int rc = model_envelope_line(fb + i * L, L, s2l, K, G, reach, owner + i * L);
        if (rc) return rc;
    }
    return 0;
}
