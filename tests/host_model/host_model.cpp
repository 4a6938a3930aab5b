// host_model.cpp -- test-only host build of the envelope machinery in
// exact_euclidean_distance_amd/csrc/envelope.h.
//
// Runs, for one line at a time, the same functions the envelope kernels run
// (the metrics' bounds and tests, build_chunk, chunk_owner_marks,
// boundary_dead) in the same phase order as the kernels, for every metric
// (squared Euclidean in float64 and in scaled integers, chessboard), with plain arrays in place of LDS, so the CPU
// test-suite can check the algorithm against the definition.  Not part of the
// library.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../exact_euclidean_distance_amd/csrc/envelope.h"

namespace {

constexpr int kWitnessScan = 16;   // chunks scanned per side for the filter's witnesses
constexpr int kWitnessScanLinf = 32;   // the same under the chessboard metric
constexpr int kCascadeFrom = 2;    // first whole-line round with cascade steps

template <class Mt> bool has_source(typename Mt::Val v);
template <> bool has_source<edt::L2Metric>(double v) { return isfinite(v); }
template <> bool has_source<edt::LinfMetric>(int v) { return v < edt::LinfMetric::kInf; }
template <> bool has_source<edt::L2IntMetric>(int v) { return v < edt::L2IntMetric::kInf; }

template <int K, class Mt>
struct LineView {
    using Mask = typename edt::MaskOf<K>::T;
    using F = typename Mt::Val;
    const F* fb;
    Mask* masks;
    uint64_t* occ;
    const uint32_t* fminc;   // chunk minima in the metric's 32-bit form
    Mt mt;
    F fmin_lb(int c) const { return Mt::lower_from_bits(fminc[c]); }
    int last_nonempty(int lo, int hi) const {
        return edt::occ_last([&](int w) { return occ[w]; }, lo, hi);
    }
    int first_nonempty(int lo, int hi) const {
        return edt::occ_first([&](int w) { return occ[w]; }, lo, hi);
    }
    void mark_empty(int c) { occ[c >> 6] &= ~(uint64_t(1) << (c & 63)); }
    Mask mask(int c) const { return masks[c]; }
    void set_mask(int c, Mask m) { masks[c] = m; }
    F f(int pos) const { return fb[pos]; }
    F Y(int pos) const { return mt.height(fb[pos], pos); }
};

// G chunk slots of K positions (G * K >= L; slots past the line stay empty).
// CAP: members reaching into a chunk from one side before the line falls back
// to whole-line rounds (0: always whole-line rounds).  fb[p]: the candidate
// value of position p (the metric's kInf, or +inf for L2, where it has none).
template <int K, int CAP, class Mt>
int run_line(const typename Mt::Val* fb, int L, const Mt& mt, int G, int32_t* owner) {
    using Mask = typename edt::MaskOf<K>::T;
    using F = typename Mt::Val;
    if ((int64_t)G * K < L) return -1;
    const int Greal = (L + K - 1) / K;
    std::vector<Mask> masks(G, 0);
    std::vector<uint64_t> occ((G + 63) / 64, 0);
    // phase 0: chunk minima, their first minimisers, and the candidate bound
    // U, in the metric's 32-bit form
    std::vector<uint32_t> fmin(G, Mt::min_bits(Mt::kInf));
    LineView<K, Mt> view{fb, masks.data(), occ.data(), fmin.data(), mt};
    std::vector<int> amin(G, -1);
    for (int g = 0; g < Greal; ++g) {
        F mn = Mt::kInf;
        for (int p = g * K; p < L && p < (g + 1) * K; ++p)
            if (has_source<Mt>(fb[p]) && fb[p] < mn) { mn = fb[p]; amin[g] = p; }
        fmin[g] = Mt::min_bits(mn);
    }
    uint32_t Ub = 0;
    for (int g = 0; g < Greal; ++g) {
        const F prev = g > 0 ? Mt::from_bits(fmin[g - 1]) : F(Mt::kInf);
        const F next = g + 1 < Greal ? Mt::from_bits(fmin[g + 1]) : F(Mt::kInf);
        const uint32_t b = mt.bound_bits(Mt::from_bits(fmin[g]), prev, next, K);
        if (b > Ub) Ub = b;
    }
    const F U = Mt::from_bits(Ub);
    constexpr int scan = CAP > 0 ? 1 : std::is_same<Mt, edt::LinfMetric>::value ? kWitnessScanLinf : kWitnessScan;
    // phase 1: local envelopes of the candidates with a value <= U that are
    // not dominated by a chunk minimiser on either side: the chunk's own where
    // it lies on that side, else the witness (the minimiser of an earlier /
    // later chunk best at the chunk's first / last position, scanning chunk
    // minima outward while the distance term alone is still better, at most
    // kWitnessScan chunks (kWitnessScanLinf for the chessboard); only the
    // neighbouring chunk where the per-chunk route is tried, CAP > 0)
    for (int g = 0; g < G; ++g) {
        const int base = g * K;
        const int n = L - base < K ? L - base : K;
        const int acur = g < Greal ? amin[g] : -1;
        int aprev = -1, anext = -1;
        if (n > 0) {
            F best = Mt::kInf;
            for (int c2 = g - 1; c2 >= 0 && c2 >= g - scan; --c2) {
                if (!(mt.dist(base - (c2 * K + K - 1)) < best)) break;
                const int k = amin[c2];
                if (k < 0) continue;
                const F v = mt.combine(Mt::from_bits(fmin[c2]), mt.dist(base - k));
                if (v < best) { best = v; aprev = k; }
            }
            best = Mt::kInf;
            const int e = base + n - 1;
            for (int c2 = g + 1; c2 < Greal && c2 <= g + scan; ++c2) {
                if (!(mt.dist(c2 * K - e) < best)) break;
                const int k = amin[c2];
                if (k < 0) continue;
                const F v = mt.combine(Mt::from_bits(fmin[c2]), mt.dist(k - e));
                if (v < best) { best = v; anext = k; }
            }
        }
        Mask cand = 0;
        for (int t = 0; t < n; ++t) {
            const int p = base + t;
            if (!has_source<Mt>(fb[p]) || !(fb[p] <= U)) continue;
            const int lo = acur >= 0 && acur < p ? acur : aprev;
            const int hi = acur > p ? acur : anext;
            if (lo >= 0 && hi >= 0 && mt.dominated(lo, view.Y(lo), p, view.Y(p), hi, view.Y(hi)))
                continue;
            cand |= Mask(1) << t;
        }
        masks[g] = edt::build_chunk<Mask>(
            mt, base, cand, [&](int t) { return fb[base + t]; },
            [&](F v, int p) { return mt.height(v, p); });
        // the unrolled sweep over heights held per position must agree
        F Yr[K];
        for (int t = 0; t < K; ++t) Yr[t] = t < n ? view.Y(base + t) : F(0);
        if (edt::build_chunk_unrolled<K>(mt, base, cand, Yr, [&](int p) { return view.Y(p); }) != masks[g])
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
        // (from round kCascadeFrom on, a round that removed something goes on
        // with a back and a front cascade step; first (last) members stay
        // during a back (front) step, so the chunks may go in any order)
        for (int r = 0;; ++r) {
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
            if (r < kCascadeFrom) continue;
            for (int g = 0; g < G; ++g) {
                if (!(masks[g] & (masks[g] - 1))) continue;
                const int cn = view.first_nonempty(g + 1, G);
                if (cn >= 0) masks[g] = edt::back_cascade<K>(view, g, masks[g], cn * K + edt::low_bit(masks[cn]));
            }
            for (int g = G - 1; g >= 0; --g) {
                if (!(masks[g] & (masks[g] - 1))) continue;
                const int cp = view.last_nonempty(0, g);
                if (cp >= 0) masks[g] = edt::front_cascade<K>(view, g, masks[g], cp * K + edt::high_bit(masks[cp]));
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
            const F Yv = view.Y(v);
            int st = 0, en = L;
            if (i > 0) {
                const int u = members[i - 1];
                st = mt.cross(u, view.Y(u), v, Yv, L);
            }
            if (i + 1 < members.size()) {
                const int w = members[i + 1];
                en = mt.cross(v, Yv, w, view.Y(w), L);
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

template <int CAP, class Mt>
int line_k(const typename Mt::Val* fb, int L, const Mt& mt, int K, int G, int32_t* owner) {
    if (K == 8) return run_line<8, CAP>(fb, L, mt, G, owner);
    if (K == 16) return run_line<16, CAP>(fb, L, mt, G, owner);
    if (K == 32) return run_line<32, CAP>(fb, L, mt, G, owner);
    if (K == 64) return run_line<64, (CAP > 0 ? 0 : 0)>(fb, L, mt, G, owner);
    return -1;
}

template <class Mt>
int line_any(const typename Mt::Val* fb, int L, const Mt& mt, int K, int G, int reach, int32_t* owner) {
    if (reach == 8) return line_k<8>(fb, L, mt, K, G, owner);
    if (reach == 1) return line_k<1>(fb, L, mt, K, G, owner);
    if (reach == 0) return line_k<0>(fb, L, mt, K, G, owner);
    return -1;
}

}  // namespace

// Squared Euclidean step: fb[p] = F_p (+inf: no source), s2l the squared
// spacing along the line.
extern "C" int model_envelope_line(const double* fb, int L, double s2l, int K, int G, int reach,
                                   int32_t* owner) {
    return line_any(fb, L, edt::L2Metric{s2l}, K, G, reach, owner);
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

// LinfMetric's crossings for candidates j < k: out[0] = the first position
// where k is strictly below j, out[1] = the first where it is at most j.
extern "C" void model_linf_crossings(int j, int gj, int k, int gk, int32_t* out) {
    out[0] = edt::LinfMetric::first_below(j, gj, k, gk);
    out[1] = edt::LinfMetric::first_at_most(j, gj, k, gk);
}

// The squared Euclidean step in exact integers (L2IntMetric): fb[p] = S F_p
// (negative: no source), s2l = S x the squared spacing along the line; every
// line of a [nlines][L] array.
extern "C" int model_envelope_lines_int(const int32_t* fb, int64_t nlines, int L, int s2l, int K, int G,
                                        int reach, int32_t* owner) {
    std::vector<int> line(L);
    for (int64_t i = 0; i < nlines; ++i) {
        for (int p = 0; p < L; ++p) {
            const int32_t v = fb[i * L + p];
            line[p] = v < 0 ? edt::L2IntMetric::kInf : v;
        }
        const int rc = line_any(line.data(), L, edt::L2IntMetric{s2l}, K, G, reach, owner + i * L);
        if (rc) return rc;
    }
    return 0;
}

// Chessboard step: gb[p] = g_p (negative: no source), every line of a
// [nlines][L] array; value[p]: the owner's value at p through the metric, as
// the kernels' output step forms it (-1 where the line has no source).
extern "C" int model_linf_envelope_lines(const int32_t* gb, int64_t nlines, int L, int K, int G,
                                         int reach, int32_t* owner, int32_t* value) {
    std::vector<int> line(L);
    const edt::LinfMetric mt{};
    for (int64_t i = 0; i < nlines; ++i) {
        for (int p = 0; p < L; ++p) {
            const int32_t v = gb[i * L + p];
            line[p] = v < 0 ? edt::LinfMetric::kInf : v;
        }
        int32_t* own = owner + i * L;
        const int rc = line_any(line.data(), L, mt, K, G, reach, own);
        if (rc) return rc;
        for (int q = 0; q < L; ++q)
            value[i * L + q] = own[q] < 0 ? -1 : mt.combine(line[own[q]], mt.dist(q - own[q]));
    }
    return 0;
}
