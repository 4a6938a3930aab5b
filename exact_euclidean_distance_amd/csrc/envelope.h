// envelope.h -- the per-line lower-envelope machinery used by both envelope
// kernels.  Written as plain templates so that it compiles both for gfx950
// (inside the kernels) and as host C++ (the test-only host model in
// tests/host_model, which drives the same functions in the kernels' phase order
// on the CPU).
//
// Geometry ("GPU-Based Parallel Euclidean Distance Transform Algorithm", §3.3,
// Figures 4 and 5; TorchMorph, the separable lower-envelope paragraph).  Along
// one line every candidate j carries the parabola pi_j(q) = s^2 (q - j)^2 + F_j,
// F_j being the squared distance already accumulated over the earlier axes.
// With the lifted height Y_j = F_j + s^2 j^2, two parabolas a < b cross at
// x(a,b) = (Y_b - Y_a) / (2 s^2 (b - a)), where the bisector of their background
// elements meets the line.  pi_b(q) < pi_a(q) exactly when
// Y_b - Y_a < 2 s^2 q (b - a).
//
// The same machinery serves the chessboard step of TorchMorph's chamfer
// transforms (read as the L-infinity metric), f_j(q) = max(g_j, |q - j|): see
// the metrics below.
#pragma once

#include <math.h>
#include <stdint.h>

#include <type_traits>

#if defined(__HIPCC__)
#define EDT_HD __host__ __device__
#else
#define EDT_HD
#endif

namespace edt {

// Bit mask of the surviving positions of one chunk of K positions.
template <int K> struct MaskOf { using T = uint32_t; };
template <> struct MaskOf<64> { using T = uint64_t; };

EDT_HD inline int low_bit(uint32_t m) { return __builtin_ctz(m); }
EDT_HD inline int low_bit(uint64_t m) { return __builtin_ctzll(m); }
EDT_HD inline int high_bit(uint32_t m) { return 31 - __builtin_clz(m); }
EDT_HD inline int high_bit(uint64_t m) { return 63 - __builtin_clzll(m); }

// bits strictly below bit i (0 <= i < width)
template <class M> EDT_HD inline M bits_below(int i) { return (M(1) << i) - M(1); }
// bits strictly above bit i (0 <= i < width)
template <class M> EDT_HD inline M bits_above(int i) { return ~((M(2) << i) - M(1)); }

// Middle member b of a < b < c leaves the envelope iff x(a,b) >= x(b,c)
// (a collinear middle point is dropped).
EDT_HD inline bool dominated(int a, double Ya, int b, double Yb, int c, double Yc) {
    return (Yb - Ya) * (double)(c - b) >= (Yc - Yb) * (double)(b - a);
}

// --------------------------------------------------------------------------
// A line of length L is cut into chunks of K positions.  One lane builds the
// lower envelope of its chunk with the insertion sweep of PR-EDT Algorithm 1
// (insert by increasing coordinate, drop the members the new one dominates);
// the stack is a K-bit mask of surviving positions, so it needs no storage
// beyond one register.  The line's envelope then follows either per chunk
// (chunk_owner_marks, below) or for whole lines in rounds (boundary_dead):
// only a chunk's first and last members have neighbours in other chunks, and
// a member whose neighbours change by a removal becomes a first or last one,
// so each round tests those two members of every chunk against the nearest
// members around them, all dominated ones leave together, and the rounds stop
// when one removes nothing.  A point above the segment between two points of
// the set stays above the lower hull of what remains, so the survivors are the
// envelope of the line -- PR-EDT Algorithm 2's outward re-checks, done at every
// junction at once.
// --------------------------------------------------------------------------

// One round for chunk c of a line of G chunks with member mask m: the bits of
// its first and last members that the dominance test removes, against the
// line as it stands at the start of the round.  View: mask(c), Y(pos), mt (the
// metric), last_nonempty / first_nonempty over a half-open chunk range (-1 if
// none).
template <int K, class View, class Mask>
EDT_HD inline Mask boundary_dead(View& v, int c, int G, Mask m) {
    if (!m) return 0;
    const int base = c * K;
    const int tf = low_bit(m), tl = high_bit(m);
    const int cp = v.last_nonempty(0, c), cn = v.first_nonempty(c + 1, G);
    const int pl = cp < 0 ? -1 : cp * K + high_bit(v.mask(cp));   // last member before the chunk
    const int nf = cn < 0 ? -1 : cn * K + low_bit(v.mask(cn));    // first member after it
    Mask dead = 0;
    {
        const int p = base + tf;
        const Mask above = m & bits_above<Mask>(tf);
        const int pn = above ? base + low_bit(above) : nf;
        if (pl >= 0 && pn >= 0 && v.mt.dominated(pl, v.Y(pl), p, v.Y(p), pn, v.Y(pn))) dead |= Mask(1) << tf;
    }
    if (tl != tf) {
        const int p = base + tl;
        const int pp = base + high_bit(m & bits_below<Mask>(tl));
        if (nf >= 0 && v.mt.dominated(pp, v.Y(pp), p, v.Y(p), nf, v.Y(nf))) dead |= Mask(1) << tl;
    }
    return dead;
}

// Cascade steps of the whole-line rounds.  back_cascade: the trailing members
// of chunk c (member mask m) leave one after another while the last one is
// dominated by its predecessor in the chunk and w, the first member of the
// next non-empty chunk (w >= 0); the chunk's first member always stays.  In a
// step where every chunk does only this, every first member stays, so w is
// present at each removal and the removals are justified one by one (unlike
// boundary_dead, where neighbours may leave together).  front_cascade is the
// mirror image: leading members leave against their successor and w, the
// last member of the previous non-empty chunk; the chunk's last member stays.
// A chunk whose interior members only the far side can dominate then empties
// down to one member in one step instead of one member per round.
template <int K, class View, class Mask>
EDT_HD inline Mask back_cascade(View& v, int c, Mask m, int w) {
    const int base = c * K;
    const auto Yw = v.Y(w);
    int tl = high_bit(m);
    auto Yl = v.Y(base + tl);
    while (m & (m - 1)) {
        const int pp = high_bit(m & bits_below<Mask>(tl));
        const auto Yp = v.Y(base + pp);
        if (!v.mt.dominated_seq(base + pp, Yp, base + tl, Yl, w, Yw)) break;
        m &= ~(Mask(1) << tl);
        tl = pp;
        Yl = Yp;
    }
    return m;
}
template <int K, class View, class Mask>
EDT_HD inline Mask front_cascade(View& v, int c, Mask m, int w) {
    const int base = c * K;
    const auto Yw = v.Y(w);
    int tf = low_bit(m);
    auto Yf = v.Y(base + tf);
    while (m & (m - 1)) {
        const int nn = low_bit(m & bits_above<Mask>(tf));
        const auto Yn = v.Y(base + nn);
        if (!v.mt.dominated_seq(w, Yw, base + tf, Yf, base + nn, Yn)) break;
        m &= ~(Mask(1) << tf);
        tf = nn;
        Yf = Yn;
    }
    return m;
}

// Non-empty chunk search over an occupancy bit set (bit c of word c / 64 set
// when chunk c has a member), for views that keep one.
template <class Words>
EDT_HD inline int occ_last(const Words& occ, int lo, int hi) {  // largest set bit in [lo, hi)
    for (int w = (hi - 1) >> 6; hi > lo && w >= (lo >> 6); --w) {
        uint64_t bits = occ(w);
        const int top = hi - 64 * w;                  // bits below top
        if (top < 64) bits &= (uint64_t(1) << top) - 1;
        const int bot = lo - 64 * w;                  // bits from bot up
        if (bot > 0) bits &= ~((uint64_t(1) << bot) - 1);
        if (bits) return 64 * w + high_bit(bits);
    }
    return -1;
}
template <class Words>
EDT_HD inline int occ_first(const Words& occ, int lo, int hi) {  // smallest set bit in [lo, hi)
    for (int w = lo >> 6; lo < hi && w <= ((hi - 1) >> 6); ++w) {
        uint64_t bits = occ(w);
        const int top = hi - 64 * w;
        if (top < 64) bits &= (uint64_t(1) << top) - 1;
        const int bot = lo - 64 * w;
        if (bot > 0) bits &= ~((uint64_t(1) << bot) - 1);
        if (bits) return 64 * w + low_bit(bits);
    }
    return -1;
}

// Local envelope of one chunk by the insertion sweep, over the candidate
// positions base + t for the set bits t of cand (increasing order); returns the
// member mask.  val_at(t) reads the stored value of position base + t and
// height(v, p) is its height Y_p under the metric mt.
template <class Mask, class Mt, class ValAt, class HeightOf>
EDT_HD inline Mask build_chunk(const Mt& mt, int base, Mask cand, ValAt val_at, HeightOf height) {
    using H = typename Mt::Val;
    Mask m = 0;
    int top = -1, sec = -1;
    H Ytop = H(0), Ysec = H(0);
    while (cand) {
        const int t = low_bit(cand);
        cand &= cand - 1;
        const int p = base + t;
        const H Y = height(val_at(t), p);
        while (sec >= 0 && mt.dominated_seq(sec, Ysec, top, Ytop, p, Y)) {
            m &= ~(Mask(1) << (top - base));
            top = sec; Ytop = Ysec;
            const Mask below = m & bits_below<Mask>(top - base);
            if (below) {
                sec = base + high_bit(below);
                Ysec = height(val_at(sec - base), sec);
            } else {
                sec = -1;
            }
        }
        m |= Mask(1) << t;
        sec = top; Ysec = Ytop;
        top = p; Ytop = Y;
    }
    return m;
}

// The same sweep with the heights of the chunk's K positions at hand (Yr[t] is
// Y of position base + t; unrolled over t, so that Yr can live in registers);
// y_at(p) gives the height of an earlier position that a removal uncovers.
template <int K, class Mask, class Mt, class YAt>
EDT_HD inline Mask build_chunk_unrolled(const Mt& mt, int base, Mask cand,
                                        const typename Mt::Val (&Yr)[K], YAt y_at) {
    using H = typename Mt::Val;
    Mask m = 0;
    int top = -1, sec = -1;
    H Ytop = H(0), Ysec = H(0);
#pragma unroll
    for (int t = 0; t < K; ++t) {
        if (!((cand >> t) & Mask(1))) continue;
        const int p = base + t;
        const H Y = Yr[t];
        while (sec >= 0 && mt.dominated_seq(sec, Ysec, top, Ytop, p, Y)) {
            m &= ~(Mask(1) << (top - base));
            top = sec; Ytop = Ysec;
            const Mask below = m & bits_below<Mask>(top - base);
            if (below) {
                sec = base + high_bit(below);
                Ysec = y_at(sec);
            } else {
                sec = -1;
            }
        }
        m |= Mask(1) << t;
        sec = top; Ysec = Ytop;
        top = p; Ytop = Y;
    }
    return m;
}

// Candidate bound.  If U bounds the final squared distance of every position
// of a line, a candidate with F_j > U owns no position (its parabola stays
// above U everywhere) and can be left out without changing any result.  A
// valid U is the largest, over the chunks of K positions, of
//   min( Fmin(c) + s^2 (K-1)^2,  Fmin(c +- 1) + s^2 (2K-1)^2 )
// where Fmin(c) is the smallest F of chunk c: every position of chunk c lies
// within K-1 of its own chunk's minimiser and within 2K-1 of a neighbour's.
EDT_HD inline double chunk_bound(double fmin_self, double fmin_prev, double fmin_next, double s2l,
                                 int K) {
    const double near = s2l * (double)(K - 1) * (double)(K - 1);
    const double far = s2l * (double)(2 * K - 1) * (double)(2 * K - 1);
    double b = fmin_self + near;
    if (fmin_prev + far < b) b = fmin_prev + far;
    if (fmin_next + far < b) b = fmin_next + far;
    return b;
}

// Smallest float32 >= x (x >= 0): bounds stored as float32 stay upper bounds.
EDT_HD inline float round_up_float(double x) {
    float f = (float)x;
    if ((double)f < x) f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) + 1u);
    return f;
}

// Approximate float32 quotient (a reciprocal estimate on the GPU).
EDT_HD inline float approx_div(float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
    return a * __builtin_amdgcn_rcpf(b);
#else
    return a / b;
#endif
}

// Smallest integer c >= 0 with A < B c (B > 0), or cap if it is cap or more.
// The estimate comes from a float32 quotient; the result is then fixed with
// exact float64 products (exact whenever heights and spacings are integers or
// short dyadic fractions), so no float64 division is needed.
EDT_HD inline int first_index_beating(double A, double B, int cap) {
    if (A < 0.0) return 0;
    const float ratio = approx_div((float)A, (float)B);
    // The float32 quotient is within a relative 1e-6 of A / B, so a quotient of
    // cap + 2 or more puts the answer at cap or beyond.
    if (!(ratio < (float)cap + 2.0f)) return cap;
    int c = (int)floorf(ratio) + 1;
    if (c > cap) c = cap;
    while (c > 0 && A < B * (double)(c - 1)) --c;
    while (c < cap && !(A < B * (double)c)) ++c;
    return c;
}

// --------------------------------------------------------------------------
// Metrics.  The envelope steps need only this of the per-candidate functions
// f_j along a line: for j < k, the positions where f_k is strictly below f_j,
// and those where it is at most f_j, are right half-lines.  Then two
// neighbouring members of an envelope hand over at one position, a candidate
// that neither of two others around it lets win is never needed, a chain in
// which no member is beaten by its two neighbours is the lower envelope, and a
// candidate that loses to a nearer one at a chunk's first position loses on the
// whole chunk.  Both families below have it:
//   L2Metric    f_j(q) = F_j + s^2 (q - j)^2   (the Euclidean step; L2IntMetric
//               the same in exact scaled integers)
//   LinfMetric  f_j(q) = max(g_j, |q - j|)    (the chessboard step; for j < k,
//               f_k - f_j is k - j far to the left and j - k far to the right,
//               and once f_k <= f_j (or <) holds it holds further right)
// A metric gives the candidate value type (Val) and the height its tests
// compare, dist(d) and combine(v, dist(d)) (a candidate of value v at signed
// offset d), the dominance test (dominated: b never strictly below the
// nearer of a and c from its own crossings on -- safe when every dominated
// member leaves at once, as in boundary_dead and the candidate filter;
// dominated_seq: b never strictly below both, ties included -- for the steps
// that remove one member at a time against members still present, which
// keeps every value and leaves no member that dominated would remove), cross (the first position, clipped to [0, cap], where
// the later of two candidates is strictly below the earlier), the chunk bound,
// and the 32-bit form in which chunk minima and bounds are kept.
// --------------------------------------------------------------------------
struct L2Metric {
    using Val = double;
    static constexpr double kInf = __builtin_huge_val();   // no source
    static constexpr double kMaxFinite = __DBL_MAX__;
    double s2;   // squared spacing along the line
    EDT_HD Val height(Val f, int p) const { return f + s2 * (double)p * (double)p; }
    EDT_HD Val dist(int d) const { return s2 * (double)d * (double)d; }
    EDT_HD static Val combine(Val f, Val dd) { return f + dd; }
    EDT_HD static bool dominated(int a, Val Ya, int b, Val Yb, int c, Val Yc) {
        return edt::dominated(a, Ya, b, Yb, c, Yc);
    }
    EDT_HD static bool dominated_seq(int a, Val Ya, int b, Val Yb, int c, Val Yc) {
        return dominated(a, Ya, b, Yb, c, Yc);
    }
    EDT_HD int cross(int a, Val Ya, int b, Val Yb, int cap) const {
        return first_index_beating(Yb - Ya, 2.0 * s2 * (double)(b - a), cap);
    }
    // chunk minima and bounds as float32 bits rounded up; a lower bound of
    // the exact minimum is one float32 step below
    EDT_HD static uint32_t min_bits(Val f) { return __builtin_bit_cast(uint32_t, round_up_float(f)); }
    EDT_HD static Val from_bits(uint32_t b) { return (double)__builtin_bit_cast(float, b); }
    EDT_HD static Val lower_from_bits(uint32_t b) { return from_bits(b) * (1.0 - 0x1p-22); }
    EDT_HD uint32_t bound_bits(Val self, Val prev, Val next, int K) const {
        return __builtin_bit_cast(uint32_t, round_up_float(chunk_bound(self, prev, next, s2, K)));
    }
};

// The same parabolas with exact integer values: every value and height is
// S times the real one (S a power of two with S * s^2 an integer for every
// axis) and stays below 2^29, so values, heights, their differences and kInf
// plus any of them fit int32 (the host checks the bound before choosing this
// metric).  The dominance test and the crossing take float64 products of
// int32 differences and offsets below 2^16: exact, as in L2Metric.
struct L2IntMetric {
    using Val = int;
    static constexpr int kInf = 0x3FFFFFFF;   // no source
    static constexpr int kMaxFinite = kInf - 1;
    int s2;   // S x squared spacing along the line
    EDT_HD Val height(Val f, int p) const { return f + s2 * p * p; }
    EDT_HD Val dist(int d) const { return s2 * d * d; }
    EDT_HD static Val combine(Val f, Val dd) { return f + dd; }
    EDT_HD static bool dominated(int a, Val Ya, int b, Val Yb, int c, Val Yc) {
        return (double)(Yb - Ya) * (double)(c - b) >= (double)(Yc - Yb) * (double)(b - a);
    }
    EDT_HD static bool dominated_seq(int a, Val Ya, int b, Val Yb, int c, Val Yc) {
        return dominated(a, Ya, b, Yb, c, Yc);
    }
    EDT_HD int cross(int a, Val Ya, int b, Val Yb, int cap) const {
        return first_index_beating((double)(Yb - Ya), 2.0 * (double)s2 * (double)(b - a), cap);
    }
    EDT_HD static uint32_t min_bits(Val f) { return (uint32_t)f; }
    EDT_HD static Val from_bits(uint32_t b) { return (int)b; }
    EDT_HD static Val lower_from_bits(uint32_t b) { return (int)b; }
    // chunk_bound in integers, saturated at kInf (no candidate nearby)
    EDT_HD uint32_t bound_bits(Val self, Val prev, Val next, int K) const {
        const int nr = s2 * (K - 1) * (K - 1), fr = s2 * (2 * K - 1) * (2 * K - 1);
        int b = self + nr;
        if (prev + fr < b) b = prev + fr;
        if (next + fr < b) b = next + fr;
        return (uint32_t)(b < kInf ? b : kInf);
    }
};

struct LinfMetric {
    using Val = int;
    static constexpr int kInf = 0x3FFFFFFF;   // no source (sums with positions stay in int32)
    static constexpr int kMaxFinite = kInf - 1;
    EDT_HD static Val height(Val g, int) { return g; }
    EDT_HD static Val dist(int d) { return d < 0 ? -d : d; }
    EDT_HD static Val combine(Val g, Val dd) { return g > dd ? g : dd; }
    // First position q where candidate k is strictly below candidate j (j < k).
    // If g_k >= g_j, f_k can only be below where f_j = q - j > g_k and q is
    // nearer k than j; otherwise already where |q - k| < g_j inside j's flat
    // part, or, past it, where q is nearer k.
    EDT_HD static int first_below(int j, int gj, int k, int gk) {
        const int mid = (j + k) >> 1;
        const int x = gk >= gj ? (j + gk > mid ? j + gk : mid) : (k - gj < mid ? k - gj : mid);
        return x + 1;
    }
    // First position q where candidate k is at most candidate j (j < k): the
    // same cases with ties counted, m rounded up.
    EDT_HD static int first_at_most(int j, int gj, int k, int gk) {
        const int mc = (j + k + 1) >> 1;
        return gk > gj ? (j + gk > mc ? j + gk : mc) : (k - gj < mc ? k - gj : mc);
    }
    EDT_HD static bool dominated(int a, Val ga, int b, Val gb, int c, Val gc) {
        return first_below(a, ga, b, gb) >= first_below(b, gb, c, gc);
    }
    // b is strictly below both a and c nowhere: from first_below(a, b) on it
    // is below a, from first_at_most(b, c) on c is at most b.  Flat bottoms
    // make such ties common (a line at equal g keeps every candidate under
    // the strict test); where removals are justified one at a time, dropping
    // them keeps every value.
    EDT_HD static bool dominated_seq(int a, Val ga, int b, Val gb, int c, Val gc) {
        return first_below(a, ga, b, gb) >= first_at_most(b, gb, c, gc);
    }
    EDT_HD static int cross(int a, Val ga, int b, Val gb, int cap) {
        const int x = first_below(a, ga, b, gb);
        return x < 0 ? 0 : x > cap ? cap : x;
    }
    EDT_HD static uint32_t min_bits(Val g) { return (uint32_t)g; }
    EDT_HD static Val from_bits(uint32_t b) { return (int)b; }
    EDT_HD static Val lower_from_bits(uint32_t b) { return (int)b; }
    // every position of chunk c lies within K - 1 of its own chunk's
    // minimiser and within 2K - 1 of a neighbour's (as chunk_bound)
    EDT_HD static uint32_t bound_bits(Val self, Val prev, Val next, int K) {
        const int a = self > K - 1 ? self : K - 1;
        const int b = prev > 2 * K - 1 ? prev : 2 * K - 1;
        const int c = next > 2 * K - 1 ? next : 2 * K - 1;
        const int m = a < b ? a : b;
        return (uint32_t)(m < c ? m : c);
    }
};

template <bool Narrow> struct SeqBits { using T = uint64_t; };
template <> struct SeqBits<true> { using T = uint32_t; };

// Up to eight 16-bit values held in four 32-bit registers; no array, so
// nothing is placed in scratch memory whatever the index.
struct Packed8 {
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    EDT_HD int get(int i) const {
        const int k = i >> 1;
        const uint32_t w = k == 0 ? w0 : k == 1 ? w1 : k == 2 ? w2 : w3;
        return (int)((w >> ((i & 1) * 16)) & 0xFFFFu);
    }
    EDT_HD void set(int i, int v) {
        const int sh = (i & 1) * 16;
        const uint32_t keep = ~(0xFFFFu << sh), put = ((uint32_t)v & 0xFFFFu) << sh;
        const int k = i >> 1;
        if (k == 0) w0 = (w0 & keep) | put;
        else if (k == 1) w1 = (w1 & keep) | put;
        else if (k == 2) w2 = (w2 & keep) | put;
        else w3 = (w3 & keep) | put;
    }
};

// Owner marks of one chunk (positions [b, e], b = cK) from its local envelope
// M and the members of other chunks that reach into it, with no merging of
// whole lines.
//
// A member m < b is needed for the chunk only if it is strictly nearer at b
// than every member between m and b: for m < x, once x is at least as near as
// m it stays so further right (the metric's half-line property), so not
// winning at b means not being needed on the whole chunk.  Scanning leftwards
// from b, such members are kept while their distance term alone, dist(b - m),
// stays below the best value at b so far (beyond that no member can beat it).
// Symmetrically on the right at e.
// The reaching members (at most CAP per side) and the chunk's members form a
// short sorted sequence whose lower envelope, on [b, e], is the line's.  Its
// members then get their owned intervals; mark(t, owner) is called at chunk
// offset t where an interval starts (t = 0 for the owner of b).  A whole chunk
// is passed over when a lower bound of its F plus the squared distance to its
// nearest position is no better than the best value so far.  Returns false
// without marking if more than CAP members reach in from one side.
// View: Y(pos), f(pos), mt (the metric), mask(c), last_nonempty /
// first_nonempty (as for boundary_dead), fmin_lb(c) (a lower bound of the
// values of chunk c).  Needs 2 CAP + K <= 64.
template <int K, int CAP, class View, class Mask, class Mark>
EDT_HD inline bool chunk_owner_marks(View& v, int c, int G, int L, Mask M, Mark mark) {
    static_assert(2 * CAP + K <= 64, "sequence index space must fit 64 bits");
    static_assert(CAP <= 8, "reach lists hold at most eight members");
    // bit set over the sequence index space below (32 bits when it fits)
    using Seq = typename SeqBits<2 * CAP + K <= 32>::T;
    const int b = c * K;
    const int n = L - b < K ? L - b : K;
    const int e = b + n - 1;
    const auto& mt = v.mt;
    using H = typename std::remove_reference_t<decltype(mt)>::Val;

    // members reaching in from the left (Lp[0] nearest) and from the right
    Packed8 Lp, Rp;
    int nL = 0, nR = 0;
    H best = mt.kInf;
    if (M) {
        const int x = b + low_bit(M);
        best = mt.combine(v.f(x), mt.dist(x - b));
    }
    for (int cc = v.last_nonempty(0, c); cc >= 0; cc = v.last_nonempty(0, cc)) {
        const H ddn = mt.dist(b - (cc * K + K - 1));   // to the chunk's nearest position
        if (!(ddn < best)) break;
        if (!(mt.combine(v.fmin_lb(cc), ddn) < best)) continue;   // no member of it can win
        Mask mk = v.mask(cc);
        bool stop = false;
        do {
            const int t = high_bit(mk);
            mk ^= Mask(1) << t;
            const int m = cc * K + t;
            const H dd = mt.dist(b - m);
            if (!(dd < best)) { stop = true; break; }
            const H p = mt.combine(v.f(m), dd);
            if (p < best) {
                if (nL == CAP) return false;
                Lp.set(nL, m);
                ++nL;
                best = p;
            }
        } while (mk);
        if (stop) break;
    }
    best = mt.kInf;
    if (M) {
        const int x = b + high_bit(M);
        best = mt.combine(v.f(x), mt.dist(e - x));
    }
    for (int cc = v.first_nonempty(c + 1, G); cc >= 0; cc = v.first_nonempty(cc + 1, G)) {
        const H ddn = mt.dist(cc * K - e);
        if (!(ddn < best)) break;
        if (!(mt.combine(v.fmin_lb(cc), ddn) < best)) continue;
        Mask mk = v.mask(cc);
        bool stop = false;
        do {
            const int t = low_bit(mk);
            mk &= mk - 1;
            const int m = cc * K + t;
            const H dd = mt.dist(m - e);
            if (!(dd < best)) { stop = true; break; }
            const H p = mt.combine(v.f(m), dd);
            if (p < best) {
                if (nR == CAP) return false;
                Rp.set(nR, m);
                ++nR;
                best = p;
            }
        } while (mk);
        if (stop) break;
    }

    // Sequence index space: [0, nL) the left members in increasing position,
    // [CAP, CAP + K) the chunk's positions, [CAP + K, CAP + K + nR) the right
    // members in increasing position.
    auto pos_of = [&](int i) -> int {
        if (i < CAP) return Lp.get(nL - 1 - i);
        if (i < CAP + K) return b + (i - CAP);
        return Rp.get(i - CAP - K);
    };

    // lower envelope of the sequence (insertion sweep; the stack top and the
    // member below it are kept with their positions and heights, and the chunk's
    // own members, already convex, are appended without tests once two of them
    // lead the stack)
    Seq alive = 0;
    int top = -1, sec = -1, ptop = 0, psec = 0;
    H Ytop = H(0), Ysec = H(0);
    auto insert = [&](int i, int p) {
        const H Y = v.Y(p);
        while (sec >= 0 && mt.dominated_seq(psec, Ysec, ptop, Ytop, p, Y)) {
            alive &= ~(Seq(1) << top);
            top = sec;
            ptop = psec;
            Ytop = Ysec;
            const Seq below = alive & ((Seq(1) << top) - 1);
            if (below) {
                sec = high_bit(below);
                psec = pos_of(sec);
                Ysec = v.Y(psec);
            } else {
                sec = -1;
            }
        }
        alive |= Seq(1) << i;
        sec = top;
        psec = ptop;
        Ysec = Ytop;
        top = i;
        ptop = p;
        Ytop = Y;
    };
    for (int i = 0; i < nL; ++i) insert(i, Lp.get(nL - 1 - i));
    Mask rest = M;
    while (rest) {
        if (sec >= CAP) {   // top and sec are both members of the chunk
            alive |= (Seq)rest << CAP;
            const int t_last = high_bit(rest);
            const Mask below = rest & ~(Mask(1) << t_last);
            if (below) {
                sec = CAP + high_bit(below);
                psec = b + high_bit(below);
                Ysec = v.Y(psec);
            } else {
                sec = top;
                psec = ptop;
                Ysec = Ytop;
            }
            top = CAP + t_last;
            ptop = b + t_last;
            Ytop = v.Y(ptop);
            break;
        }
        const int t = low_bit(rest);
        rest &= rest - 1;
        insert(CAP + t, b + t);
    }
    for (int i = 0; i < nR; ++i) insert(CAP + K + i, Rp.get(i));

    // owned intervals: member i owns [st, en), st where it is strictly nearer
    // than its predecessor, en where its successor is; clipped to [b, e]
    if (!alive) return true;
    int i = low_bit(alive);
    int pi = pos_of(i);
    H Yi = v.Y(pi);
    int st = b;
    for (;;) {
        const Seq after = i + 1 < (int)(8 * sizeof(Seq)) ? alive & ~((Seq(2) << i) - 1) : Seq(0);
        int en = e + 1;
        int j = -1, pj = 0;
        H Yj = H(0);
        if (after) {
            j = low_bit(after);
            pj = pos_of(j);
            Yj = v.Y(pj);
            en = mt.cross(pi, Yi, pj, Yj, e + 1);
        }
        const int lo = st > b ? st : b;
        if (lo < en) mark(lo - b, pi);
        if (j < 0 || en > e) break;
        i = j;
        pi = pj;
        Yi = Yj;
        st = en;
    }
    return true;
}

}  // namespace edt
