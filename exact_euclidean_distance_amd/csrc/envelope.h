// envelope.h -- the per-line lower-envelope machinery used by both envelope
// kernels.  Written as plain templates so that it compiles both for gfx950
// (inside the kernels) and as host C++ (the test-only host model in
// tests/host_model, which drives the same functions in the kernels' phase order
// on the CPU).
#pragma once

#include <math.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define EDT_HD __host__ __device__
#else
#define EDT_HD
#endif

namespace edt {

template <int K> struct MaskOf;
template <> struct MaskOf<32> { using T = uint32_t; };
template <> struct MaskOf<64> { using T = uint64_t; };

EDT_HD inline int low_bit(uint32_t m) { return __builtin_ctz(m); }
EDT_HD inline int low_bit(uint64_t m) { return __builtin_ctzll(m); }
EDT_HD inline int high_bit(uint32_t m) { return 31 - __builtin_clz(m); }
EDT_HD inline int high_bit(uint64_t m) { return 63 - __builtin_clzll(m); }

// bits strictly below bit i
template <class M> EDT_HD inline M bits_below(int i) { return (M(1) << i) - M(1); }
// bits strictly above bit i (i <= width-1)
template <class M> EDT_HD inline M bits_above(int i) { return ~((M(2) << i) - M(1)); }

// Middle member b of a < b < c leaves the envelope iff x(a,b) >= x(b,c).
EDT_HD inline bool dominated(int a, double Ya, int b, double Yb, int c, double Yc) {
    return (Yb - Ya) * (double)(c - b) >= (Yc - Yb) * (double)(b - a);
}

// --------------------------------------------------------------------------
// Envelope machinery shared by both pass layouts.
//
// A line of length L is cut into G chunks of K positions.  One lane builds the
// lower envelope of its chunk with the insertion sweep of PR-EDT Algorithm 1
// (insert by increasing coordinate, drop the members the new one dominates);
// the stack is a K-bit mask of surviving positions, so it needs no storage
// beyond one register.  Neighbouring chunk envelopes are then merged in a
// binary tree: at each junction one lane removes, from the inner ends of the
// two convex chains, members dominated by their current neighbours until both
// junction triples are convex -- the outward re-checks of PR-EDT Algorithm 2.
// Every merged chain stays locally convex, hence is the envelope of its union.
// --------------------------------------------------------------------------

// View of one line: chunk masks and parabola heights Y.  Implemented by the
// two layouts below.
template <class View, class Mask, int K>
struct Chain {
    View& v;
    EDT_HD Chain(View& vv) : v(vv) {}

    EDT_HD int last_in(int c0, int c1) {  // largest member in chunks [c0, c1)
        for (int c = c1 - 1; c >= c0; --c) {
            const Mask m = v.mask(c);
            if (m) return c * K + high_bit(m);
        }
        return -1;
    }
    EDT_HD int first_in(int c0, int c1) {  // smallest member in chunks [c0, c1)
        for (int c = c0; c < c1; ++c) {
            const Mask m = v.mask(c);
            if (m) return c * K + low_bit(m);
        }
        return -1;
    }
    EDT_HD int prev_member(int pos, int c_lo) {  // largest member < pos, chunks >= c_lo
        const int c = pos / K;
        const Mask m = v.mask(c) & bits_below<Mask>(pos % K);
        if (m) return c * K + high_bit(m);
        return last_in(c_lo, c);
    }
    EDT_HD int next_member(int pos, int c_hi) {  // smallest member > pos, chunks < c_hi
        const int c = pos / K;
        const Mask m = v.mask(c) & bits_above<Mask>(pos % K);
        if (m) return c * K + low_bit(m);
        return first_in(c + 1, c_hi);
    }
    EDT_HD void remove(int pos) {
        const int c = pos / K;
        v.set_mask(c, v.mask(c) & ~(Mask(1) << (pos % K)));
    }

    // Merge the envelopes of chunks [cl, cm) and [cm, cr).
    EDT_HD void junction(int cl, int cm, int cr) {
        int a = last_in(cl, cm);
        if (a < 0) return;
        int b = first_in(cm, cr);
        if (b < 0) return;
        double Ya = v.Y(a), Yb = v.Y(b);
        int a2 = prev_member(a, cl);
        double Ya2 = a2 >= 0 ? v.Y(a2) : 0.0;
        int b2 = next_member(b, cr);
        double Yb2 = b2 >= 0 ? v.Y(b2) : 0.0;
        for (;;) {
            if (a2 >= 0 && dominated(a2, Ya2, a, Ya, b, Yb)) {
                remove(a);
                a = a2; Ya = Ya2;
                a2 = prev_member(a, cl);
                if (a2 >= 0) Ya2 = v.Y(a2);
            } else if (b2 >= 0 && dominated(a, Ya, b, Yb, b2, Yb2)) {
                remove(b);
                b = b2; Yb = Yb2;
                b2 = next_member(b, cr);
                if (b2 >= 0) Yb2 = v.Y(b2);
            } else {
                break;
            }
        }
    }
};

// Local envelope of chunk g by the insertion sweep; returns the member mask.
// Y(pos) re-reads a member's height after a removal exposes it.
template <class Mask, int K, class ValAt, class IsValid, class HeightOf>
EDT_HD inline Mask build_chunk(int g, int L, ValAt val_at, IsValid valid,
                                            HeightOf height) {
    Mask m = 0;
    int top = -1, sec = -1;
    double Ytop = 0.0, Ysec = 0.0;
    const int base = g * K;
    for (int t = 0; t < K; ++t) {
        const int p = base + t;
        if (p >= L) break;
        const auto v = val_at(t);
        if (!valid(v)) continue;
        const double Y = height(v, p);
        while (sec >= 0 && dominated(sec, Ysec, top, Ytop, p, Y)) {
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

// First position at which member v is strictly nearer than its predecessor u
// on the line: floor(x(u,v)) + 1.  float64 division of integers below 2^53 with
// a denominator below 2^17 cannot round across an integer, so this is exact for
// unit spacing.
EDT_HD inline double start_after(int u, double Yu, int v, double Yv, double s2l) {
    return floor((Yv - Yu) / (2.0 * s2l * (double)(v - u))) + 1.0;
}


// Index of the first chunk (of K positions, G chunks in the line) whose first
// position member v owns, given its predecessor u on the merged envelope
// (u < 0: none, v owns from the start); G if v owns no chunk start.
EDT_HD inline int first_owned_chunk(int u, double Yu, int v, double Yv, double s2l, int K, int G) {
    if (u < 0) return 0;
    const double st = start_after(u, Yu, v, Yv, s2l);
    if (st <= 0.0) return 0;
    if (st > (double)G * K) return G;
    return (int)ceil(st / (double)K);
}

// Owner of every position of chunk g, starting from the owner v of its first
// position: the next member w takes over at the first q where it is strictly
// nearer (ties stay with the smaller coordinate), the query of the line's 1-D
// Voronoi diagram (PR-EDT §3.4).  emit(t, owner) for t in [0, K), q < L.
template <class NextOf, class HeightOf, class Emit>
EDT_HD inline void walk_chunk(int g, int K, int L, int v, double s2l, NextOf next_of,
                              HeightOf Y, Emit emit) {
    double Yv = Y(v);
    int w = next_of(v);
    double Yw = w >= 0 ? Y(w) : 0.0;
    const double two_s2 = 2.0 * s2l;
    for (int t = 0; t < K; ++t) {
        const int q = g * K + t;
        if (q >= L) break;
        while (w >= 0 && (Yw - Yv) < two_s2 * (double)q * (double)(w - v)) {
            v = w;
            Yv = Yw;
            w = next_of(v);
            if (w >= 0) Yw = Y(w);
        }
        emit(t, v);
    }
}

}  // namespace edt
