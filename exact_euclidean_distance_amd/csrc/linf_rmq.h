// linf_rmq.h -- the 1-D chessboard (L-infinity) step with amortised constant
// work per position.  Written as plain templates so that it compiles both for
// gfx950 (inside the chessboard kernels) and as host C++ (the test-only host
// model in tests/host_model).
//
// After the axis-0 pass, each further axis of the chessboard transform (the
// chamfer transform TorchMorph ships beside its EDT, read as SciPy's
// "chessboard" metric) applies, along every line,
//     h(q) = min_j max(g(j), |q - j|),
// g(j) being the distance already accumulated at source j (none: no source).
// Two facts make it cheap:
//   (1) h(q) <= r  exactly when some source j with |q - j| <= r has g(j) <= r,
//       i.e. when the minimum of g over the window [q - r, q + r] is <= r;
//   (2) h changes by at most one between neighbouring positions (each term
//       max(g(j), |q - j|) does).
// So a lane that answers a run of consecutive positions finds h at the first
// one by bisection over r with (1) (between the line's smallest g and the
// value of the best source of the nearby blocks), then at each next position
// tests r = h - 1 and r = h only -- fewer where the last winner's own value
// already decides -- and if neither window holds a small enough source, h
// grows by one and the last winner still attains it (it is at most one
// further away).  Window minima come from a blocked range-minimum structure: per
// block of kRmqBlock positions the prefix and suffix minima, and a sparse
// table over the block minima, so any window is a suffix, whole blocks (two
// overlapping powers of two) and a prefix.  Values are keys g << 16 | j, so a
// minimum also names a source that attains it (ties: the smaller g, then the
// smaller j).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define EDT_LINF_HD __host__ __device__
#else
#define EDT_LINF_HD
#endif

namespace edt {

constexpr int kRmqBlock = 8;                   // positions per block (and per run of a lane)
constexpr uint32_t kRmqNone = 0xFFFFFFFFu;     // no source (above every key: g <= 65534)
constexpr uint16_t kRmqNoG = 0xFFFFu;          // staged g of a position without a source

EDT_LINF_HD inline uint32_t rmq_min(uint32_t a, uint32_t b) { return a < b ? a : b; }
EDT_LINF_HD inline uint32_t rmq_key(uint32_t g, int j) { return (g << 16) | (uint32_t)j; }
EDT_LINF_HD inline int rmq_g(uint32_t key) { return (int)(key >> 16); }
EDT_LINF_HD inline int rmq_j(uint32_t key) { return (int)(key & 0xFFFFu); }
EDT_LINF_HD inline int rmq_log2(int n) {   // floor(log2 n), n >= 1
    return 31 - __builtin_clz((unsigned)n);
}

// Number of table levels for nb blocks: level k holds minima of 2^k blocks.
EDT_LINF_HD inline int rmq_levels(int nb) { return rmq_log2(nb) + 1; }

// Per block, prefix and suffix keys take kRmqKeyStride words and the staged g
// kRmqGStride halfwords: both odd numbers of 32-bit words (9 and 5), so that
// lanes at the same offset of neighbouring blocks use different LDS banks.
constexpr int kRmqKeyStride = kRmqBlock + 1;
constexpr int kRmqGStride = kRmqBlock + 2;
EDT_LINF_HD inline int rmq_ki(int j) { return (j / kRmqBlock) * kRmqKeyStride + j % kRmqBlock; }
EDT_LINF_HD inline int rmq_gi(int j) { return (j / kRmqBlock) * kRmqGStride + j % kRmqBlock; }
// halfwords of one line's staged g
EDT_LINF_HD inline int rmq_g_halves(int L) { return ((L + kRmqBlock - 1) / kRmqBlock) * kRmqGStride; }

// 32-bit words of one line's structure: prefix and suffix keys and the table
// (levels x nb); the staged g is kept apart.
EDT_LINF_HD inline int rmq_words(int L) {
    const int nb = (L + kRmqBlock - 1) / kRmqBlock;
    return 2 * nb * kRmqKeyStride + rmq_levels(nb) * nb;
}

// One line's structure in memory: g[rmq_gi(j)] (kRmqNoG for none),
// pre[rmq_ki(j)] / suf[rmq_ki(j)] the minimum key from the start of j's block
// to j / from j to the end of its block, tab[k * nb + i] the minimum key of
// blocks i .. i + 2^k - 1.
struct RmqLine {
    const uint16_t* g;
    uint32_t* pre;
    uint32_t* suf;
    uint32_t* tab;
    int L, nb;

    EDT_LINF_HD RmqLine(const uint16_t* g_, uint32_t* words, int L_)
        : g(g_), L(L_), nb((L_ + kRmqBlock - 1) / kRmqBlock) {
        pre = words;
        suf = words + nb * kRmqKeyStride;
        tab = words + 2 * nb * kRmqKeyStride;
    }

    EDT_LINF_HD int g_at(int j) const { return (int)g[rmq_gi(j)]; }
    EDT_LINF_HD uint32_t key_at(int j) const {
        const uint16_t v = g[rmq_gi(j)];
        return v == kRmqNoG ? kRmqNone : rmq_key(v, j);
    }

    // Step 1, per block b: prefix / suffix keys and the block minimum (level
    // 0); returns the number of sources in the block.
    EDT_LINF_HD int build_block(int b) {
        const int s = b * kRmqBlock;
        const int e = s + kRmqBlock < L ? s + kRmqBlock : L;
        uint32_t m = kRmqNone;
        int ns = 0;
        for (int j = s; j < e; ++j) {
            const uint32_t k = key_at(j);
            ns += k != kRmqNone;
            m = rmq_min(m, k);
            pre[rmq_ki(j)] = m;
        }
        tab[b] = m;
        m = kRmqNone;
        for (int j = e - 1; j >= s; --j) {
            m = rmq_min(m, key_at(j));
            suf[rmq_ki(j)] = m;
        }
        return ns;
    }

    // Step 2, level k >= 1 entry i (i + 2^k <= nb), after level k - 1 is whole.
    EDT_LINF_HD void build_level(int k, int i) {
        tab[k * nb + i] = rmq_min(tab[(k - 1) * nb + i], tab[(k - 1) * nb + i + (1 << (k - 1))]);
    }

    // Minimum key over positions [a, b] (0 <= a <= b < L).
    EDT_LINF_HD uint32_t query(int a, int b) const {
        const int ba = a / kRmqBlock, bb = b / kRmqBlock;
        if (ba == bb) {
            if (a == ba * kRmqBlock) return pre[rmq_ki(b)];
            if (b == bb * kRmqBlock + kRmqBlock - 1 || b == L - 1) return suf[rmq_ki(a)];
            uint32_t m = kRmqNone;
            for (int j = a; j <= b; ++j) m = rmq_min(m, key_at(j));
            return m;
        }
        uint32_t m = rmq_min(suf[rmq_ki(a)], pre[rmq_ki(b)]);
        const int n = bb - ba - 1;   // whole blocks between
        if (n > 0) {
            const int k = rmq_log2(n);
            m = rmq_min(m, rmq_min(tab[k * nb + ba + 1], tab[k * nb + bb - (1 << k)]));
        }
        return m;
    }

    // Minimum key over the window of radius r around q, clipped to the line.
    EDT_LINF_HD uint32_t window(int q, int r) const {
        return query(q - r > 0 ? q - r : 0, q + r < L - 1 ? q + r : L - 1);
    }

    // Value of source key k at position q: max(g, |q - j|) (k not kRmqNone).
    EDT_LINF_HD static int value_at(uint32_t k, int q) {
        const int d = q > rmq_j(k) ? q - rmq_j(k) : rmq_j(k) - q;
        return rmq_g(k) > d ? rmq_g(k) : d;
    }

    // The smallest key of the whole line (kRmqNone: the line has no source).
    EDT_LINF_HD uint32_t line_min() const {
        const int k = rmq_log2(nb);
        return rmq_min(tab[k * nb], tab[k * nb + nb - (1 << k)]);
    }

    // h and a source attaining it for the n <= kRmqBlock positions q0 ..
    // q0 + n - 1, into hs[t] / js[t] (t < n; the loop over t is unrolled, so
    // the arrays stay in registers); kall is line_min(), not kRmqNone.
    EDT_LINF_HD void answer_run(int q0, int n, uint32_t kall, int (&hs)[kRmqBlock],
                                int (&js)[kRmqBlock]) const {
        // bisection at q0: h(q0) <= r is monotone in r.  Bounds: every
        // source has g >= the line's smallest g; the best source of the
        // block of q0 and of its two neighbours, and the line's best one,
        // each give an upper bound.
        int lo = rmq_g(kall);
        int hi = value_at(kall, q0);
        const int b = q0 / kRmqBlock;
        for (int bb = b > 0 ? b - 1 : 0; bb <= b + 1 && bb < nb; ++bb) {
            const uint32_t kb = tab[bb];
            if (kb != kRmqNone) {
                const int v = value_at(kb, q0);
                if (v < hi) hi = v;
            }
        }
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (rmq_g(window(q0, mid)) <= mid) hi = mid;
            else lo = mid + 1;
        }
        int h = lo;
        int j = rmq_j(window(q0, h));
        hs[0] = h;
        js[0] = j;
#pragma unroll
        for (int t = 1; t < kRmqBlock; ++t) {
            if (t < n) {
                const int q = q0 + t;
                // h(q) is h - 1, h or h + 1; the last winner's value at q,
                // also one of them, is an upper bound
                const int dj = q > j ? q - j : j - q;
                const int gj = g_at(j);
                const int vj = gj > dj ? gj : dj;
                if (vj == h - 1) {   // the bound is the lowest possible value
                    h -= 1;
                } else {
                    uint32_t k = h > 0 ? window(q, h - 1) : kRmqNone;
                    if (h > 0 && rmq_g(k) <= h - 1) {
                        h -= 1;
                        j = rmq_j(k);
                    } else if (vj != h) {   // (vj == h: the winner keeps h)
                        k = window(q, h);
                        if (rmq_g(k) <= h) j = rmq_j(k);
                        else h += 1;   // the last winner: g <= h, at most h + 1 away (vj = h + 1)
                    }
                }
                hs[t] = h;
                js[t] = j;
            }
        }
    }
};

}  // namespace edt
