// kernels.hip -- gfx950 kernels of the separable exact EDT.
//
// The method ("TorchMorph: CUDA-accelerated Morphological Transforms", the
// separable lower-envelope EDT paragraph; "GPU-Based Parallel Euclidean
// Distance Transform Algorithm", §2.1 independent scanning):
//   pass 0  along axis 0: nearest background on every line (PR-EDT §3.2 builds
//           the same information as upper/lower candidate matrices);
//   pass k  along each further axis: the lower envelope of the parabolas
//           s_k^2 (q - j)^2 + F(j) of a line, then every position q takes the
//           envelope member below it (PR-EDT §3.4).
// Intermediates between passes are the nearest background's coordinates, not
// distances: uint16 after pass 0, packed uint32 (axis0 << 16 | axis1) after the
// middle pass of a volume.  Distances are recomputed exactly from them.
//
// Exactness.  Parabola values are formed in float64 from integer coordinates
// and the squared spacings; with unit spacing every value is an integer below
// 2^53, so all comparisons below are exact.  Parabolas a < b meet at
// x(a,b) = (Y_b - Y_a) / (2 s^2 (b - a)), Y_j = F(j) + s^2 j^2: the bisector of
// the two background elements crosses the line there (PR-EDT §3.3, Figure 4).
// The middle of three members a < b < c is dropped when x(a,b) >= x(b,c)
// (Figure 5), tested without division.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "envelope.h"
#include "kernels.h"

namespace edt {

// --------------------------------------------------------------------------
// helpers
// --------------------------------------------------------------------------

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// Raise the dynamic-LDS ceiling of a kernel to the gfx950 LDS size.  A failure
// is not fatal here: a launch that really needs more LDS fails on its own.
static void allow_large_lds(const void* fn) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        (void)hipGetLastError();
}

hipError_t KernelTimer::begin(const char* kname, hipStream_t s) {
    if (n >= capacity || n >= kMax) { ok = false; return hipSuccess; }
    hipError_t e = hipEventCreate(&ev[2 * n]);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&ev[2 * n + 1]);
    if (e != hipSuccess) { (void)hipEventDestroy(ev[2 * n]); return e; }
    created = n + 1;
    e = hipEventRecord(ev[2 * n], s);
    name[n] = kname;
    return e;
}

hipError_t KernelTimer::end(hipStream_t s) {
    if (n >= capacity || n >= kMax) return hipSuccess;
    hipError_t e = hipEventRecord(ev[2 * n + 1], s);
    ++n;
    return e;
}

// Launch bracket: optional timing events, then the launch error check.
#define EDT_LAUNCH(tm, kname, stream, ...)                                   \
    do {                                                                     \
        if (tm) { hipError_t e_ = (tm)->begin(kname, stream); if (e_ != hipSuccess) return e_; } \
        __VA_ARGS__;                                                         \
        hipError_t e2_ = hipGetLastError();                                  \
        if (e2_ != hipSuccess) return e2_;                                   \
        if (tm) { hipError_t e_ = (tm)->end(stream); if (e_ != hipSuccess) return e_; } \
    } while (0)

// --------------------------------------------------------------------------
// Pass 0: nearest background along axis 0, in three kernels over segments of
// kSegRows rows (so that long, few lines still fill the machine):
//   summary  first/last background row of every (segment, column);
//   scan     per column, nearest background strictly above / below each segment;
//   resolve  per (segment, column), the nearest background of every row from a
//            64-bit background bitmask of the segment plus the two carries.
// Columns are the contiguous innermost index m (one lane per VEC columns), so
// every load and store is coalesced.
// --------------------------------------------------------------------------

template <int VEC>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint8_t (&out)[VEC]) {
    if constexpr (VEC == 1) {
        out[0] = *p;
    } else if constexpr (VEC == 4) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int v = 0; v < 4; ++v) out[v] = (uint8_t)(w >> (8 * v));
    } else {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int v = 0; v < 16; ++v) out[v] = (uint8_t)(ws[v >> 2] >> (8 * (v & 3)));
    }
}

template <int VEC>
__device__ __forceinline__ void store_u16(uint16_t* p, const uint16_t (&v)[VEC]) {
    if constexpr (VEC == 1) {
        p[0] = v[0];
    } else if constexpr (VEC == 4) {
        uint2 w;
        w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
        w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
        *reinterpret_cast<uint2*>(p) = w;
    } else {
        uint4 a, b;
        a.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
        a.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
        a.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
        a.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
        b.x = (uint32_t)v[8] | ((uint32_t)v[9] << 16);
        b.y = (uint32_t)v[10] | ((uint32_t)v[11] << 16);
        b.z = (uint32_t)v[12] | ((uint32_t)v[13] << 16);
        b.w = (uint32_t)v[14] | ((uint32_t)v[15] << 16);
        reinterpret_cast<uint4*>(p)[0] = a;
        reinterpret_cast<uint4*>(p)[1] = b;
    }
}

template <int VEC>
__device__ __forceinline__ void load_u16(const uint16_t* p, uint16_t (&v)[VEC]) {
    if constexpr (VEC == 1) {
        v[0] = p[0];
    } else if constexpr (VEC == 4) {
        uint2 w = *reinterpret_cast<const uint2*>(p);
        v[0] = (uint16_t)w.x; v[1] = (uint16_t)(w.x >> 16);
        v[2] = (uint16_t)w.y; v[3] = (uint16_t)(w.y >> 16);
    } else {
        uint4 a = reinterpret_cast<const uint4*>(p)[0];
        uint4 b = reinterpret_cast<const uint4*>(p)[1];
        uint32_t ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (uint16_t)(ws[i >> 1] >> (16 * (i & 1)));
    }
}

template <int VEC>
__global__ __launch_bounds__(256) void k_axis0_summary(const uint8_t* __restrict__ mask, int n0,
                                                        int64_t M, int nseg,
                                                        uint16_t* __restrict__ first,
                                                        uint16_t* __restrict__ last) {
    const int64_t col = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    if (col >= M) return;
    const int i0 = s * kSegRows;
    const int i1 = min(n0, i0 + kSegRows);
    const uint8_t* src = mask + (int64_t)b * n0 * M + col;
    uint16_t f[VEC], l[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { f[v] = kNone16; l[v] = kNone16; }
#pragma unroll 4
    for (int i = i0; i < i1; ++i) {
        uint8_t x[VEC];
        load_bytes<VEC>(src + (int64_t)i * M, x);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const bool bg = (x[v] == 0);
            f[v] = (bg && f[v] == kNone16) ? (uint16_t)i : f[v];
            l[v] = bg ? (uint16_t)i : l[v];
        }
    }
    const int64_t o = ((int64_t)b * nseg + s) * M + col;
    store_u16<VEC>(first + o, f);
    store_u16<VEC>(last + o, l);
}

// After this kernel last[b][s][m] holds the nearest background row above
// segment s (kNone16 if none) and first[b][s][m] the nearest one below it.
constexpr int kScanQ = 16;   // segment groups per column (threads along y)

__global__ __launch_bounds__(64 * kScanQ) void k_axis0_scan(uint16_t* __restrict__ first,
                                                            uint16_t* __restrict__ last,
                                                            int nseg, int64_t M) {
    __shared__ int agg_last[kScanQ][64];
    __shared__ int agg_first[kScanQ][64];
    const int x = threadIdx.x, q = threadIdx.y;
    const int64_t col = (int64_t)blockIdx.x * 64 + x;
    const int b = blockIdx.y;
    const bool ok = col < M;
    const int per = (nseg + kScanQ - 1) / kScanQ;
    const int s0 = min(nseg, q * per), s1 = min(nseg, s0 + per);
    const int64_t base = (int64_t)b * nseg * M + col;

    int al = -1, af = INT_MAX;
    if (ok) {
        for (int s = s0; s < s1; ++s) {
            const uint16_t l = last[base + (int64_t)s * M];
            const uint16_t f = first[base + (int64_t)s * M];
            if (l != kNone16) al = l;
            if (f != kNone16 && af == INT_MAX) af = f;
        }
    }
    agg_last[q][x] = al;
    agg_first[q][x] = af;
    __syncthreads();
    if (!ok) return;
    int up = -1, dn = INT_MAX;
    for (int qq = 0; qq < q; ++qq) if (agg_last[qq][x] >= 0) up = agg_last[qq][x];
    for (int qq = kScanQ - 1; qq > q; --qq) if (agg_first[qq][x] != INT_MAX) dn = agg_first[qq][x];
    for (int s = s0; s < s1; ++s) {
        const int64_t o = base + (int64_t)s * M;
        const uint16_t l = last[o];
        last[o] = up < 0 ? kNone16 : (uint16_t)up;
        if (l != kNone16) up = l;
    }
    for (int s = s1 - 1; s >= s0; --s) {
        const int64_t o = base + (int64_t)s * M;
        const uint16_t f = first[o];
        first[o] = dn == INT_MAX ? kNone16 : (uint16_t)dn;
        if (f != kNone16) dn = f;
    }
}

template <int VEC>
__global__ __launch_bounds__(256) void k_axis0_resolve(const uint8_t* __restrict__ mask, int n0,
                                                        int64_t M, int nseg,
                                                        const uint16_t* __restrict__ up_carry,
                                                        const uint16_t* __restrict__ dn_carry,
                                                        uint16_t* __restrict__ c0) {
    const int64_t col = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    if (col >= M) return;
    const int i0 = s * kSegRows;
    const int i1 = min(n0, i0 + kSegRows);
    const uint8_t* src = mask + (int64_t)b * n0 * M + col;
    uint64_t bm[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) bm[v] = 0;
#pragma unroll 4
    for (int i = i0; i < i1; ++i) {
        uint8_t x[VEC];
        load_bytes<VEC>(src + (int64_t)i * M, x);
#pragma unroll
        for (int v = 0; v < VEC; ++v) bm[v] |= (uint64_t)(x[v] == 0) << (i - i0);
    }
    const int64_t so = ((int64_t)b * nseg + s) * M + col;
    uint16_t upc[VEC], dnc[VEC];
    load_u16<VEC>(up_carry + so, upc);
    load_u16<VEC>(dn_carry + so, dnc);
    uint16_t* dst = c0 + (int64_t)b * n0 * M + col;
    for (int i = i0; i < i1; ++i) {
        const int r = i - i0;
        uint16_t out[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const uint64_t below = bm[v] >> r;                        // rows >= i
            const uint64_t above = bm[v] & ((uint64_t(2) << r) - 1);  // rows <= i
            const int dn = below ? i + __builtin_ctzll(below)
                                 : (dnc[v] == kNone16 ? -1 : (int)dnc[v]);
            const int up = above ? i0 + 63 - __builtin_clzll(above)
                                 : (upc[v] == kNone16 ? -1 : (int)upc[v]);
            // the nearer one; the smaller coordinate on a tie
            const int g = (up >= 0 && (dn < 0 || i - up <= dn - i)) ? up : dn;
            out[v] = g < 0 ? kNone16 : (uint16_t)g;
        }
        store_u16<VEC>(dst + (int64_t)i * M, out);
    }
}

hipError_t launch_axis0(const uint8_t* mask, int B, int n0, int64_t M, uint16_t* first,
                        uint16_t* last, uint16_t* c0, hipStream_t s, KernelTimer* tm) {
    const int nseg = (n0 + kSegRows - 1) / kSegRows;
    int vec = 1;
    if (M % 16 == 0 && ((uintptr_t)mask & 15) == 0) vec = 16;
    else if (M % 4 == 0 && ((uintptr_t)mask & 3) == 0) vec = 4;
    const int64_t lanes = M / vec + (M % vec ? 1 : 0);
    dim3 grid((unsigned)((lanes + 255) / 256), (unsigned)nseg, (unsigned)B);
    dim3 block(256);
    if (vec == 16) {
        EDT_LAUNCH(tm, "axis0_summary", s, hipLaunchKernelGGL(k_axis0_summary<16>, grid, block, 0, s, mask, n0, M, nseg, first, last));
    } else if (vec == 4) {
        EDT_LAUNCH(tm, "axis0_summary", s, hipLaunchKernelGGL(k_axis0_summary<4>, grid, block, 0, s, mask, n0, M, nseg, first, last));
    } else {
        EDT_LAUNCH(tm, "axis0_summary", s, hipLaunchKernelGGL(k_axis0_summary<1>, grid, block, 0, s, mask, n0, M, nseg, first, last));
    }
    dim3 sgrid((unsigned)((M + 63) / 64), (unsigned)B);
    dim3 sblock(64, kScanQ);
    EDT_LAUNCH(tm, "axis0_scan", s, hipLaunchKernelGGL(k_axis0_scan, sgrid, sblock, 0, s, first, last, nseg, M));
    if (vec == 16) {
        EDT_LAUNCH(tm, "axis0_resolve", s, hipLaunchKernelGGL(k_axis0_resolve<16>, grid, block, 0, s, mask, n0, M, nseg, last, first, c0));
    } else if (vec == 4) {
        EDT_LAUNCH(tm, "axis0_resolve", s, hipLaunchKernelGGL(k_axis0_resolve<4>, grid, block, 0, s, mask, n0, M, nseg, last, first, c0));
    } else {
        EDT_LAUNCH(tm, "axis0_resolve", s, hipLaunchKernelGGL(k_axis0_resolve<1>, grid, block, 0, s, mask, n0, M, nseg, last, first, c0));
    }
    return hipSuccess;
}

// --------------------------------------------------------------------------
// Row layout: lines contiguous in memory (the last axis).  A work-group holds
// LPW lines; lane g of a line owns chunk g.  LDS per chunk: its K values plus a
// one-word pad (so chunk reads at stride K are bank-conflict free), its K owner
// slots, and a few words of chunk metadata.  The final owner of every position
// is written to LDS and the epilogue then streams the outputs coalesced.
// --------------------------------------------------------------------------

struct Geo2D {          // rows of an H x W image; value = axis-0 coordinate
    double s2a, s2l;    // squared spacing of axis 0 and along the row
    int W;
    using Val = uint16_t;
    __device__ static bool valid(uint16_t v) { return v != kNone16; }
    __device__ double baseF(int64_t line, uint16_t v) const {
        const double t = (double)((int)line - (int)v);
        return s2a * t * t;
    }
    __device__ int32_t index(int64_t line, uint16_t v, int pos) const { return (int32_t)v * W + pos; }
    __device__ double virtF(int64_t line, int q) const {
        const double t = (double)(line + 1);
        return s2a * t * t + s2l * (double)q * (double)q;
    }
    __device__ int32_t virt_index() const { return -W; }
};

struct Geo3D {          // rows along W of B x D x H x W volumes; value = packed (axis0, axis1)
    double s2a, s2b, s2l;
    int D, H, W;
    using Val = uint32_t;
    __device__ static bool valid(uint32_t v) { return v != kNone32; }
    __device__ double baseF(int64_t line, uint32_t v) const {
        const int h = (int)(line % H);
        const int d = (int)((line / H) % D);
        const double t0 = (double)(d - (int)(v >> 16));
        const double t1 = (double)(h - (int)(v & 0xFFFFu));
        return s2a * t0 * t0 + s2b * t1 * t1;
    }
    __device__ int32_t index(int64_t line, uint32_t v, int pos) const {
        return ((int32_t)(v >> 16) * H + (int32_t)(v & 0xFFFFu)) * W + pos;
    }
    __device__ double virtF(int64_t line, int q) const {
        const int h = (int)(line % H);
        const int d = (int)((line / H) % D);
        const double t0 = (double)(d + 1);
        return s2a * t0 * t0 + s2b * (double)h * (double)h + s2l * (double)q * (double)q;
    }
    __device__ int32_t virt_index() const { return -(H * W); }
};

template <class Val, int K>
struct RowLayout {
    static constexpr int kPadV = 4 / (int)sizeof(Val);
    static constexpr int kVStride = K + kPadV;   // Val units per chunk
    static constexpr int kOStride = K + 2;       // uint16 units per chunk
    using Mask = typename MaskOf<K>::T;
    static size_t bytes(int nchunks) {
        return align16((size_t)nchunks * kVStride * sizeof(Val)) +
               align16((size_t)nchunks * kOStride * sizeof(uint16_t)) +
               align16((size_t)nchunks * sizeof(Mask)) + 3 * align16((size_t)nchunks * 4);
    }
};

template <class Geo, int K>
struct RowView {
    using Val = typename Geo::Val;
    using Lay = RowLayout<Val, K>;
    using Mask = typename Lay::Mask;
    const Val* sval;   // this line's first chunk
    Mask* scm;         // this line's first chunk mask
    const Geo& geo;
    int64_t line;
    __device__ Mask mask(int c) const { return scm[c]; }
    __device__ void set_mask(int c, Mask m) { scm[c] = m; }
    __device__ Val val(int pos) const { return sval[(pos / K) * Lay::kVStride + pos % K]; }
    __device__ double Y(int pos) const {
        return geo.baseF(line, val(pos)) + geo.s2l * (double)pos * (double)pos;
    }
};

template <class Geo, int K>
__global__ __launch_bounds__(1024) void k_envelope_rows(const typename Geo::Val* __restrict__ in,
                                                        int L, int64_t nlines, int G, int LPW,
                                                        Geo geo, int32_t* __restrict__ sqdist,
                                                        float* __restrict__ dist,
                                                        int32_t* __restrict__ indices) {
    using Val = typename Geo::Val;
    using Lay = RowLayout<Val, K>;
    using Mask = typename Lay::Mask;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nchunks = G * LPW;
    Val* sval = reinterpret_cast<Val*>(smem);
    size_t off = align16((size_t)nchunks * Lay::kVStride * sizeof(Val));
    uint16_t* sown = reinterpret_cast<uint16_t*>(smem + off);
    off += align16((size_t)nchunks * Lay::kOStride * sizeof(uint16_t));
    Mask* scm = reinterpret_cast<Mask*>(smem + off);
    off += align16((size_t)nchunks * sizeof(Mask));
    int* sA = reinterpret_cast<int*>(smem + off);       // last member, then prefix max
    off += align16((size_t)nchunks * 4);
    int* sB = reinterpret_cast<int*>(smem + off);       // first member, then suffix min
    off += align16((size_t)nchunks * 4);
    unsigned* sslot = reinterpret_cast<unsigned*>(smem + off);

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int g = tid % G;
    const int r = tid / G;
    const int c = tid;                      // chunk index within the work-group
    const int64_t line0 = (int64_t)blockIdx.x * LPW;
    const int nl = (int)min((int64_t)LPW, nlines - line0);
    const bool active = r < nl;
    const int64_t line = line0 + r;

    // ---- load the work-group's lines (contiguous in memory) into LDS ----
    {
        const Val* src = in + line0 * (int64_t)L;
        const int64_t nelem = (int64_t)nl * L;
        int rr = tid / L, p = tid % L;
        for (int64_t e = tid; e < nelem; e += nthr) {
            sval[(rr * G + p / K) * Lay::kVStride + p % K] = src[e];
            p += nthr;
            while (p >= L) { p -= L; ++rr; }
        }
    }
    __syncthreads();

    RowView<Geo, K> view{sval + (size_t)r * G * Lay::kVStride, scm + (size_t)r * G, geo, line};

    // ---- local envelope of every chunk ----
    Mask m = 0;
    if (active) {
        const Val* cv = sval + (size_t)c * Lay::kVStride;
        m = build_chunk<Mask, K>(
            g, L, [&](int t) { return cv[t]; }, [](Val v) { return Geo::valid(v); },
            [&](Val v, int p) { return geo.baseF(line, v) + geo.s2l * (double)p * (double)p; });
    }
    scm[c] = m;

    // ---- merge tree ----
    for (int h = 1; h < G; h <<= 1) {
        __syncthreads();
        if (active && (g & (2 * h - 1)) == h) {
            Chain<RowView<Geo, K>, Mask, K> ch(view);
            ch.junction(g - h, g, min(g + h, G));
        }
    }
    __syncthreads();

    // ---- per line: last member up to each chunk, first member from each chunk ----
    {
        const Mask mm = active ? scm[c] : Mask(0);
        sA[c] = mm ? g * K + high_bit(mm) : -1;
        sB[c] = mm ? g * K + low_bit(mm) : INT_MAX;
    }
    for (int d = 1; d < G; d <<= 1) {
        __syncthreads();
        const int a = (g >= d) ? sA[c - d] : -1;
        const int bb = (g + d < G) ? sB[c + d] : INT_MAX;
        __syncthreads();
        sA[c] = max(sA[c], a);
        sB[c] = min(sB[c], bb);
    }
    sslot[c] = 0u;
    __syncthreads();

    // ---- every member marks the first chunk whose first position it owns ----
    if (active) {
        Mask mm = scm[c];
        int u = (g > 0) ? sA[c - 1] : -1;
        double Yu = u >= 0 ? view.Y(u) : 0.0;
        while (mm) {
            const int vpos = g * K + low_bit(mm);
            mm &= mm - 1;
            const double Yv = view.Y(vpos);
            const int sc = first_owned_chunk(u, Yu, vpos, Yv, geo.s2l, K, G);
            if (sc < G) atomicMax(&sslot[r * G + sc], (unsigned)(vpos + 1));
            u = vpos;
            Yu = Yv;
        }
    }
    for (int d = 1; d < G; d <<= 1) {
        __syncthreads();
        const unsigned a = (g >= d) ? sslot[c - d] : 0u;
        __syncthreads();
        sslot[c] = max(sslot[c], a);
    }
    __syncthreads();

    // ---- walk the chunk's positions, recording each position's owner ----
    if (active) {
        uint16_t* own = sown + (size_t)c * Lay::kOStride;
        int v = (int)sslot[c] - 1;
        if (v < 0) {
            for (int t = 0; t < K; ++t) own[t] = kNone16;
        } else {
            auto next_of = [&](int pos) -> int {
                const int cc = pos / K;
                const Mask nm = scm[r * G + cc] & bits_above<Mask>(pos % K);
                if (nm) return cc * K + low_bit(nm);
                const int nf = (cc + 1 < G) ? sB[r * G + cc + 1] : INT_MAX;
                return nf == INT_MAX ? -1 : nf;
            };
            walk_chunk(g, K, L, v, geo.s2l, next_of, [&](int pos) { return view.Y(pos); },
                       [&](int t, int o) { own[t] = (uint16_t)o; });
        }
    }
    __syncthreads();

    // ---- epilogue: distances and indices, streamed coalesced ----
    {
        const int64_t nelem = (int64_t)nl * L;
        int rr = tid / L, p = tid % L;
        for (int64_t e = tid; e < nelem; e += nthr) {
            const int64_t ln = line0 + rr;
            const int o = sown[(rr * G + p / K) * Lay::kOStride + p % K];
            double F;
            int32_t ix;
            if (o == kNone16) {
                F = geo.virtF(ln, p);
                ix = geo.virt_index();
            } else {
                const Val v = sval[(rr * G + o / K) * Lay::kVStride + o % K];
                const double t = (double)(p - o);
                F = geo.baseF(ln, v) + geo.s2l * t * t;
                ix = geo.index(ln, v, o);
            }
            const int64_t go = line0 * (int64_t)L + e;
            if (sqdist) sqdist[go] = (int32_t)F;
            if (dist) dist[go] = sqrtf((float)F);
            if (indices) indices[go] = ix;
            p += nthr;
            while (p >= L) { p -= L; ++rr; }
        }
    }
}

struct RowPlan {
    int K, G, LPW;
    size_t lds;
};

static RowPlan plan_rows(int L, int value_bytes) {
    RowPlan p{};
    p.K = (L <= 8192) ? 32 : 64;
    int chunks = (L + p.K - 1) / p.K;
    p.G = 1;
    while (p.G < chunks) p.G <<= 1;
    p.LPW = p.G >= 256 ? 1 : 256 / p.G;
    const int nch = p.G * p.LPW;
    if (value_bytes == 2)
        p.lds = p.K == 32 ? RowLayout<uint16_t, 32>::bytes(nch) : RowLayout<uint16_t, 64>::bytes(nch);
    else
        p.lds = p.K == 32 ? RowLayout<uint32_t, 32>::bytes(nch) : RowLayout<uint32_t, 64>::bytes(nch);
    return p;
}

size_t rows_lds_bytes(int L, int value_bytes) {
    RowPlan p = plan_rows(L, value_bytes);
    if (p.G > 1024) return 0;
    return p.lds;
}

template <class Geo, int K>
static hipError_t launch_rows_t(const typename Geo::Val* in, int L, int64_t nlines, const RowPlan& p,
                                const Geo& geo, int32_t* sqdist, float* dist, int32_t* indices,
                                hipStream_t s, KernelTimer* tm, const char* kname) {
    static bool attr_done = false;
    if (!attr_done) {
        allow_large_lds((const void*)k_envelope_rows<Geo, K>);
        attr_done = true;
    }
    const int64_t nblocks = (nlines + p.LPW - 1) / p.LPW;
    EDT_LAUNCH(tm, kname, s,
               hipLaunchKernelGGL((k_envelope_rows<Geo, K>), dim3((unsigned)nblocks),
                                  dim3(p.G * p.LPW), p.lds, s, in, L, nlines, p.G, p.LPW, geo,
                                  sqdist, dist, indices));
    return hipSuccess;
}

hipError_t launch_rows_2d(const uint16_t* c0, int H, int W, double s2_0, double s2_1,
                          int32_t* sqdist, float* dist, int32_t* indices, hipStream_t s,
                          KernelTimer* tm) {
    const RowPlan p = plan_rows(W, 2);
    Geo2D geo{s2_0, s2_1, W};
    if (p.K == 32)
        return launch_rows_t<Geo2D, 32>(c0, W, H, p, geo, sqdist, dist, indices, s, tm, "envelope_rows_2d");
    return launch_rows_t<Geo2D, 64>(c0, W, H, p, geo, sqdist, dist, indices, s, tm, "envelope_rows_2d");
}

hipError_t launch_rows_3d(const uint32_t* c01, int B, int D, int H, int W, double s2_0,
                          double s2_1, double s2_2, int32_t* sqdist, float* dist,
                          int32_t* indices, hipStream_t s, KernelTimer* tm) {
    const RowPlan p = plan_rows(W, 4);
    Geo3D geo{s2_0, s2_1, s2_2, D, H, W};
    const int64_t nlines = (int64_t)B * D * H;
    if (p.K == 32)
        return launch_rows_t<Geo3D, 32>(c01, W, nlines, p, geo, sqdist, dist, indices, s, tm, "envelope_rows_3d");
    return launch_rows_t<Geo3D, 64>(c01, W, nlines, p, geo, sqdist, dist, indices, s, tm, "envelope_rows_3d");
}

// --------------------------------------------------------------------------
// Column layout: the middle axis of a volume, lines strided by W.  A
// work-group takes 64 neighbouring lines (lane x = line, so every LDS row and
// every global access is 64 consecutive elements) and G = ceil(H/K) waves
// (wave g = chunk g of all 64 lines).  Outputs go straight from the walk to
// memory: at each step the 64 lanes of a wave write 64 consecutive words.
// --------------------------------------------------------------------------

template <int K>
struct ColView {
    using Mask = typename MaskOf<K>::T;
    const uint16_t* sval;  // [H][64]
    Mask* scm;             // [G][64]
    int x, d;
    double s2a, s2l;
    __device__ Mask mask(int c) const { return scm[c * 64 + x]; }
    __device__ void set_mask(int c, Mask m) { scm[c * 64 + x] = m; }
    __device__ double Y(int pos) const {
        const double t = (double)(d - (int)sval[pos * 64 + x]);
        return s2a * t * t + s2l * (double)pos * (double)pos;
    }
};

size_t cols_lds_bytes(int H) {
    const int K = H <= 512 ? 32 : 64;
    const int G = (H + K - 1) / K;
    const size_t mb = K == 32 ? 4 : 8;
    return align16((size_t)H * 64 * 2) + align16((size_t)G * 64 * mb) + align16((size_t)G * 64 * 4);
}

template <int K>
__global__ __launch_bounds__(1024) void k_envelope_cols(const uint16_t* __restrict__ c0,
                                                        uint32_t* __restrict__ out, int D, int H,
                                                        int W, int G, double s2a, double s2l) {
    using Mask = typename MaskOf<K>::T;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* sval = reinterpret_cast<uint16_t*>(smem);
    size_t off = align16((size_t)H * 64 * 2);
    Mask* scm = reinterpret_cast<Mask*>(smem + off);
    off += align16((size_t)G * 64 * sizeof(Mask));
    unsigned* sslot = reinterpret_cast<unsigned*>(smem + off);

    const int x = threadIdx.x;
    const int g = threadIdx.y;
    const int tiles = (W + 63) / 64;
    const int64_t plane = blockIdx.x / tiles;
    const int w0 = (blockIdx.x % tiles) * 64;
    const bool active = (w0 + x) < W;
    const int d = (int)(plane % D);

    const uint16_t* src = c0 + plane * (int64_t)H * W + w0 + x;
    for (int h = g; h < H; h += G) sval[h * 64 + x] = active ? src[(int64_t)h * W] : kNone16;
    __syncthreads();

    ColView<K> view{sval, scm, x, d, s2a, s2l};
    Mask m = 0;
    if (active) {
        m = build_chunk<Mask, K>(
            g, H, [&](int t) { return sval[(g * K + t) * 64 + x]; },
            [](uint16_t v) { return v != kNone16; },
            [&](uint16_t v, int p) {
                const double t = (double)(d - (int)v);
                return s2a * t * t + s2l * (double)p * (double)p;
            });
    }
    scm[g * 64 + x] = m;

    for (int h = 1; h < G; h <<= 1) {
        __syncthreads();
        if (active && (g & (2 * h - 1)) == h) {
            Chain<ColView<K>, Mask, K> ch(view);
            ch.junction(g - h, g, min(g + h, G));
        }
    }
    sslot[g * 64 + x] = 0u;
    __syncthreads();

    Chain<ColView<K>, Mask, K> ch(view);
    if (active) {
        Mask mm = scm[g * 64 + x];
        int u = ch.last_in(0, g);
        double Yu = u >= 0 ? view.Y(u) : 0.0;
        while (mm) {
            const int vpos = g * K + low_bit(mm);
            mm &= mm - 1;
            const double Yv = view.Y(vpos);
            const int sc = first_owned_chunk(u, Yu, vpos, Yv, s2l, K, G);
            if (sc < G) atomicMax(&sslot[sc * 64 + x], (unsigned)(vpos + 1));
            u = vpos;
            Yu = Yv;
        }
    }
    __syncthreads();

    if (active) {
        unsigned best = 0;
        for (int cc = 0; cc <= g; ++cc) best = max(best, sslot[cc * 64 + x]);
        int v = (int)best - 1;
        uint32_t* dst = out + plane * (int64_t)H * W + w0 + x;
        if (v < 0) {
            for (int t = 0; t < K; ++t) {
                const int q = g * K + t;
                if (q >= H) break;
                dst[(int64_t)q * W] = kNone32;
            }
        } else {
            walk_chunk(g, K, H, v, s2l, [&](int pos) { return ch.next_member(pos, G); },
                       [&](int pos) { return view.Y(pos); },
                       [&](int t, int o) {
                           dst[(int64_t)(g * K + t) * W] = ((uint32_t)sval[o * 64 + x] << 16) | (uint32_t)o;
                       });
        }
    }
}

hipError_t launch_cols_3d(const uint16_t* c0, int B, int D, int H, int W, double s2_0,
                          double s2_1, uint32_t* c01, hipStream_t s, KernelTimer* tm) {
    const int K = H <= 512 ? 32 : 64;
    const int G = (H + K - 1) / K;
    const size_t lds = cols_lds_bytes(H);
    const int tiles = (W + 63) / 64;
    const int64_t nblocks = (int64_t)B * D * tiles;
    if (K == 32) {
        static bool attr = false;
        if (!attr) {
            allow_large_lds((const void*)k_envelope_cols<32>);
            attr = true;
        }
        EDT_LAUNCH(tm, "envelope_cols_3d", s,
                   hipLaunchKernelGGL(k_envelope_cols<32>, dim3((unsigned)nblocks), dim3(64, G), lds, s,
                                      c0, c01, D, H, W, G, s2_0, s2_1));
    } else {
        static bool attr = false;
        if (!attr) {
            allow_large_lds((const void*)k_envelope_cols<64>);
            attr = true;
        }
        EDT_LAUNCH(tm, "envelope_cols_3d", s,
                   hipLaunchKernelGGL(k_envelope_cols<64>, dim3((unsigned)nblocks), dim3(64, G), lds, s,
                                      c0, c01, D, H, W, G, s2_0, s2_1));
    }
    return hipSuccess;
}

}  // namespace edt
