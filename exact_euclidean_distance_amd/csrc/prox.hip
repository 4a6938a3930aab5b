// prox.hip -- the row pass of "GPU-Based Parallel Euclidean Distance Transform
// Algorithm" (PR-EDT) on gfx950: the sub-block, row-recursive proximate-point
// method of its §3.3-§3.4, an alternative to the separable row pass.
//
// The image is cut into sub-blocks of rows (§3.1); one work-group takes one
// sub-block.  For every row it keeps the row's upper proximate-point set: the
// background pixels, at or above the row, whose Voronoi cells meet the row
// (one candidate per column, the nearest at or above; §3.2's upper candidate
// set), stored as a compact array sorted by column (§3.5: shared memory, one
// thread per point, prefix-sum compaction):
//   first row   Algorithm 1 (§3.3.1): the candidates in column order, each
//               inserted and the points it masks removed -- sequential per
//               sub-block, in parallel over sub-blocks.
//   next rows   Algorithm 3 (§3.3.2): every point tests whether its two
//               neighbours mask it at the new row (the bisector intersections
//               of Figure 5 in the wrong order, equality included); a masked
//               point also tests the points to its right against its left
//               neighbour (Algorithm 2); the marked points are compacted away.
//               The row's background pixels then replace their columns'
//               candidates or join the set, and the tests run again.  The
//               tests repeat until one pass marks nothing, so the set is
//               exactly the row's proximate points however long the chains
//               of masked points are.
//   query       §3.4: each pixel of the row finds its cell with a binary
//               search over the set (the nearer of two consecutive points is
//               monotone in the point index along a proximate-point set).
// The lower sets follow from the bottom row of the sub-block upwards, and each
// pixel keeps the nearer of its upper and lower answers (§3.4).
//
// Differences from the page: sub-blocks are 16 or 64 rows (the page uses 20),
// four or one to each 64-row segment of the axis-0 summary kernels, whose nearest
// background above / below each segment and per-segment background-row bits
// stand in for the full candidate matrices of §3.2 (a sub-block's first row
// takes its candidates from them, the rows after it need only the bits); the
// first row's sweep runs on one thread of the work-group.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

constexpr int kProxThreads = 1024;
// Rows per sub-block: 16 (a quarter of a 64-row summary segment) for rows
// of up to 4096 pixels, a whole segment beyond: Algorithm 1's sweep costs the
// row's width once per sub-block, which for wide rows outweighs the
// parallelism of more sub-blocks (16384^2: 24.5 ms with 16 rows, 11.0 with
// 64; 1024^2: 0.88 against 1.77 ms).
int sub_rows(int W) { return W <= 4096 ? 16 : kSegRows; }
constexpr int kProxMaxW = 16384;
constexpr int kProxPer = kProxMaxW / kProxThreads;   // array entries per thread at most
constexpr uint32_t kNoCand = 0xFFFFFFFFu;

// a point of a set: column in the low 16 bits, row in the high 16
__device__ __forceinline__ int pcol(uint32_t p) { return (int)(p & 0xFFFFu); }
__device__ __forceinline__ int prow(uint32_t p) { return (int)(p >> 16); }

struct RowMetric {
    double s2r, s2c;   // squared spacings of rows and columns
    int row;           // the row being answered
    __device__ double F(uint32_t p) const {   // squared distance from the row to p's row
        const double t = (double)(row - prow(p));
        return s2r * t * t;
    }
    __device__ double Y(uint32_t p) const {
        const double c = (double)pcol(p);
        return F(p) + s2c * c * c;
    }
    __device__ double at(uint32_t p, int q) const {
        const double d = (double)(q - pcol(p));
        return F(p) + s2c * d * d;
    }
    // b is masked by a and c at this row (a < b < c by column)
    __device__ bool masked(uint32_t a, uint32_t b, uint32_t c) const {
        const double Ya = Y(a), Yb = Y(b), Yc = Y(c);
        return (Yb - Ya) * (double)(pcol(c) - pcol(b)) >= (Yc - Yb) * (double)(pcol(b) - pcol(a));
    }
};

// exclusive prefix sum of one int per thread over the work-group; *total gets
// the sum.  Uses wsum[kProxThreads / 64 + 1].
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int k = 0; k < kProxThreads / 64; ++k) {
            const int t = wsum[k];
            wsum[k] = acc;
            acc += t;
        }
        wsum[kProxThreads / 64] = acc;
    }
    __syncthreads();
    const int res = wsum[w] + x - v;
    *total = wsum[kProxThreads / 64];
    __syncthreads();
    return res;
}

// Keep the entries k < n of Q with keep(k): in place, order kept (each thread
// stages its contiguous range in registers first).  Returns the new size.
template <class Keep>
__device__ int compact(uint32_t* Q, int n, int* wsum, Keep keep) {
    const int tid = threadIdx.x;
    const int per = (n + kProxThreads - 1) / kProxThreads;
    const int k0 = tid * per;
    uint32_t stage[kProxPer];
    uint32_t kept = 0;   // bit u: entry k0 + u stays
#pragma unroll
    for (int u = 0; u < kProxPer; ++u) {
        const int k = k0 + u;
        stage[u] = 0;
        if (u < per && k < n && keep(k)) {
            stage[u] = Q[k];
            kept |= 1u << u;
        }
    }
    int total;
    int off = block_exclusive_scan(__builtin_popcount(kept), wsum, &total);
#pragma unroll
    for (int u = 0; u < kProxPer; ++u)
        if ((kept >> u) & 1u) Q[off++] = stage[u];
    __syncthreads();
    return total;
}

// The dense per-column candidates (dense[j] = point, kNoCand: none) as the
// compact set Q, in column order.  Returns the set's size.
__device__ int dense_to_set(const uint32_t* dense, uint32_t* Q, int W, int* wsum) {
    const int tid = threadIdx.x;
    const int cw = (W + kProxThreads - 1) / kProxThreads;
    const int j0 = tid * cw;
    int cnt = 0;
    for (int u = 0; u < cw; ++u) {
        const int j = j0 + u;
        if (j < W && dense[j] != kNoCand) ++cnt;
    }
    int total;
    int off = block_exclusive_scan(cnt, wsum, &total);
    for (int u = 0; u < cw; ++u) {
        const int j = j0 + u;
        if (j < W && dense[j] != kNoCand) Q[off++] = dense[j];
    }
    __syncthreads();
    return total;
}

// Algorithms 2-3's tests at the metric's row: points masked by their
// neighbours are marked (a masked point also tests the points to its right
// against its left neighbour, at most kProp of them), then compacted away;
// repeated until a pass marks nothing.  mark[] has n entries.
constexpr int kProp = 64;

__device__ int remove_masked(uint32_t* Q, int n, uint8_t* mark, int* flag, int* wsum, const RowMetric& M) {
    const int tid = threadIdx.x;
    for (;;) {
        for (int k = tid; k < n; k += kProxThreads) mark[k] = 0;
        if (tid == 0) *flag = 0;
        __syncthreads();
        for (int k = 1 + tid; k < n - 1; k += kProxThreads) {
            const uint32_t a = Q[k - 1];
            if (!M.masked(a, Q[k], Q[k + 1])) continue;
            mark[k] = 1;
            *flag = 1;
            int c = k + 1;   // Algorithm 2: P_c and the points after it against P_a
            for (int s = 0; s < kProp && c + 1 < n; ++s) {
                if (!M.masked(a, Q[c], Q[c + 1])) break;
                mark[c] = 1;
                ++c;
            }
        }
        __syncthreads();
        if (*flag == 0) return n;
        n = compact(Q, n, wsum, [&](int k) { return mark[k] == 0; });
    }
}

// Algorithm 1 (one thread): the insertion sweep over the candidates Q[0..n)
// in column order, the set kept as a stack at the front of Q.
__device__ int sweep(uint32_t* Q, int n, const RowMetric& M) {
    int m = 0;
    for (int k = 0; k < n; ++k) {
        const uint32_t p = Q[k];
        while (m >= 2 && M.masked(Q[m - 2], Q[m - 1], p)) --m;
        Q[m++] = p;
    }
    return m;
}

// §3.4: the owner of pixel q among the set (binary search: the owner is the
// last point that is strictly nearer than the one before it).
__device__ int owner_of(const uint32_t* Q, int n, int q, const RowMetric& M) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (M.at(Q[mid], q) < M.at(Q[mid - 1], q)) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

struct ProxOut {
    int32_t* sqdist;
    float* dist;
    int32_t* indices;
};

// One sub-block (rows [rs, re) of image b): the upper sets from rs down, then
// the lower sets from re - 1 up.  above / below: per (image, segment, column)
// the nearest background row strictly above / below the segment (kNone16:
// none); bits: the segment's background rows per column.  tmpF / tmpI hold
// each pixel's upper answer until the lower pass.
__global__ __launch_bounds__(kProxThreads) void k_prox_rows(
    const uint16_t* __restrict__ above, const uint16_t* __restrict__ below,
    const uint64_t* __restrict__ bits, int H, int W, int nseg, double s2r, double s2c,
    double* __restrict__ tmpF, int32_t* __restrict__ tmpI, ProxOut out, int kSub) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t* Q = reinterpret_cast<uint32_t*>(smem);              // [W]
    uint32_t* dense = Q + kProxMaxW;                              // [W]
    uint8_t* mark = reinterpret_cast<uint8_t*>(dense + kProxMaxW);   // [W]
    int* wsum = reinterpret_cast<int*>(mark + kProxMaxW);         // [kProxThreads / 64 + 1]
    int* flag = wsum + kProxThreads / 64 + 2;
    int* nset = flag + 1;

    const int tid = threadIdx.x;
    const int rs = blockIdx.x * kSub;       // the sub-block's rows [rs, re)
    if (rs >= H) return;                    // (the whole work-group: no barrier reached)
    const int re = min(rs + kSub, H);
    const int s = rs / kSegRows;            // its summary segment, rows [r0, ...)
    const int64_t b = blockIdx.y;
    const int r0 = s * kSegRows;
    const int64_t so = (b * nseg + s) * (int64_t)W;
    const int64_t img = b * (int64_t)H * W;
    RowMetric M{s2r, s2c, rs};
    // the sub-block's background-row bits of the thread's columns
    // j = tid + kProxThreads * u
    uint64_t cb[kProxPer];
#pragma unroll
    for (int u = 0; u < kProxPer; ++u) {
        const int j = tid + kProxThreads * u;
        cb[u] = j < W ? bits[so + j] : 0ull;
    }

    for (int pass = 0; pass < 2; ++pass) {   // 0: upper sets, top-down; 1: lower sets, bottom-up
        const int first = pass == 0 ? rs : re - 1;
        // the first row's candidates: the nearest background of the column at
        // or above it (at or below, bottom-up) -- within the segment from its
        // row bits, else beyond the segment
        const int fb = first - r0;
#pragma unroll
        for (int u = 0; u < kProxPer; ++u) {
            const int j = tid + kProxThreads * u;
            if (j >= W) break;
            int r = -1;
            const uint64_t near = pass == 0 ? (fb == 63 ? cb[u] : cb[u] & ((2ull << fb) - 1ull))
                                            : cb[u] & ~((1ull << fb) - 1ull);
            if (near) {
                r = r0 + (pass == 0 ? 63 - __builtin_clzll(near) : __builtin_ctzll(near));
            } else {   // beyond the segment (nothing for an image of a single segment)
                const uint16_t* beyond = pass == 0 ? above : below;
                const uint16_t c = beyond ? beyond[so + j] : kNone16;
                if (c != kNone16) r = c;
            }
            dense[j] = r < 0 ? kNoCand : ((uint32_t)r << 16) | (uint32_t)j;
        }
        __syncthreads();
        int n = dense_to_set(dense, Q, W, wsum);
        M.row = first;
        if (tid == 0) *nset = sweep(Q, n, M);   // Algorithm 1
        __syncthreads();
        n = *nset;
        for (int step = 0;; ++step) {
            const int row = pass == 0 ? first + step : first - step;
            if (row < rs || row >= re) break;
            M.row = row;
            if (step > 0) {
                // Algorithm 3: masked points at the new row leave; the row's
                // background pixels replace their columns' candidates or join
                n = remove_masked(Q, n, mark, flag, wsum, M);
                for (int j = tid; j < W; j += kProxThreads) dense[j] = kNoCand;
                __syncthreads();
                for (int k = tid; k < n; k += kProxThreads) dense[pcol(Q[k])] = Q[k];
                __syncthreads();
                const int bit = row - r0;
#pragma unroll
                for (int u = 0; u < kProxPer; ++u) {
                    const int j = tid + kProxThreads * u;
                    if (j < W && ((cb[u] >> bit) & 1ull)) dense[j] = ((uint32_t)row << 16) | (uint32_t)j;
                }
                __syncthreads();
                n = dense_to_set(dense, Q, W, wsum);
            }
            n = remove_masked(Q, n, mark, flag, wsum, M);
            // §3.4: every pixel of the row against the set
            const int64_t rb = img + (int64_t)row * W;
            for (int q = tid; q < W; q += kProxThreads) {
                double f;
                int32_t ix;
                if (n > 0) {
                    const uint32_t p = Q[owner_of(Q, n, q, M)];
                    f = M.at(p, q);
                    ix = prow(p) * W + pcol(p);
                } else {
                    f = __builtin_huge_val();
                    ix = 0;
                }
                if (pass == 0) {
                    tmpF[rb + q] = f;
                    tmpI[rb + q] = ix;
                } else {
                    const double fu = tmpF[rb + q];
                    if (fu <= f) {   // the upper answer wins ties
                        f = fu;
                        ix = tmpI[rb + q];
                    }
                    if (!(f < __builtin_huge_val())) {   // no background in the image
                        const double t = (double)(row + 1);
                        f = s2r * t * t + s2c * (double)q * (double)q;
                        ix = -W;
                    }
                    if (out.sqdist) out.sqdist[rb + q] = (int32_t)f;
                    if (out.dist) out.dist[rb + q] = (float)sqrt(f);
                    if (out.indices) out.indices[rb + q] = ix;
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace

size_t prox_lds_bytes() {
    return (size_t)kProxMaxW * 4 * 2 + kProxMaxW + (kProxThreads / 64 + 4) * 4;
}

int prox_max_width() { return kProxMaxW; }

hipError_t launch_prox_rows_2d(const uint16_t* above, const uint16_t* below, const uint64_t* bits,
                               int B, int H, int W, double s2r, double s2c, double* tmpF,
                               int32_t* tmpI, int32_t* sqdist, float* dist, int32_t* indices,
                               hipStream_t s, KernelTimer* tm) {
    static unsigned long long lds_done = 0;
    hipError_t le = large_lds_once((const void*)k_prox_rows, &lds_done);
    if (le != hipSuccess) return le;
    const int nseg = (H + kSegRows - 1) / kSegRows;
    const int kSub = sub_rows(W);
    const int nsub = (H + kSub - 1) / kSub;
    ProxOut out{sqdist, dist, indices};
    if (nseg == 1) above = below = nullptr;   // (the axis-0 scan did not run)
    EDT_LAUNCH(tm, "proximate_rows_2d", s,
               hipLaunchKernelGGL(k_prox_rows, dim3((unsigned)nsub, (unsigned)B), dim3(kProxThreads),
                                  prox_lds_bytes(), s, above, below, bits, H, W, nseg, s2r, s2c, tmpF,
                                  tmpI, out, kSub));
    return hipSuccess;
}

}  // namespace edt
