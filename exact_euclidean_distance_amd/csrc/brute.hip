// brute.hip -- the transforms by their definition, on the GPU: every element
// against every background element of its image (TorchMorph's brute-force
// transform, the exactness oracle beside its EDT; the Voronoi page's per-cell
// search).  O(elements x background elements): a checker, not a fast path.
//
//   k_bg_count / k_bg_scan / k_bg_write
//                per image, the flat indices of its background elements in
//                ascending order and their count (counts per block of 4096
//                elements, an exclusive scan of them per image, then each
//                block writes its elements from its offset);
//   k_brute      squared Euclidean distance with any spacing, in float64;
//   k_brute_int  integer metrics: squared Euclidean at unit spacing, city
//                block (L1) and chessboard (L-infinity).  Each thread takes
//                kEpt elements; the background list is read in tiles of 256
//                (coordinates and flat index, decoded once per tile) through
//                LDS; coordinates are below 65536, so |p_k - b_k| is one
//                v_sad_u16.  The list is in ascending index order, so a strict
//                compare keeps the smallest index among equally near elements.
// Images without background take the virtual element at (-1, 0, ..., 0).
// The smallest index among equally near background elements is returned.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

constexpr int kBruteTile = 256;
constexpr int kEpt = 4;   // elements per thread of k_brute_int

struct ImageShape {
    int ndim;          // 1..3
    int n[3];          // extents, axis 0 first
    double s2[3];      // squared spacings
    int64_t per;       // elements per image
};

__device__ inline void coords_of(const ImageShape& sh, int f, int c[3]) {
    c[0] = c[1] = c[2] = 0;
    if (sh.ndim == 1) {
        c[0] = f;
    } else if (sh.ndim == 2) {
        c[0] = f / sh.n[1];
        c[1] = f - c[0] * sh.n[1];
    } else {
        const int plane = sh.n[1] * sh.n[2];
        c[0] = f / plane;
        const int r = f - c[0] * plane;
        c[1] = r / sh.n[2];
        c[2] = r - c[1] * sh.n[2];
    }
}

// Distance of metric M between two points of ND axes (coordinates < 65536,
// so the absolute difference of an axis is one v_sad_u16).
template <int M, int ND>
__device__ inline uint32_t metric_of(const uint32_t p[3], const uint4& t) {
    const uint32_t tc[3] = {t.x, t.y, t.z};
    uint32_t d = 0;
#pragma unroll
    for (int a = 0; a < ND; ++a) {
        if (M == kBruteTaxicab) {
            d = __builtin_amdgcn_sad_u16(p[a], tc[a], d);
        } else if (M == kBruteChessboard) {
            d = max(d, __builtin_amdgcn_sad_u16(p[a], tc[a], 0u));
        } else {
            const uint32_t g = __builtin_amdgcn_sad_u16(p[a], tc[a], 0u);
            d += (uint32_t)__umul24(g, g);
        }
    }
    return d;
}

// The virtual element's distance for an image without background.
template <int M>
__device__ inline uint32_t virtual_metric(const uint32_t p[3], int ndim) {
    uint32_t d = M == kBruteSquared ? (p[0] + 1) * (p[0] + 1) : p[0] + 1;
    for (int a = 1; a < ndim; ++a) {
        if (M == kBruteTaxicab) d += p[a];
        else if (M == kBruteChessboard) d = max(d, p[a]);
        else d += p[a] * p[a];
    }
    return d;
}

}  // namespace

constexpr int kListPer = 16;                  // elements per thread of the list kernels
constexpr int kListBlock = 256 * kListPer;    // elements per block

// Background bits of the kListPer elements thread t of block blk covers.
__device__ inline uint32_t bg_bits(const uint8_t* __restrict__ m, int64_t per, int64_t blk) {
    const int64_t e0 = blk * kListBlock + (int64_t)threadIdx.x * kListPer;
    uint32_t z = 0;
#pragma unroll
    for (int j = 0; j < kListPer; ++j)
        if (e0 + j < per && m[e0 + j] == 0) z |= 1u << j;
    return z;
}

// Exclusive prefix of v over a block of 256 threads; *total gets the sum.
__device__ inline int block_scan256(int v, int* total) {
    __shared__ int wsum[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        before += k < w ? wsum[k] : 0;
        all += wsum[k];
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// grid: (blocks of kListBlock elements, images)
__global__ __launch_bounds__(256) void k_bg_count(const uint8_t* __restrict__ mask, int64_t per,
                                                  int32_t* __restrict__ block_off) {
    const int64_t b = blockIdx.y, nblk = gridDim.x;
    int total;
    (void)block_scan256(__popc(bg_bits(mask + b * per, per, blockIdx.x)), &total);
    if (threadIdx.x == 0) block_off[b * nblk + blockIdx.x] = total;
}

// grid: images; block_off[b][*] becomes its exclusive prefix, counts[b] the total
__global__ __launch_bounds__(256) void k_bg_scan(int32_t* __restrict__ block_off, int64_t nblk,
                                                 int32_t* __restrict__ counts) {
    int32_t* o = block_off + (int64_t)blockIdx.x * nblk;
    int run = 0;
    for (int64_t c = 0; c < nblk; c += 256) {
        const int64_t i = c + threadIdx.x;
        const int v = i < nblk ? o[i] : 0;
        int total;
        const int ex = block_scan256(v, &total);
        if (i < nblk) o[i] = run + ex;
        run += total;
    }
    if (threadIdx.x == 0) counts[blockIdx.x] = run;
}

// grid: (blocks of kListBlock elements, images)
__global__ __launch_bounds__(256) void k_bg_write(const uint8_t* __restrict__ mask, int64_t per,
                                                  const int32_t* __restrict__ block_off,
                                                  int32_t* __restrict__ list) {
    const int64_t b = blockIdx.y, nblk = gridDim.x;
    uint32_t z = bg_bits(mask + b * per, per, blockIdx.x);
    int total;
    int at = block_off[b * nblk + blockIdx.x] + block_scan256(__popc(z), &total);
    const int32_t e0 = (int32_t)((int64_t)blockIdx.x * kListBlock + (int64_t)threadIdx.x * kListPer);
    int32_t* out = list + b * per;
    while (z) {
        out[at++] = e0 + __builtin_ctz(z);
        z &= z - 1;
    }
}

// grid: (element blocks, images); every thread of a block takes part in the
// tile loads, so none leaves before the loop ends
__global__ __launch_bounds__(256) void k_brute(const int32_t* __restrict__ list,
                                               const int32_t* __restrict__ counts, ImageShape sh,
                                               int32_t* __restrict__ sqdist, float* __restrict__ dist,
                                               int32_t* __restrict__ indices) {
    __shared__ int32_t tile[kBruteTile];          // flat index
    __shared__ int32_t tc[3][kBruteTile];         // its coordinates, decoded once per tile
    const int64_t b = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool mine = i < sh.per;
    int p[3];
    coords_of(sh, mine ? (int)i : 0, p);
    const int nbg = counts[b];
    const int32_t* lb = list + b * sh.per;
    double best = __builtin_huge_val();
    int32_t bidx = 0x7FFFFFFF;
    for (int t0 = 0; t0 < nbg; t0 += kBruteTile) {
        const int m = min(kBruteTile, nbg - t0);
        __syncthreads();
        if ((int)threadIdx.x < m) {
            const int32_t f = lb[t0 + threadIdx.x];
            int c[3];
            coords_of(sh, f, c);
            tile[threadIdx.x] = f;
            tc[0][threadIdx.x] = c[0];
            tc[1][threadIdx.x] = c[1];
            tc[2][threadIdx.x] = c[2];
        }
        __syncthreads();
        // unused axes have coordinate 0 on both sides and spacing 0
        for (int k = 0; k < m; ++k) {
            const int32_t f = tile[k];
            const double d0 = (double)(p[0] - tc[0][k]);
            const double d1 = (double)(p[1] - tc[1][k]);
            const double d2a = (double)(p[2] - tc[2][k]);
            const double d2 = sh.s2[0] * d0 * d0 + sh.s2[1] * d1 * d1 + sh.s2[2] * d2a * d2a;
            if (d2 < best || (d2 == best && f < bidx)) {
                best = d2;
                bidx = f;
            }
        }
    }
    if (!mine) return;
    if (nbg == 0) {   // the virtual element at (-1, 0, ..., 0)
        const double d0 = (double)(p[0] + 1);
        best = sh.s2[0] * d0 * d0;
        for (int a = 1; a < sh.ndim; ++a) best += sh.s2[a] * (double)p[a] * (double)p[a];
        bidx = (int32_t)(-(sh.per / sh.n[0]));
    }
    const int64_t o = b * sh.per + i;
    if (sqdist) sqdist[o] = (int32_t)best;
    if (dist) dist[o] = __builtin_amdgcn_sqrtf((float)best);
    if (indices) indices[o] = bidx;
}

// grid: (ceil(per / (256 * kEpt)), images).  Element j of a thread is
// blockIdx.x * 256 * kEpt + j * 256 + threadIdx.x.  Outputs: idist (the
// integer distance), fdist (its float32 square root, squared metric only),
// indices; each may be null.
template <int M, int ND>
__global__ __launch_bounds__(256) void k_brute_int(const int32_t* __restrict__ list,
                                                   const int32_t* __restrict__ counts, ImageShape sh,
                                                   int32_t* __restrict__ idist,
                                                   float* __restrict__ fdist,
                                                   int32_t* __restrict__ indices) {
    __shared__ uint4 tile[kBruteTile];   // {c0, c1, c2, flat index}
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kEpt) + threadIdx.x;
    uint32_t p[kEpt][3];
    uint32_t best[kEpt];
    int32_t bidx[kEpt];
#pragma unroll
    for (int j = 0; j < kEpt; ++j) {
        const int64_t i = i0 + j * 256;
        int c[3];
        coords_of(sh, i < sh.per ? (int)i : 0, c);
        p[j][0] = (uint32_t)c[0];
        p[j][1] = (uint32_t)c[1];
        p[j][2] = (uint32_t)c[2];
        best[j] = 0xFFFFFFFFu;
        bidx[j] = 0x7FFFFFFF;
    }
    const int nbg = counts[b];
    const int32_t* lb = list + b * sh.per;
    for (int t0 = 0; t0 < nbg; t0 += kBruteTile) {
        const int m = min(kBruteTile, nbg - t0);
        __syncthreads();
        if ((int)threadIdx.x < m) {
            const int32_t f = lb[t0 + threadIdx.x];
            int c[3];
            coords_of(sh, f, c);
            tile[threadIdx.x] = make_uint4((uint32_t)c[0], (uint32_t)c[1], (uint32_t)c[2], (uint32_t)f);
        }
        __syncthreads();
        for (int k = 0; k < m; ++k) {
            const uint4 t = tile[k];
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const uint32_t d = metric_of<M, ND>(p[j], t);
                if (d < best[j]) {   // ascending list: the first minimiser is the smallest index
                    best[j] = d;
                    bidx[j] = (int32_t)t.w;
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kEpt; ++j) {
        const int64_t i = i0 + j * 256;
        if (i >= sh.per) continue;
        uint32_t d = best[j];
        int32_t idx = bidx[j];
        if (nbg == 0) {
            d = virtual_metric<M>(p[j], sh.ndim);
            idx = (int32_t)(-(sh.per / sh.n[0]));
        }
        const int64_t o = b * sh.per + i;
        if (idist) idist[o] = (int32_t)d;
        if (fdist) fdist[o] = __builtin_amdgcn_sqrtf((float)d);
        if (indices) indices[o] = idx;
    }
}

namespace {

ImageShape make_shape(int ndim, const int* n, const double* s2) {
    ImageShape sh{};
    sh.ndim = ndim;
    sh.per = 1;
    for (int a = 0; a < 3; ++a) {
        sh.n[a] = a < ndim ? n[a] : 1;
        sh.s2[a] = (a < ndim && s2) ? s2[a] : 0.0;
        sh.per *= sh.n[a];
    }
    return sh;
}

int64_t list_blocks(int64_t per) { return (per + kListBlock - 1) / kListBlock; }

hipError_t build_list(const uint8_t* mask, int B, const ImageShape& sh, int32_t* list,
                      int32_t* counts, int32_t* block_off, hipStream_t s) {
    const int64_t nblk = list_blocks(sh.per);
    const dim3 grid((unsigned)nblk, (unsigned)B);
    hipLaunchKernelGGL(k_bg_count, grid, dim3(256), 0, s, mask, sh.per, block_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bg_scan, dim3((unsigned)B), dim3(256), 0, s, block_off, nblk, counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bg_write, grid, dim3(256), 0, s, mask, sh.per, block_off, list);
    return hipGetLastError();
}

template <int M>
hipError_t launch_int(const ImageShape& sh, int B, const int32_t* list, const int32_t* counts,
                      int32_t* idist, float* fdist, int32_t* indices, hipStream_t s) {
    const dim3 grid((unsigned)((sh.per + 256 * kEpt - 1) / (256 * kEpt)), (unsigned)B);
    if (sh.ndim == 1)
        hipLaunchKernelGGL((k_brute_int<M, 1>), grid, dim3(256), 0, s, list, counts, sh, idist, fdist, indices);
    else if (sh.ndim == 2)
        hipLaunchKernelGGL((k_brute_int<M, 2>), grid, dim3(256), 0, s, list, counts, sh, idist, fdist, indices);
    else
        hipLaunchKernelGGL((k_brute_int<M, 3>), grid, dim3(256), 0, s, list, counts, sh, idist, fdist, indices);
    return hipGetLastError();
}

}  // namespace

size_t brute_list_block_count(int64_t per) { return (size_t)list_blocks(per); }

hipError_t launch_brute(const uint8_t* mask, int B, int ndim, const int* n, const double* s2,
                        int32_t* list, int32_t* counts, int32_t* block_off, int32_t* sqdist,
                        float* dist, int32_t* indices, hipStream_t s) {
    const ImageShape sh = make_shape(ndim, n, s2);
    hipError_t e = build_list(mask, B, sh, list, counts, block_off, s);
    if (e != hipSuccess) return e;
    // unit spacing with every squared distance (the virtual element's
    // included) below 2^31: the integer kernel gives the same values
    bool unit = true;
    double mx = 0.0;
    for (int a = 0; a < ndim; ++a) {
        unit = unit && s2[a] == 1.0;
        mx += (double)n[a] * (double)n[a];
    }
    if (unit && mx <= 2147483647.0)
        return launch_int<kBruteSquared>(sh, B, list, counts, sqdist, dist, indices, s);
    const dim3 grid((unsigned)((sh.per + 255) / 256), (unsigned)B);
    hipLaunchKernelGGL(k_brute, grid, dim3(256), 0, s, list, counts, sh, sqdist, dist, indices);
    return hipGetLastError();
}

hipError_t launch_brute_metric(const uint8_t* mask, int B, int ndim, const int* n, int metric,
                               int32_t* list, int32_t* counts, int32_t* block_off, int32_t* dist,
                               int32_t* indices, hipStream_t s) {
    const ImageShape sh = make_shape(ndim, n, nullptr);
    hipError_t e = build_list(mask, B, sh, list, counts, block_off, s);
    if (e != hipSuccess) return e;
    if (metric == kBruteTaxicab)
        return launch_int<kBruteTaxicab>(sh, B, list, counts, dist, nullptr, indices, s);
    if (metric == kBruteChessboard)
        return launch_int<kBruteChessboard>(sh, B, list, counts, dist, nullptr, indices, s);
    return hipErrorInvalidValue;
}

}  // namespace edt
