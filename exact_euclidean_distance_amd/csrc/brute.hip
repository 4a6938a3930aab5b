// brute.hip -- the transform by its definition, on the GPU: every element
// against every background element of its image (TorchMorph's brute-force
// transform, the exactness oracle beside its EDT; the Voronoi page's per-cell
// search).  O(elements x background elements): a checker for small images,
// not a fast path.
//
//   k_bg_list   per image, the flat indices of its background elements
//               (order unspecified) and their count;
//   k_brute     per element, the lexicographically smallest (squared distance,
//               index) over its image's list, read in tiles of 256 through
//               LDS; images without background take the virtual element at
//               (-1, 0, ..., 0).
// The smallest index among equally near background elements is returned, so
// the result does not depend on the list order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

constexpr int kBruteTile = 256;

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

}  // namespace

__global__ __launch_bounds__(256) void k_zero_counts(int32_t* __restrict__ counts, int B) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < B) counts[i] = 0;
}

// grid: (element blocks, images)
__global__ __launch_bounds__(256) void k_bg_list(const uint8_t* __restrict__ mask, int64_t per,
                                                 int32_t* __restrict__ list,
                                                 int32_t* __restrict__ counts) {
    const int64_t b = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool bg = i < per && mask[b * per + i] == 0;
    const uint64_t vote = __ballot(bg);
    if (!vote) return;
    const int lane = threadIdx.x & 63;
    const int leader = __builtin_ctzll(vote);
    int base = 0;
    if (lane == leader) base = atomicAdd(&counts[b], __popcll(vote));
    base = __shfl(base, leader);
    if (bg) {
        const int rank = __popcll(vote & ((uint64_t(1) << lane) - 1));
        list[b * per + base + rank] = (int32_t)i;
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

hipError_t launch_brute(const uint8_t* mask, int B, int ndim, const int* n, const double* s2,
                        int32_t* list, int32_t* counts, int32_t* sqdist, float* dist,
                        int32_t* indices, hipStream_t s) {
    ImageShape sh{};
    sh.ndim = ndim;
    sh.per = 1;
    for (int a = 0; a < 3; ++a) {
        sh.n[a] = a < ndim ? n[a] : 1;
        sh.s2[a] = a < ndim ? s2[a] : 0.0;
        sh.per *= sh.n[a];
    }
    hipLaunchKernelGGL(k_zero_counts, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, counts, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((sh.per + 255) / 256), (unsigned)B);
    hipLaunchKernelGGL(k_bg_list, grid, dim3(256), 0, s, mask, sh.per, list, counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_brute, grid, dim3(256), 0, s, list, counts, sh, sqdist, dist, indices);
    return hipGetLastError();
}

}  // namespace edt
