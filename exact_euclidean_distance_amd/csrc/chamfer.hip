// chamfer.hip -- the city-block (taxicab, L1) distance transform, one of the
// chamfer transforms TorchMorph ships beside its EDT (the pages name them
// without defining them; read as the L1 metric, SciPy's `taxicab`).
//
// The L1 distance is a sum of per-axis terms, so it separates like the EDT:
// after the axis-0 pass (the nearest background row of each column is the
// nearest in |.| as well), every further axis applies the 1-D transform
//   h(q) = min_j ( |q - j| + g(j) )
//        = min( q + min_{j <= q} (g(j) - j),  -q + min_{j >= q} (g(j) + j) ),
// a prefix minimum and a suffix minimum -- no envelope is needed.  Minima are
// taken over packed 64-bit keys ((value + offset) << 32 | j), so that one
// integer minimum gives both the value and its (smallest) position.
//
//   k_l1_rows   last axis + outputs: lane g of a line holds K = 32 consecutive
//               positions; in-chunk prefix minima stay in registers, the
//               chunks of a line are joined by segmented wave shuffles (and
//               LDS across the waves of a long line), then a backward sweep
//               adds the suffix minima and writes int32 distances and indices.
//   k_l1_cols   middle axis of a volume: one lane per line (neighbouring lanes,
//               neighbouring columns), a forward sweep storing the prefix
//               owners and a backward sweep finishing them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

constexpr int kL1K = 32;                       // positions per lane (last axis)
constexpr int64_t kL1Off = int64_t(1) << 20;   // keeps g - j + offset positive
constexpr uint64_t kL1Inf = ~uint64_t(0);

__device__ inline uint64_t l1_key(int64_t v, int j) {
    return ((uint64_t)(v + kL1Off) << 32) | (uint32_t)j;
}
__device__ inline int64_t l1_val(uint64_t k) { return (int64_t)(k >> 32) - kL1Off; }
__device__ inline int l1_arg(uint64_t k) { return (int)(uint32_t)k; }
__device__ inline uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

}  // namespace

// Rows of B images (2-D): value = nearest background row of the column.
struct L1Rows2D {
    using Val = uint16_t;
    int H, W;
    __device__ static bool valid(Val v) { return v != kNone16; }
    // row of line ln within its image
    __device__ unsigned ctx(int64_t ln) const { return (unsigned)(ln % H); }
    __device__ int g(unsigned c, Val v) const {
        const int row = (int)c;
        return row > (int)v ? row - (int)v : (int)v - row;
    }
    __device__ int32_t index(unsigned, Val v, int j) const { return (int32_t)v * W + j; }
    __device__ int virt(unsigned c, int q) const { return (int)c + 1 + q; }
    __device__ int32_t virt_index() const { return -W; }
};

// Rows of B volumes (3-D): value = packed (axis0 << 16 | axis1) owner.
struct L1Rows3D {
    using Val = uint32_t;
    int D, H, W;
    __device__ static bool valid(Val v) { return v != kNone32; }
    // (d << 16 | h) of line ln
    __device__ unsigned ctx(int64_t ln) const {
        const int64_t dh = ln % ((int64_t)D * H);
        return (unsigned)(((dh / H) << 16) | (dh % H));
    }
    __device__ int g(unsigned c, Val v) const {
        const int d = (int)(c >> 16), h = (int)(c & 0xFFFFu);
        const int z = (int)(v >> 16), y = (int)(v & 0xFFFFu);
        return (d > z ? d - z : z - d) + (h > y ? h - y : y - h);
    }
    __device__ int32_t index(unsigned, Val v, int j) const {
        return (int32_t)(((int64_t)(v >> 16) * H + (v & 0xFFFFu)) * W + j);
    }
    __device__ int virt(unsigned c, int q) const { return (int)(c >> 16) + 1 + (int)(c & 0xFFFFu) + q; }
    __device__ int32_t virt_index() const { return -(H * W); }
};

// Gp lanes per line (power of two, Gp * kL1K >= L), LPW lines per block of
// max(Gp, 64) threads.  For Gp > 64 the line spans Gp / 64 waves.
template <class Geo>
__global__ __launch_bounds__(1024) void k_l1_rows(const typename Geo::Val* __restrict__ in, int L,
                                                  int64_t nlines, int lgGp, Geo geo,
                                                  int32_t* __restrict__ dist,
                                                  int32_t* __restrict__ indices) {
    using Val = typename Geo::Val;
    __shared__ uint64_t wf[16], wb[16];   // per-wave totals of a long line
    const int Gp = 1 << lgGp;
    const int tid = threadIdx.x;
    const int g = tid & (Gp - 1);
    const int64_t line = (int64_t)blockIdx.x * (blockDim.x >> lgGp) + (tid >> lgGp);
    const bool active = line < nlines;
    const unsigned c = geo.ctx(active ? line : 0);
    const Val* src = in + (active ? line : 0) * (int64_t)L;
    const int p0 = g * kL1K;

    // in-chunk prefix minima of the forward keys (kept as the winner's offset
    // in the chunk, 8 bits each, 0xFF: none yet), and the chunk's backward minimum
    uint32_t pk[kL1K / 4];
    uint64_t run = kL1Inf, bmin = kL1Inf;
    uint32_t woff = 0xFFu;
#pragma unroll
    for (int t = 0; t < kL1K; ++t) {
        const int p = p0 + t;
        if (active && p < L) {
            const Val v = src[p];
            if (Geo::valid(v)) {
                const int gv = geo.g(c, v);
                const uint64_t kf = l1_key((int64_t)gv - p, p);
                if (kf < run) { run = kf; woff = (uint32_t)t; }
                bmin = umin64(bmin, l1_key((int64_t)gv + p, p));
            }
        }
        if ((t & 3) == 0) pk[t >> 2] = 0;
        pk[t >> 2] |= woff << (8 * (t & 3));
    }
    // exclusive minima over the chunks before (forward) and after (backward)
    const int S = Gp < 64 ? Gp : 64;   // chunks of the line in this wave
    const int pos = g & (S - 1);
    uint64_t fx = run, bx = bmin;
    for (int d = 1; d < S; d <<= 1) {
        const uint64_t u = __shfl_up(fx, d, S);
        const uint64_t w = __shfl_down(bx, d, S);
        if (pos >= d) fx = umin64(fx, u);
        if (pos + d < S) bx = umin64(bx, w);
    }
    uint64_t fe = __shfl_up(fx, 1, S), be = __shfl_down(bx, 1, S);
    if (pos == 0) fe = kL1Inf;
    if (pos == S - 1) be = kL1Inf;
    if (Gp > 64) {   // the waves of one long line (one line per block)
        const int wv = tid >> 6, nw = Gp >> 6;
        if ((tid & 63) == 63) wf[wv] = fx;
        if ((tid & 63) == 0) wb[wv] = bx;
        __syncthreads();
        for (int k = 0; k < wv; ++k) fe = umin64(fe, wf[k]);
        for (int k = wv + 1; k < nw; ++k) be = umin64(be, wb[k]);
    }
    if (!active || p0 >= L) return;

    // backward sweep: suffix minima, combined with the forward ones
    int32_t* dst = dist ? dist + line * (int64_t)L : nullptr;
    int32_t* ixd = indices ? indices + line * (int64_t)L : nullptr;
    uint64_t rb = be;
#pragma unroll
    for (int t = kL1K - 1; t >= 0; --t) {
        const int p = p0 + t;
        if (p < L) {
            const Val v = src[p];
            if (Geo::valid(v)) rb = umin64(rb, l1_key((int64_t)geo.g(c, v) + p, p));
            const uint32_t o = (pk[t >> 2] >> (8 * (t & 3))) & 0xFFu;
            uint64_t kf = fe;
            if (o != 0xFFu) {
                const int jf = p0 + (int)o;
                kf = umin64(kf, l1_key((int64_t)geo.g(c, src[jf]) - jf, jf));
            }
            int out;
            int32_t ix;
            if (kf == kL1Inf && rb == kL1Inf) {   // no background in the image
                out = geo.virt(c, p);
                ix = geo.virt_index();
            } else {
                const int64_t vf = kf == kL1Inf ? INT64_MAX : l1_val(kf) + p;
                const int64_t vb = rb == kL1Inf ? INT64_MAX : l1_val(rb) - p;
                const bool f = vf <= vb;
                const int j = f ? l1_arg(kf) : l1_arg(rb);
                out = (int)(f ? vf : vb);
                ix = geo.index(c, src[j], j);
            }
            if (dst) dst[p] = out;
            if (ixd) ixd[p] = ix;
        }
    }
}

// Middle axis of B volumes: lines along axis 1 at fixed (volume, d, w); input
// the axis-0 nearest coordinate, output packed (axis0 << 16 | axis1) owners.
__global__ __launch_bounds__(256) void k_l1_cols(const uint16_t* __restrict__ c0,
                                                 uint32_t* __restrict__ out, int D, int H, int W,
                                                 int64_t nlines) {
    const int64_t ln = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (ln >= nlines) return;
    const int64_t plane = ln / W;          // volume * D + d
    const int w = (int)(ln - plane * W);
    const int d = (int)(plane % D);
    const uint16_t* src = c0 + plane * (int64_t)H * W + w;
    uint32_t* dst = out + plane * (int64_t)H * W + w;
    // forward: owner of the smallest g(j) - j over j <= y
    uint64_t run = kL1Inf;
    uint32_t rz = 0;
    for (int y = 0; y < H; ++y) {
        const uint16_t v = src[(int64_t)y * W];
        if (v != kNone16) {
            const int gv = d > (int)v ? d - (int)v : (int)v - d;
            const uint64_t k = l1_key((int64_t)gv - y, y);
            if (k < run) { run = k; rz = v; }
        }
        dst[(int64_t)y * W] = run == kL1Inf ? kNone32 : ((rz << 16) | (uint32_t)l1_arg(run));
    }
    // backward: owner of the smallest g(j) + j over j >= y; keep the nearer
    run = kL1Inf;
    rz = 0;
    for (int y = H - 1; y >= 0; --y) {
        const uint16_t v = src[(int64_t)y * W];
        if (v != kNone16) {
            const int gv = d > (int)v ? d - (int)v : (int)v - d;
            const uint64_t k = l1_key((int64_t)gv + y, y);
            if (k < run) { run = k; rz = v; }
        }
        if (run == kL1Inf) continue;   // the forward owner (or none) stands
        const uint32_t f = dst[(int64_t)y * W];
        const int64_t vb = l1_val(run) - y;
        bool take_b = true;
        if (f != kNone32) {
            const int z = (int)(f >> 16), yf = (int)(f & 0xFFFFu);
            const int64_t vf = (d > z ? d - z : z - d) + (y - yf);
            take_b = vb < vf;
        }
        if (take_b) dst[(int64_t)y * W] = (rz << 16) | (uint32_t)l1_arg(run);
    }
}

namespace {

template <class Geo>
hipError_t launch_l1_rows_t(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                            int32_t* dist, int32_t* indices, hipStream_t s, KernelTimer* tm) {
    int lg = 0;
    while ((kL1K << lg) < L) ++lg;
    if (lg > 10) return hipErrorInvalidValue;   // more than 1024 lanes
    const int Gp = 1 << lg;
    const int threads = Gp < 64 ? 64 : Gp;
    const int64_t per_block = threads >> lg;
    const int64_t blocks = (nlines + per_block - 1) / per_block;
    EDT_LAUNCH(tm, "taxicab_rows", s,
               hipLaunchKernelGGL(k_l1_rows<Geo>, dim3((unsigned)blocks), dim3(threads), 0, s, in, L,
                                  nlines, lg, geo, dist, indices));
    return hipSuccess;
}

}  // namespace

hipError_t launch_l1_rows_2d(const uint16_t* c0, int B, int H, int W, int32_t* dist,
                             int32_t* indices, hipStream_t s, KernelTimer* tm) {
    return launch_l1_rows_t(c0, W, (int64_t)B * H, L1Rows2D{H, W}, dist, indices, s, tm);
}

hipError_t launch_l1_cols_3d(const uint16_t* c0, int B, int D, int H, int W, uint32_t* c01,
                             hipStream_t s, KernelTimer* tm) {
    const int64_t nlines = (int64_t)B * D * W;
    EDT_LAUNCH(tm, "taxicab_cols", s,
               hipLaunchKernelGGL(k_l1_cols, dim3((unsigned)((nlines + 255) / 256)), dim3(256), 0, s,
                                  c0, c01, D, H, W, nlines));
    return hipSuccess;
}

hipError_t launch_l1_rows_3d(const uint32_t* c01, int B, int D, int H, int W, int32_t* dist,
                             int32_t* indices, hipStream_t s, KernelTimer* tm) {
    return launch_l1_rows_t(c01, W, (int64_t)B * D * H, L1Rows3D{D, H, W}, dist, indices, s, tm);
}

}  // namespace edt
