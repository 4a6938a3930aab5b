// chamfer.hip -- the city-block (taxicab) transform, one of the chamfer
// transforms TorchMorph ships beside its EDT (the pages name them without
// defining them; read as the L1 and L-infinity metrics, SciPy's `taxicab`
// and `chessboard`).
//
// The L1 distance is a sum of per-axis terms, so it separates like the EDT:
// after the axis-0 pass (the nearest background row of each column is the
// nearest in |.| as well), every further axis applies the 1-D transform
//   h(q) = min_j ( |q - j| + g(j) )
//        = min( q + min_{j <= q} (g(j) - j),  -q + min_{j >= q} (g(j) + j) ),
// a prefix minimum and a suffix minimum -- no envelope is needed.  Minima are
// taken over packed 64-bit keys (value first, then position, and in the row
// pass the source value too), so that one integer minimum gives the value and
// its (smallest) position.
//
//   k_l1_rows   last axis + outputs: a wave takes tiles of 256 positions of a
//               line, four consecutive positions per lane (coalesced loads
//               and stores); prefix minima in a forward sweep and suffix
//               minima in a backward one, each in-lane, then by a wave scan,
//               then across tiles (and across the waves of a long line
//               through LDS); the keys carry the owner's source value, so
//               the index needs no second read.
//   k_l1_cols   middle axis of a volume: one lane per line (neighbouring lanes,
//               neighbouring columns), a forward sweep storing the prefix
//               owners and a backward sweep finishing them, both reading
//               batches of rows so that many loads are in flight.
//
// The chessboard (L-infinity) distance separates as well: after the axis-0
// pass every further axis applies h(q) = min_j max(g(j), |q - j|), a min-max
// with no prefix-minimum form.  It runs on the envelope kernels of
// kernels.hip under the chessboard metric (LinfMetric in envelope.h:
// integer crossings of the functions max(g_j, |q - j|), which change places
// once, as parabolas do).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

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

// Keys of the row pass: value << 47 | position << 32 | source value.  The
// value is below 2^17 (g <= 65534 + 32767, rows of at most 32768, offset
// 2^15 on the forward side) and the position below 2^15, so one unsigned
// minimum gives the smallest value, then the smallest position, and carries
// the owner's source value along for its index.
constexpr int kRowOff = 1 << 15;   // g(j) - j + kRowOff >= 1

__device__ inline uint64_t row_key(int val, int j, uint32_t v) {
    return ((uint64_t)(uint32_t)val << 47) | ((uint64_t)(uint32_t)j << 32) | v;
}
__device__ inline int row_val(uint64_t k) { return (int)(k >> 47); }
__device__ inline int row_pos(uint64_t k) { return (int)((k >> 32) & 0x7FFFu); }

__device__ inline uint64_t wave_prefix_min(uint64_t x, int lane) {   // lanes <= lane
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t u = __shfl_up(x, d, 64);
        if (lane >= d) x = umin64(x, u);
    }
    return x;
}
__device__ inline uint64_t wave_suffix_min(uint64_t x, int lane) {   // lanes >= lane
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t u = __shfl_down(x, d, 64);
        if (lane + d < 64) x = umin64(x, u);
    }
    return x;
}
__device__ inline uint64_t wave_min(uint64_t x) {
    for (int d = 1; d < 64; d <<= 1) x = umin64(x, __shfl_xor(x, d, 64));
    return x;
}

// Last axis + outputs.  A wave owns a segment of T tiles of 256 positions of a
// line; in tile t lane l holds the four positions 256 t + 4 l + (0..3), so that
// loads and stores are coalesced 8- or 16-byte pieces.  A forward sweep over
// the tiles takes prefix minima of the forward keys (in-lane, then a wave scan,
// then the running minimum of the tiles before); a backward sweep takes the
// suffix minima the same way and writes each position's nearer side.  NW == 1:
// four lines per block, one per wave; NW > 1: one line per block, its NW waves
// joined through the per-wave minima in LDS.
template <class Geo, int T>
__global__ __launch_bounds__(1024) void k_l1_rows(const typename Geo::Val* __restrict__ in, int L,
                                                  int64_t nlines, int NW, int vec, Geo geo,
                                                  int32_t* __restrict__ dist,
                                                  int32_t* __restrict__ indices) {
    using Val = typename Geo::Val;
    constexpr Val kNone = (Val)~Val(0);
    __shared__ uint64_t wtf[16], wtb[16];   // per-wave minima of a line of several waves
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t line = NW == 1 ? (int64_t)blockIdx.x * (blockDim.x >> 6) + w : (int64_t)blockIdx.x;
    if (line >= nlines) return;   // only when NW == 1: no barrier follows there
    const int seg0 = NW == 1 ? 0 : w * (T * 256);
    const unsigned c = geo.ctx(line);
    const Val* src = in + line * (int64_t)L;

    Val v[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int p = seg0 + 256 * t + 4 * lane;
        if (vec && p < L) {   // L % 4 == 0: the whole piece is in the line
            if constexpr (sizeof(Val) == 4) {
                const uint4 x = *reinterpret_cast<const uint4*>(src + p);
                v[t][0] = x.x; v[t][1] = x.y; v[t][2] = x.z; v[t][3] = x.w;
            } else {
                const uint2 x = *reinterpret_cast<const uint2*>(src + p);
                v[t][0] = (Val)x.x; v[t][1] = (Val)(x.x >> 16); v[t][2] = (Val)x.y; v[t][3] = (Val)(x.y >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[t][i] = p + i < L ? src[p + i] : kNone;
        }
    }
    auto kf = [&](int t, int i) -> uint64_t {   // forward key of a position (none: all ones)
        const Val x = v[t][i];
        const int p = seg0 + 256 * t + 4 * lane + i;
        return Geo::valid(x) ? row_key(geo.g(c, x) - p + kRowOff, p, (uint32_t)x) : kL1Inf;
    };
    auto kb = [&](int t, int i) -> uint64_t {   // backward key
        const Val x = v[t][i];
        const int p = seg0 + 256 * t + 4 * lane + i;
        return Geo::valid(x) ? row_key(geo.g(c, x) + p, p, (uint32_t)x) : kL1Inf;
    };

    uint64_t cf = kL1Inf, cb = kL1Inf;   // minima over the positions before / after the segment
    if (NW > 1) {
        uint64_t tf = kL1Inf, tb = kL1Inf;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tf = umin64(tf, kf(t, i));
                tb = umin64(tb, kb(t, i));
            }
        tf = wave_min(tf);
        tb = wave_min(tb);
        if (lane == 0) {
            wtf[w] = tf;
            wtb[w] = tb;
        }
        __syncthreads();
        for (int k = 0; k < w; ++k) cf = umin64(cf, wtf[k]);
        for (int k = w + 1; k < NW; ++k) cb = umin64(cb, wtb[k]);
    }

    // forward sweep: fx[t] = minimum over the positions before this lane's piece
    uint64_t fx[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        uint64_t a = kL1Inf;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = umin64(a, kf(t, i));
        const uint64_t inc = wave_prefix_min(a, lane);
        uint64_t ex = __shfl_up(inc, 1, 64);
        if (lane == 0) ex = kL1Inf;
        fx[t] = umin64(ex, cf);
        cf = umin64(cf, __shfl(inc, 63, 64));
    }

    // backward sweep and outputs
    const bool vout = vec != 0;
    int32_t* drow = dist ? dist + line * (int64_t)L : nullptr;
    int32_t* irow = indices ? indices + line * (int64_t)L : nullptr;
#pragma unroll
    for (int t = T - 1; t >= 0; --t) {
        uint64_t b = kL1Inf;
#pragma unroll
        for (int i = 0; i < 4; ++i) b = umin64(b, kb(t, i));
        const uint64_t sinc = wave_suffix_min(b, lane);
        uint64_t rb = __shfl_down(sinc, 1, 64);
        if (lane == 63) rb = kL1Inf;
        rb = umin64(rb, cb);
        cb = umin64(cb, __shfl(sinc, 0, 64));

        const int p = seg0 + 256 * t + 4 * lane;
        if (p >= L) continue;
        uint64_t f[4];
        uint64_t run = fx[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run = umin64(run, kf(t, i));
            f[i] = run;
        }
        int out[4];
        int32_t ix[4];
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            rb = umin64(rb, kb(t, i));
            const int q = p + i;
            if (f[i] == kL1Inf && rb == kL1Inf) {   // no background in the image
                out[i] = geo.virt(c, q);
                ix[i] = geo.virt_index();
            } else {
                const int vf = f[i] == kL1Inf ? INT32_MAX : row_val(f[i]) - kRowOff + q;
                const int vb = rb == kL1Inf ? INT32_MAX : row_val(rb) - q;
                const uint64_t k = vf <= vb ? f[i] : rb;
                out[i] = vf <= vb ? vf : vb;
                ix[i] = geo.index(c, (Val)(uint32_t)k, row_pos(k));
            }
        }
        if (vout) {
            if (drow) *reinterpret_cast<int4*>(drow + p) = make_int4(out[0], out[1], out[2], out[3]);
            if (irow) *reinterpret_cast<int4*>(irow + p) = make_int4(ix[0], ix[1], ix[2], ix[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (p + i < L) {
                    if (drow) drow[p + i] = out[i];
                    if (irow) irow[p + i] = ix[i];
                }
            }
        }
    }
}

// Middle axis of B volumes: lines along axis 1 at fixed (volume, d, w); input
// the axis-0 nearest coordinate, output packed (axis0 << 16 | axis1) owners.
// Rows are read kColBatch at a time, so that a lane keeps that many loads in
// flight instead of one.
constexpr int kColBatch = 8;

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
    for (int y0 = 0; y0 < H; y0 += kColBatch) {
        uint16_t vb[kColBatch];
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) vb[i] = y0 + i < H ? src[(int64_t)(y0 + i) * W] : kNone16;
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) {
            const int y = y0 + i;
            if (y >= H) break;
            const uint16_t v = vb[i];
            if (v != kNone16) {
                const int gv = d > (int)v ? d - (int)v : (int)v - d;
                const uint64_t k = l1_key((int64_t)gv - y, y);
                if (k < run) { run = k; rz = v; }
            }
            dst[(int64_t)y * W] = run == kL1Inf ? kNone32 : ((rz << 16) | (uint32_t)l1_arg(run));
        }
    }
    // backward: owner of the smallest g(j) + j over j >= y; keep the nearer
    run = kL1Inf;
    rz = 0;
    for (int y0 = ((H - 1) / kColBatch) * kColBatch; y0 >= 0; y0 -= kColBatch) {
        uint16_t vb[kColBatch];
        uint32_t fb[kColBatch];
#pragma unroll
        for (int i = 0; i < kColBatch; ++i) {
            const bool in = y0 + i < H;
            vb[i] = in ? src[(int64_t)(y0 + i) * W] : kNone16;
            fb[i] = in ? dst[(int64_t)(y0 + i) * W] : kNone32;
        }
#pragma unroll
        for (int i = kColBatch - 1; i >= 0; --i) {
            const int y = y0 + i;
            if (y >= H) continue;
            const uint16_t v = vb[i];
            if (v != kNone16) {
                const int gv = d > (int)v ? d - (int)v : (int)v - d;
                const uint64_t k = l1_key((int64_t)gv + y, y);
                if (k < run) { run = k; rz = v; }
            }
            if (run == kL1Inf) continue;   // the forward owner (or none) stands
            const uint32_t f = fb[i];
            const int64_t vbk = l1_val(run) - y;
            bool take_b = true;
            if (f != kNone32) {
                const int z = (int)(f >> 16), yf = (int)(f & 0xFFFFu);
                const int64_t vf = (d > z ? d - z : z - d) + (y - yf);
                take_b = vbk < vf;
            }
            if (take_b) dst[(int64_t)y * W] = (rz << 16) | (uint32_t)l1_arg(run);
        }
    }
}

namespace {

template <class Geo>
hipError_t launch_l1_rows_t(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                            int32_t* dist, int32_t* indices, hipStream_t s, KernelTimer* tm) {
    using Val = typename Geo::Val;
    const int T = L <= 256 ? 1 : L <= 512 ? 2 : L <= 16384 ? 4 : 8;
    const int NW = (L + 256 * T - 1) / (256 * T);
    if (L > 32768 || NW > 16) return hipErrorInvalidValue;
    const int threads = NW == 1 ? 256 : 64 * NW;
    const int64_t blocks = NW == 1 ? (nlines + 3) / 4 : nlines;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const bool al_in = ((uintptr_t)in % (4 * sizeof(Val))) == 0;
    const bool al_out = ((uintptr_t)dist % 16) == 0 && ((uintptr_t)indices % 16) == 0;
    const int vec = (L % 4 == 0 && al_in && al_out) ? 1 : 0;
#define EDT_L1_ROWS(TT)                                                                          \
    EDT_LAUNCH(tm, "taxicab_rows", s,                                                            \
               hipLaunchKernelGGL((k_l1_rows<Geo, TT>), dim3((unsigned)blocks), dim3(threads), 0, s, \
                                  in, L, nlines, NW, vec, geo, dist, indices))
    switch (T) {
        case 1: EDT_L1_ROWS(1); break;
        case 2: EDT_L1_ROWS(2); break;
        case 4: EDT_L1_ROWS(4); break;
        default: EDT_L1_ROWS(8); break;
    }
#undef EDT_L1_ROWS
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
