// chamfer.hip -- the chamfer transforms TorchMorph ships beside its EDT (the
// pages name them without defining them; read as the L1 and L-infinity
// metrics, SciPy's `taxicab` and `chessboard`).
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
// pass every further axis applies h(q) = min_j max(g(j), |q - j|).  That
// min-max has no prefix-minimum form.  Lines of up to kRmqMaxLine positions
// take amortised constant work per position (linf_rmq.h): h(q) <= r exactly
// when the window [q - r, q + r] holds a source with g <= r, and h moves by
// at most one between neighbours, so a lane bisects h at the first position
// of its run of 8 and then tests at most two windows per position, each
// answered from a blocked range-minimum structure in LDS.  Lines with at most
// kLinfList sources take the minimum over a list of them instead.
//
//   k_linf_rmq_cols  middle axis of a volume: a block stages g of TW
//                    neighbouring columns of one plane and writes packed
//                    (axis0 << 16 | axis1) owners.
//   k_linf_rmq_rows  last axis + outputs: a block stages g of whole lines and
//                    writes int32 distances and flat indices; the winners'
//                    source values are read back from the input together.
//
// Longer lines keep an outward search: each position scans its line staged
// in LDS (r = 0, 1, 2, ...); a source r away adds at least r, so the search
// ends once r reaches the best value found (work per position: its own
// distance), with the source list for sparse lines and per-bucket lists of
// the sources with small g for lines of 2048 or more:
//
//   k_linf_cols  middle axis of a volume (H > kRmqMaxLine).
//   k_linf_rows  last axis + outputs (W > kRmqMaxLine).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "linf_rmq.h"

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

// ---------------------------------------------------------------------------
// Chessboard (L-infinity) transform
// ---------------------------------------------------------------------------

// Rows of B images (2-D): value = nearest background row of the column.
struct LinfRows2D {
    using Val = uint16_t;
    int H, W;
    __device__ static bool valid(Val v) { return v != kNone16; }
    __device__ unsigned ctx(int64_t ln) const { return (unsigned)(ln % H); }
    __device__ int g(unsigned c, Val v) const {
        const int row = (int)c;
        return row > (int)v ? row - (int)v : (int)v - row;
    }
    __device__ int32_t index(unsigned, Val v, int j) const { return (int32_t)v * W + j; }
    __device__ int virt(unsigned c, int q) const { return max((int)c + 1, q); }
    __device__ int32_t virt_index() const { return -W; }
};

// Rows of B volumes (3-D): value = packed (axis0 << 16 | axis1) owner.
struct LinfRows3D {
    using Val = uint32_t;
    int D, H, W;
    __device__ static bool valid(Val v) { return v != kNone32; }
    __device__ unsigned ctx(int64_t ln) const {
        const int64_t dh = ln % ((int64_t)D * H);
        return (unsigned)(((dh / H) << 16) | (dh % H));
    }
    __device__ int g(unsigned c, Val v) const {
        const int d = (int)(c >> 16), h = (int)(c & 0xFFFFu);
        const int z = (int)(v >> 16), y = (int)(v & 0xFFFFu);
        return max(d > z ? d - z : z - d, h > y ? h - y : y - h);
    }
    __device__ int32_t index(unsigned, Val v, int j) const {
        return (int32_t)(((int64_t)(v >> 16) * H + (v & 0xFFFFu)) * W + j);
    }
    __device__ int virt(unsigned c, int q) const {
        return max(max((int)(c >> 16) + 1, (int)(c & 0xFFFFu)), q);
    }
    __device__ int32_t virt_index() const { return -(H * W); }
};

constexpr int kLinfStage = 2048;   // lines up to this length share a block
constexpr int kLinfThreads = 512;  // threads per block of either search pass
constexpr int kLinfList = 32;      // lines with at most this many sources scan them as a list
constexpr int kLinfBT = 128;       // bucket width = the g threshold of the bucket lists
constexpr int kLinfBC = 16;        // sources per bucket list
constexpr int kLinfBLine = 2048;   // lines this long or longer use the bucket lists (shorter
                                   // ones measured faster without their bookkeeping)

__host__ __device__ inline size_t linf_flags_offset(size_t bytes) { return (bytes + 15) & ~size_t(15); }

// Smallest max(g(j), |q - j|) over the sources of a staged line of L values,
// stride apart (at least one is a source), searching outward from q; ties go
// to the nearer, then the lower j.  gof(v): g of a source value, -1 for none.
template <class Val, class GFn>
__device__ inline int linf_search(const Val* lv, int stride, int q, int L, const GFn& gof, int& bj) {
    constexpr int R = 4;   // radii per step: their 2R reads are issued together
    int best = INT32_MAX;
    bj = -1;
    for (int r0 = 0; r0 < best; r0 += R) {
        if (q - r0 < 0 && q + r0 >= L) break;
        int gl[R], gr[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int j0 = q - r0 - k, j1 = q + r0 + k;
            gl[k] = j0 >= 0 ? gof(lv[j0 * stride]) : -1;
            gr[k] = j1 < L ? gof(lv[j1 * stride]) : -1;
        }
        // in the order of a one-radius-at-a-time search (radii past the end
        // add max(g, r) >= best and change nothing)
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int r = r0 + k;
            if (gl[k] >= 0 && max(gl[k], r) < best) { best = max(gl[k], r); bj = q - r; }
            if (r > 0 && gr[k] >= 0 && max(gr[k], r) < best) { best = max(gr[k], r); bj = q + r; }
        }
    }
    return best;
}

// The same minimum over a line's n sources listed by position (any order):
// for lines with few sources, whose outward search would walk far.
template <class GAt>
__device__ inline int linf_list(const uint16_t* lst, int n, int q, const GAt& gat, int& bj) {
    int best = INT32_MAX, bd = INT32_MAX;
    bj = -1;
    for (int i = 0; i < n; ++i) {
        const int j = lst[i];
        const int dj = q > j ? q - j : j - q;
        const int v = max(gat(j), dj);
        if (v < best || (v == best && (dj < bd || (dj == bd && j < bj)))) {
            best = v;
            bd = dj;
            bj = j;
        }
    }
    return best;
}

// LPB lines of L values per block (L <= kLinfStage: LPB = kLinfStage / L,
// else 1).  The lines are staged as g (16 bits, kNone16 for no source: g <=
// 65534 on every accepted shape); threads take consecutive positions of the
// block's lines, and the winner's source value is read back from the input
// for its index.
template <class Geo, bool BUCKETS>
__global__ __launch_bounds__(kLinfThreads) void k_linf_rows(const typename Geo::Val* __restrict__ in, int L,
                                                   int64_t nlines, int LPB, int vec, Geo geo,
                                                   int32_t* __restrict__ dist,
                                                   int32_t* __restrict__ indices) {
    using Val = typename Geo::Val;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* sg = reinterpret_cast<uint16_t*>(smem);                              // [LPB][L]
    int* cnt = reinterpret_cast<int*>(smem + linf_flags_offset((size_t)LPB * L * 2));   // [LPB] sources
    int* fill = cnt + LPB;                                                          // [LPB]
    unsigned* ctx = reinterpret_cast<unsigned*>(fill + LPB);                        // [LPB]
    int* small = reinterpret_cast<int*>(ctx + LPB);                                 // [LPB] g <= kLinfBT
    const int nbk = (L + kLinfBT - 1) / kLinfBT;                                    // buckets per line
    int* bcnt = small + LPB;                                                        // [LPB][nbk]
    uint16_t* blst = reinterpret_cast<uint16_t*>(bcnt + (L >= kLinfBLine ? LPB * nbk : 0));  // [LPB][nbk][kLinfBC]
    uint16_t* lst = blst + (L >= kLinfBLine ? LPB * nbk * kLinfBC : 0);              // [LPB][kLinfList]
    const bool lists = LPB <= kLinfList;   // (lines shorter than that search little anyway)
    constexpr bool buckets = BUCKETS;   // launched with L >= kLinfBLine
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t line0 = (int64_t)blockIdx.x * LPB;
    const int nl = (int)min<int64_t>(LPB, nlines - line0);
    const int total = nl * L;
    for (int l = tid; l < LPB; l += nt) {
        cnt[l] = 0;
        fill[l] = 0;
        small[l] = 0;
        ctx[l] = geo.ctx(line0 + (l < nl ? l : 0));
    }
    if (buckets)
        for (int i = tid; i < LPB * nbk; i += nt) bcnt[i] = 0;
    __syncthreads();
    const Val* src = in + line0 * (int64_t)L;
    auto gval = [&](Val v, unsigned c) -> uint16_t {
        return Geo::valid(v) ? (uint16_t)geo.g(c, v) : kNone16;
    };
    if (vec) {   // 16-byte pieces, each within one line (L * sizeof(Val) % 16 == 0)
        constexpr int VN = 16 / (int)sizeof(Val);
        const int npc = total / VN;
#pragma unroll 4
        for (int i = tid; i < npc; i += nt) {
            const uint4 w = reinterpret_cast<const uint4*>(src)[i];
            const int l = (i * VN) / L;
            const unsigned c = ctx[l];
            const Val* pv = reinterpret_cast<const Val*>(&w);
            uint16_t gs[VN];
            int nv = 0, ns = 0;
#pragma unroll
            for (int k = 0; k < VN; ++k) {
                gs[k] = gval(pv[k], c);
                nv += gs[k] != kNone16;
                ns += gs[k] <= kLinfBT;   // (kNone16 > kLinfBT)
            }
            if constexpr (VN == 8) {
                reinterpret_cast<uint4*>(sg)[i] =
                    make_uint4(gs[0] | ((uint32_t)gs[1] << 16), gs[2] | ((uint32_t)gs[3] << 16),
                               gs[4] | ((uint32_t)gs[5] << 16), gs[6] | ((uint32_t)gs[7] << 16));
            } else {
                reinterpret_cast<uint2*>(sg)[i] =
                    make_uint2(gs[0] | ((uint32_t)gs[1] << 16), gs[2] | ((uint32_t)gs[3] << 16));
            }
            if (nv) atomicAdd(&cnt[l], nv);
            if (buckets && ns) atomicAdd(&small[l], ns);
        }
    } else {
#pragma unroll 4
        for (int e = tid; e < total; e += nt) {
            const int l = e / L;
            const uint16_t gv = gval(src[e], ctx[l]);
            sg[e] = gv;
            if (gv != kNone16) atomicAdd(&cnt[l], 1);
            if (buckets && gv <= kLinfBT) atomicAdd(&small[l], 1);
        }
    }
    __syncthreads();
    // Lines with few sources list them all (any order).  Lines whose sources
    // of g <= kLinfBT are sparse enough list those per bucket of kLinfBT
    // positions (a bucket past kLinfBC of them is marked full by its count).
    auto bucketed = [&](int l) { return buckets && cnt[l] > kLinfList && small[l] <= (kLinfBC / 2) * nbk; };
    if (lists || buckets) {
        for (int e = tid; e < total; e += nt) {
            const int l = e / L, q = e - l * L;
            if (sg[e] == kNone16) continue;
            if (lists && cnt[l] <= kLinfList) {
                const int slot = atomicAdd(&fill[l], 1);   // < cnt[l]
                lst[l * kLinfList + slot] = (uint16_t)q;
            } else if (bucketed(l) && sg[e] <= kLinfBT) {
                const int bk = l * nbk + q / kLinfBT;
                const int slot = atomicAdd(&bcnt[bk], 1);
                if (slot < kLinfBC) blst[bk * kLinfBC + slot] = (uint16_t)q;
            }
        }
        __syncthreads();
    }
    auto gof = [](uint16_t gv) { return gv != kNone16 ? (int)gv : -1; };
    for (int e = tid; e < total; e += nt) {
        const int l = e / L, q = e - l * L;
        const int64_t ln = line0 + l;
        const unsigned c = ctx[l];
        const int n = cnt[l];
        int best;
        int32_t ix;
        if (n == 0) {   // no source on the line: only in an image without background
            best = geo.virt(c, q);
            ix = geo.virt_index();
        } else {
            const uint16_t* lg = sg + l * L;
            int bj = -1;
            auto gat = [&](int j) { return (int)lg[j]; };
            if (lists && n <= kLinfList) {
                best = linf_list(lst + l * kLinfList, n, q, gat, bj);
            } else {
                // buckets b - 1 .. b + 1 hold every source of g <= kLinfBT within
                // kLinfBT of q; a best found there that is <= kLinfBT is the
                // minimum (any other source is farther or has a larger g)
                best = INT32_MAX;
                if (buckets && bucketed(l)) {
                    const int b = q / kLinfBT;
                    bool full = false;
                    int bd = INT32_MAX;
                    for (int bb = max(b - 1, 0); bb <= min(b + 1, nbk - 1); ++bb) {
                        const int bk = l * nbk + bb;
                        const int m = bcnt[bk];
                        if (m > kLinfBC) { full = true; break; }
                        int j1, d1;
                        const int v = linf_list(blst + bk * kLinfBC, m, q, gat, j1);
                        if (j1 >= 0) {
                            d1 = q > j1 ? q - j1 : j1 - q;
                            if (v < best || (v == best && (d1 < bd || (d1 == bd && j1 < bj)))) {
                                best = v;
                                bd = d1;
                                bj = j1;
                            }
                        }
                    }
                    if (full || best > kLinfBT) best = INT32_MAX;
                }
                if (best == INT32_MAX) best = linf_search(lg, 1, q, L, gof, bj);
            }
            ix = geo.index(c, src[(int64_t)l * L + bj], bj);
        }
        if (dist) dist[ln * (int64_t)L + q] = best;
        if (indices) indices[ln * (int64_t)L + q] = ix;
    }
}

// Middle axis of B volumes: a block stages g of TW neighbouring columns (w0 ..
// w0 + TW - 1) of one plane (volume, d), all H rows, as sv[y][x]; thread x of
// row group yg answers rows yg, yg + kLinfThreads / TW, ... of column x.  Output: the
// packed (axis0 << 16 | axis1) owner, kNone32 for a column without a source.
__global__ __launch_bounds__(kLinfThreads) void k_linf_cols(const uint16_t* __restrict__ c0,
                                                   uint32_t* __restrict__ out, int D, int H, int W,
                                                   int TW, int vec) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* sv = reinterpret_cast<uint16_t*>(smem);                              // [H][TW]
    int* cnt = reinterpret_cast<int*>(smem + linf_flags_offset((size_t)H * TW * 2));   // [TW] sources
    int* fill = cnt + TW;                                                           // [TW]
    uint16_t* lst = reinterpret_cast<uint16_t*>(fill + TW);                         // [TW][kLinfList]
    const int tid = threadIdx.x;
    const int tiles = (W + TW - 1) / TW;
    const int64_t plane = blockIdx.x / tiles;          // volume * D + d
    const int w0 = (int)(blockIdx.x % tiles) * TW;
    const int d = (int)(plane % D);
    const int tw = min(TW, W - w0);                    // columns of this tile
    const uint16_t* src = c0 + plane * (int64_t)H * W + w0;
    uint32_t* dst = out + plane * (int64_t)H * W + w0;
    for (int x = tid; x < TW; x += kLinfThreads) {
        cnt[x] = 0;
        fill[x] = 0;
    }
    __syncthreads();
    // staged as g = |d - axis0| (kNone16: no source)
    auto gval = [&](uint16_t v) -> uint16_t {
        return v != kNone16 ? (uint16_t)(d > (int)v ? d - (int)v : (int)v - d) : kNone16;
    };
    if (vec && tw == TW) {   // rows of the tile in 16-byte pieces of 8 columns
        const int pr = TW / 8;   // pieces per row
#pragma unroll 4
        for (int i = tid; i < H * pr; i += kLinfThreads) {
            const int y = i / pr, k = i - y * pr;
            const uint4 w = *reinterpret_cast<const uint4*>(src + (int64_t)y * W + 8 * k);
            const uint16_t* pv = reinterpret_cast<const uint16_t*>(&w);
            uint16_t gs[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                gs[c] = gval(pv[c]);
                if (gs[c] != kNone16) atomicAdd(&cnt[8 * k + c], 1);
            }
            reinterpret_cast<uint4*>(sv + y * TW)[k] =
                make_uint4(gs[0] | ((uint32_t)gs[1] << 16), gs[2] | ((uint32_t)gs[3] << 16),
                           gs[4] | ((uint32_t)gs[5] << 16), gs[6] | ((uint32_t)gs[7] << 16));
        }
    } else {
#pragma unroll 4
        for (int e = tid; e < H * TW; e += kLinfThreads) {
            const int y = e / TW, x = e - y * TW;
            const uint16_t gv = x < tw ? gval(src[(int64_t)y * W + x]) : kNone16;
            sv[e] = gv;
            if (gv != kNone16) atomicAdd(&cnt[x], 1);
        }
    }
    __syncthreads();
    for (int e = tid; e < H * TW; e += kLinfThreads) {   // the sources of columns with few of them
        const int y = e / TW, x = e - y * TW;
        if (cnt[x] <= kLinfList && sv[e] != kNone16) {
            const int slot = atomicAdd(&fill[x], 1);   // < cnt[x]
            lst[x * kLinfList + slot] = (uint16_t)y;
        }
    }
    __syncthreads();
    const int x = tid % TW, yg = tid / TW, ys = kLinfThreads / TW;
    if (x >= tw || yg >= ys) return;   // no barrier follows
    const int n = cnt[x];
    auto gof = [](uint16_t gv) { return gv != kNone16 ? (int)gv : -1; };
    for (int y = yg; y < H; y += ys) {
        uint32_t o = kNone32;
        if (n > 0) {
            int bj;
            if (n <= kLinfList)
                linf_list(lst + x * kLinfList, n, y, [&](int j) { return (int)sv[j * TW + x]; }, bj);
            else
                linf_search(sv + x, TW, y, H, gof, bj);
            o = ((uint32_t)src[(int64_t)bj * W + x] << 16) | (uint32_t)bj;
        }
        dst[(int64_t)y * W + x] = o;
    }
}

// ---------------------------------------------------------------------------
// Chessboard lines with amortised constant work per position (linf_rmq.h):
// lines of at most kRmqMaxLine positions.  A block stages g of its lines (16
// bits, kRmqNoG for no source), builds each line's blocked range-minimum
// structure in LDS, and every thread answers runs of kRmqBlock consecutive
// positions (bisection at the first, then at most two window minima per
// position).
// ---------------------------------------------------------------------------

constexpr int kRmqMaxLine = 4096;
constexpr int kRmqThreads = 512;
constexpr size_t kRmqLineBudget = 56 * 1024;   // LDS of a block's lines (two blocks per CU)

// Per line: the staged g (halfwords) and the structure (words), each an odd
// number of 32-bit words, so that lanes at the same offset of different lines
// use different LDS banks.
__host__ __device__ inline int rmq_gstride(int L) { return 2 * ((rmq_g_halves(L) / 2 + 1) | 1); }
__host__ __device__ inline int rmq_stride(int L) { return rmq_words(L) | 1; }
__host__ __device__ inline size_t rmq_line_bytes(int L) {
    return (size_t)rmq_gstride(L) * 2 + (size_t)rmq_stride(L) * 4;
}

// Counts each of nl lines' sources into cnt[l] (zero on entry); lists the
// positions of those of lines with at most kLinfList of them in
// lst[l][0 .. cnt[l]) (any order; fill[l] is scratch, zero on entry); and
// builds the range-minimum structures of the other lines (line l: g at gbase +
// l * gstride, words at wbase + l * wstride).  Every thread of the block calls
// it (barriers).
__device__ inline void rmq_build_lines(const uint16_t* gbase, int gstride, uint32_t* wbase, int wstride,
                                       int nl, int L, int* cnt, int* fill, uint16_t* lst) {
    const int nb = (L + kRmqBlock - 1) / kRmqBlock;
    for (int u = threadIdx.x; u < nl * nb; u += blockDim.x) {
        const int l = u / nb, b = u - l * nb;
        const uint16_t* g = gbase + (size_t)l * gstride;
        int ns = 0;
        for (int j = b * kRmqBlock; j < min(L, (b + 1) * kRmqBlock); ++j) ns += g[rmq_gi(j)] != kRmqNoG;
        if (ns) atomicAdd(&cnt[l], ns);
    }
    __syncthreads();
    for (int u = threadIdx.x; u < nl * nb; u += blockDim.x) {
        const int l = u / nb, b = u - l * nb;
        const uint16_t* g = gbase + (size_t)l * gstride;
        if (cnt[l] > kLinfList) {
            RmqLine(g, wbase + (size_t)l * wstride, L).build_block(b);
        } else {   // a sparse line: its sources' positions
            for (int j = b * kRmqBlock; j < min(L, (b + 1) * kRmqBlock); ++j)
                if (g[rmq_gi(j)] != kRmqNoG) lst[l * kLinfList + atomicAdd(&fill[l], 1)] = (uint16_t)j;
        }
    }
    __syncthreads();
    const int lev = rmq_levels(nb);
    for (int k = 1; k < lev; ++k) {
        for (int u = threadIdx.x; u < nl * nb; u += blockDim.x) {
            const int l = u / nb, i = u - l * nb;
            if (cnt[l] > kLinfList && i + (1 << k) <= nb)
                RmqLine(gbase + (size_t)l * gstride, wbase + (size_t)l * wstride, L).build_level(k, i);
        }
        __syncthreads();
    }
}

// Last axis + outputs: LPB lines of L positions per block.
template <class Geo>
__global__ __launch_bounds__(kRmqThreads) void k_linf_rmq_rows(const typename Geo::Val* __restrict__ in,
                                                               int L, int64_t nlines, int LPB, int vec,
                                                               int vec_out, Geo geo,
                                                               int32_t* __restrict__ dist,
                                                               int32_t* __restrict__ indices) {
    using Val = typename Geo::Val;
    extern __shared__ __align__(16) unsigned char smem[];
    const int gs = rmq_gstride(L), nw = rmq_stride(L);
    uint32_t* words = reinterpret_cast<uint32_t*>(smem);                                // [LPB][nw]
    uint16_t* sg = reinterpret_cast<uint16_t*>(words + (size_t)LPB * nw);              // [LPB][gs]
    unsigned* ctx = reinterpret_cast<unsigned*>(sg + (size_t)LPB * gs);                 // [LPB]
    int* cnt = reinterpret_cast<int*>(ctx + LPB);                                        // [LPB]
    int* fill = cnt + LPB;                                                               // [LPB]
    uint16_t* lst = reinterpret_cast<uint16_t*>(fill + LPB);                            // [LPB][kLinfList]
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t line0 = (int64_t)blockIdx.x * LPB;
    const int nl = (int)min<int64_t>(LPB, nlines - line0);
    for (int l = tid; l < LPB; l += nt) {
        ctx[l] = geo.ctx(line0 + (l < nl ? l : 0));
        cnt[l] = 0;
        fill[l] = 0;
    }
    __syncthreads();
    const Val* src = in + line0 * (int64_t)L;
    auto gval = [&](Val v, unsigned c) -> uint16_t {
        return Geo::valid(v) ? (uint16_t)geo.g(c, v) : kRmqNoG;
    };
    if (vec) {   // 16-byte pieces, each within one line (L * sizeof(Val) % 16 == 0)
        constexpr int VN = 16 / (int)sizeof(Val);
        const int ppl = L / VN;   // pieces per line
        for (int i = tid; i < nl * ppl; i += nt) {
            const uint4 w = reinterpret_cast<const uint4*>(src)[i];
            const int l = i / ppl, p0 = (i - l * ppl) * VN;
            const unsigned c = ctx[l];
            const Val* pv = reinterpret_cast<const Val*>(&w);
#pragma unroll
            for (int k = 0; k < VN; ++k) sg[l * gs + rmq_gi(p0 + k)] = gval(pv[k], c);
        }
    } else {
        for (int e = tid; e < nl * L; e += nt) {
            const int l = e / L;
            sg[l * gs + rmq_gi(e - l * L)] = gval(src[e], ctx[l]);
        }
    }
    __syncthreads();
    rmq_build_lines(sg, gs, words, nw, nl, L, cnt, fill, lst);
    const int nb = (L + kRmqBlock - 1) / kRmqBlock;
    for (int u = tid; u < nl * nb; u += nt) {
        const int l = u / nb, b = u - l * nb;
        const int64_t ob = (line0 + l) * (int64_t)L;
        const unsigned c = ctx[l];
        const int q0 = b * kRmqBlock, n = min(kRmqBlock, L - q0);
        const int ns = cnt[l];
        if (ns == 0) {   // no source on the line: only in an image without background
            for (int q = q0; q < q0 + n; ++q) {
                if (dist) dist[ob + q] = geo.virt(c, q);
                if (indices) indices[ob + q] = geo.virt_index();
            }
            continue;
        }
        RmqLine line(sg + l * gs, words + (size_t)l * nw, L);
        int hs[kRmqBlock], js[kRmqBlock];
        if (ns <= kLinfList) {   // few sources: the minimum over their list
#pragma unroll
            for (int t = 0; t < kRmqBlock; ++t)
                if (t < n) hs[t] = linf_list(lst + l * kLinfList, ns, q0 + t, [&](int j) { return line.g_at(j); }, js[t]);
        } else {
            line.answer_run(q0, n, line.line_min(), hs, js);
        }
        // the winners' source values are read together (for the indices),
        // and a whole run is stored in two 16-byte pieces where aligned
        if (vec_out && n == kRmqBlock) {
            if (dist) {
                *reinterpret_cast<int4*>(dist + ob + q0) = make_int4(hs[0], hs[1], hs[2], hs[3]);
                *reinterpret_cast<int4*>(dist + ob + q0 + 4) = make_int4(hs[4], hs[5], hs[6], hs[7]);
            }
            if (indices) {
                Val sv[kRmqBlock];
#pragma unroll
                for (int t = 0; t < kRmqBlock; ++t) sv[t] = src[(int64_t)l * L + js[t]];
                int32_t ix[kRmqBlock];
#pragma unroll
                for (int t = 0; t < kRmqBlock; ++t) ix[t] = geo.index(c, sv[t], js[t]);
                *reinterpret_cast<int4*>(indices + ob + q0) = make_int4(ix[0], ix[1], ix[2], ix[3]);
                *reinterpret_cast<int4*>(indices + ob + q0 + 4) = make_int4(ix[4], ix[5], ix[6], ix[7]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < kRmqBlock; ++t) {
                if (t < n) {
                    if (dist) dist[ob + q0 + t] = hs[t];
                    if (indices) indices[ob + q0 + t] = geo.index(c, src[(int64_t)l * L + js[t]], js[t]);
                }
            }
        }
    }
}

// Middle axis of B volumes: a block takes TW neighbouring columns (lines along
// axis 1) of one plane, all H rows; output the packed (axis0 << 16 | axis1)
// owner, kNone32 for a column without a source.
__global__ __launch_bounds__(kRmqThreads) void k_linf_rmq_cols(const uint16_t* __restrict__ c0,
                                                               uint32_t* __restrict__ out, int D, int H,
                                                               int W, int TW, int vec) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int gs = rmq_gstride(H), nw = rmq_stride(H);
    uint32_t* words = reinterpret_cast<uint32_t*>(smem);                                // [TW][nw]
    uint16_t* sg = reinterpret_cast<uint16_t*>(words + (size_t)TW * nw);               // [TW][gs]
    int* cnt = reinterpret_cast<int*>(sg + (size_t)TW * gs);                             // [TW]
    int* fill = cnt + TW;                                                                // [TW]
    uint16_t* lst = reinterpret_cast<uint16_t*>(fill + TW);                             // [TW][kLinfList]
    const int tid = threadIdx.x, nt = blockDim.x;
    const int tiles = (W + TW - 1) / TW;
    const int64_t plane = blockIdx.x / tiles;          // volume * D + d
    const int w0 = (int)(blockIdx.x % tiles) * TW;
    const int d = (int)(plane % D);
    const int tw = min(TW, W - w0);
    const uint16_t* src = c0 + plane * (int64_t)H * W + w0;
    uint32_t* dst = out + plane * (int64_t)H * W + w0;
    auto gval = [&](uint16_t v) -> uint16_t {
        return v != kNone16 ? (uint16_t)(d > (int)v ? d - (int)v : (int)v - d) : kRmqNoG;
    };
    for (int x = tid; x < TW; x += nt) {
        cnt[x] = 0;
        fill[x] = 0;
    }
    if (vec && tw == TW) {   // rows of the tile in 16-byte pieces of 8 columns
        const int pr = TW / 8;
        for (int i = tid; i < H * pr; i += nt) {
            const int y = i / pr, k = i - y * pr;
            const uint4 w = *reinterpret_cast<const uint4*>(src + (int64_t)y * W + 8 * k);
            const uint16_t* pv = reinterpret_cast<const uint16_t*>(&w);
            const int gy = rmq_gi(y);
#pragma unroll
            for (int c = 0; c < 8; ++c) sg[(8 * k + c) * gs + gy] = gval(pv[c]);
        }
    } else {
        for (int e = tid; e < H * TW; e += nt) {
            const int y = e / TW, x = e - y * TW;
            sg[x * gs + rmq_gi(y)] = x < tw ? gval(src[(int64_t)y * W + x]) : kRmqNoG;
        }
    }
    __syncthreads();
    rmq_build_lines(sg, gs, words, nw, TW, H, cnt, fill, lst);
    const int nb = (H + kRmqBlock - 1) / kRmqBlock;
    // neighbouring threads take neighbouring columns of one run of rows, so
    // every store of a wave covers TW consecutive elements of a row
    for (int u = tid; u < TW * nb; u += nt) {
        const int b = u / TW, x = u - b * TW;
        if (x >= tw) continue;
        const int y0 = b * kRmqBlock, n = min(kRmqBlock, H - y0);
        const int ns = cnt[x];
        if (ns == 0) {
            for (int y = y0; y < y0 + n; ++y) dst[(int64_t)y * W + x] = kNone32;
            continue;
        }
        RmqLine line(sg + x * gs, words + (size_t)x * nw, H);
        int hs[kRmqBlock], js[kRmqBlock];
        if (ns <= kLinfList) {   // few sources: the minimum over their list
#pragma unroll
            for (int t = 0; t < kRmqBlock; ++t)
                if (t < n) hs[t] = linf_list(lst + x * kLinfList, ns, y0 + t, [&](int j) { return line.g_at(j); }, js[t]);
        } else {
            line.answer_run(y0, n, line.line_min(), hs, js);
        }
        uint16_t sv[kRmqBlock];   // the winners' axis-0 coordinates, read together
#pragma unroll
        for (int t = 0; t < kRmqBlock; ++t) sv[t] = t < n ? src[(int64_t)js[t] * W + x] : 0;
#pragma unroll
        for (int t = 0; t < kRmqBlock; ++t)
            if (t < n) dst[(int64_t)(y0 + t) * W + x] = ((uint32_t)sv[t] << 16) | (uint32_t)js[t];
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

namespace {

template <class Geo>
hipError_t launch_linf_rows_t(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                              int32_t* dist, int32_t* indices, hipStream_t s, KernelTimer* tm) {
    using Val = typename Geo::Val;
    if (L <= kRmqMaxLine) {   // amortised constant work per position
        static unsigned long long rmq_done = 0;
        hipError_t le = large_lds_once((const void*)k_linf_rmq_rows<Geo>, &rmq_done);
        if (le != hipSuccess) return le;
        const size_t per = rmq_line_bytes(L);
        int LPB = (int)(kRmqLineBudget / per);
        if (LPB < 1) LPB = 1;
        const int nb = (L + kRmqBlock - 1) / kRmqBlock;
        if (LPB * nb > 4 * kRmqThreads) LPB = (4 * kRmqThreads) / nb > 0 ? (4 * kRmqThreads) / nb : 1;
        const size_t lds = (size_t)LPB * per + (size_t)LPB * (12 + 2 * kLinfList);
        const int64_t blocks = (nlines + LPB - 1) / LPB;
        if (blocks > INT32_MAX || lds > 160 * 1024) return hipErrorInvalidValue;
        const int vec = ((size_t)L * sizeof(Val) % 16 == 0 && ((uintptr_t)in & 15) == 0) ? 1 : 0;
        // runs start at multiples of 8 positions: 16-byte stores when rows
        // are whole 16-byte pieces and the outputs 16-byte aligned
        const int vec_out = (L % 4 == 0 && ((((uintptr_t)dist) | ((uintptr_t)indices)) & 15) == 0) ? 1 : 0;
        EDT_LAUNCH(tm, "chessboard_rows", s,
                   hipLaunchKernelGGL((k_linf_rmq_rows<Geo>), dim3((unsigned)blocks), dim3(kRmqThreads), lds,
                                      s, in, L, nlines, LPB, vec, vec_out, geo, dist, indices));
        return hipSuccess;
    }
    static unsigned long long lds_done[2] = {0, 0};
    hipError_t le = large_lds_once((const void*)k_linf_rows<Geo, false>, &lds_done[0]);
    if (le == hipSuccess) le = large_lds_once((const void*)k_linf_rows<Geo, true>, &lds_done[1]);
    if (le != hipSuccess) return le;
    const int LPB = L <= kLinfStage ? kLinfStage / L : 1;
    const int nbk = (L + kLinfBT - 1) / kLinfBT;
    const size_t lds = linf_flags_offset((size_t)LPB * L * 2) + (size_t)LPB * 16 +
                       (L >= kLinfBLine ? (size_t)LPB * nbk * (4 + 2 * kLinfBC) : 0) +
                       (LPB <= kLinfList ? (size_t)LPB * kLinfList * 2 : 0);
    const int64_t blocks = (nlines + LPB - 1) / LPB;
    if (blocks > INT32_MAX || lds > 160 * 1024) return hipErrorInvalidValue;
    const int vec = ((size_t)L * sizeof(Val) % 16 == 0 && ((uintptr_t)in & 15) == 0) ? 1 : 0;
    if (L >= kLinfBLine) {
        EDT_LAUNCH(tm, "chessboard_rows", s,
                   hipLaunchKernelGGL((k_linf_rows<Geo, true>), dim3((unsigned)blocks), dim3(kLinfThreads), lds,
                                      s, in, L, nlines, LPB, vec, geo, dist, indices));
    } else {
        EDT_LAUNCH(tm, "chessboard_rows", s,
                   hipLaunchKernelGGL((k_linf_rows<Geo, false>), dim3((unsigned)blocks), dim3(kLinfThreads), lds,
                                      s, in, L, nlines, LPB, vec, geo, dist, indices));
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_linf_rows_2d(const uint16_t* c0, int B, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm) {
    return launch_linf_rows_t(c0, W, (int64_t)B * H, LinfRows2D{H, W}, dist, indices, s, tm);
}

hipError_t launch_linf_cols_3d(const uint16_t* c0, int B, int D, int H, int W, uint32_t* c01,
                               hipStream_t s, KernelTimer* tm) {
    if (H <= kRmqMaxLine) {   // amortised constant work per position
        static unsigned long long rmq_done = 0;
        hipError_t le = large_lds_once((const void*)k_linf_rmq_cols, &rmq_done);
        if (le != hipSuccess) return le;
        const size_t per = rmq_line_bytes(H);
        int TW = 8;   // columns per block: one 16-byte piece of every row
        while (TW > 1 && (size_t)TW * per > kRmqLineBudget) TW >>= 1;
        const size_t lds = (size_t)TW * per + (size_t)TW * (8 + 2 * kLinfList);
        const int64_t blocks = (int64_t)B * D * ((W + TW - 1) / TW);
        if (blocks > INT32_MAX || lds > 160 * 1024) return hipErrorInvalidValue;
        const int vec = (W % 8 == 0 && TW % 8 == 0 && ((uintptr_t)c0 & 15) == 0) ? 1 : 0;
        EDT_LAUNCH(tm, "chessboard_cols", s,
                   hipLaunchKernelGGL(k_linf_rmq_cols, dim3((unsigned)blocks), dim3(kRmqThreads), lds, s, c0,
                                      c01, D, H, W, TW, vec));
        return hipSuccess;
    }
    static unsigned long long lds_done = 0;
    hipError_t le = large_lds_once((const void*)k_linf_cols, &lds_done);
    if (le != hipSuccess) return le;
    int TW = 32;   // columns per block: their H rows of 2-byte values within 32 KB (64 KB
                   // for one column of the longest lines), several blocks per CU
    while (TW > 1 && (size_t)H * TW * 2 > 32 * 1024) TW >>= 1;
    if ((size_t)H * TW * 2 > 64 * 1024) return hipErrorInvalidValue;
    const size_t lds = linf_flags_offset((size_t)H * TW * 2) + (size_t)TW * (8 + 2 * kLinfList);
    const int64_t blocks = (int64_t)B * D * ((W + TW - 1) / TW);
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    // 16-byte pieces: rows 16-byte aligned and tiles of whole pieces
    const int vec = (W % 8 == 0 && TW % 8 == 0 && ((uintptr_t)c0 & 15) == 0) ? 1 : 0;
    EDT_LAUNCH(tm, "chessboard_cols", s,
               hipLaunchKernelGGL(k_linf_cols, dim3((unsigned)blocks), dim3(kLinfThreads), lds, s, c0, c01, D, H,
                                  W, TW, vec));
    return hipSuccess;
}

hipError_t launch_linf_rows_3d(const uint32_t* c01, int B, int D, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm) {
    return launch_linf_rows_t(c01, W, (int64_t)B * D * H, LinfRows3D{D, H, W}, dist, indices, s, tm);
}

}  // namespace edt
