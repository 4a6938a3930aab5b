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
#include <cmath>
#include <algorithm>
#include <type_traits>

#include "envelope.h"
#include "kernels.h"

namespace edt {

// --------------------------------------------------------------------------
// helpers
// --------------------------------------------------------------------------

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

hipError_t large_lds_once(const void* fn, unsigned long long* done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
    if (bit && (__atomic_load_n(done, __ATOMIC_ACQUIRE) & bit)) return hipSuccess;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
        (void)hipGetLastError();
    if (bit) __atomic_fetch_or(done, bit, __ATOMIC_RELEASE);
    return hipSuccess;
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


// --------------------------------------------------------------------------
// Pass 0: nearest background along axis 0, in three kernels over segments of
// kSegRows rows (so that long, few lines still fill the machine):
//   summary  per (segment, column), the 64-bit mask of background rows and the
//            first/last of them;
//   scan     per column, nearest background strictly above / below each segment
//            (not needed, and not launched, when a line is a single segment);
//   resolve  per (segment, column), the nearest background of every row from
//            the segment's mask plus the two carries (the mask bytes are read
//            once, by the summary).
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

// Bit 7 of each byte of the result is set where that byte of w is zero.
__device__ __forceinline__ uint32_t zero_bytes(uint32_t w) {
    return ~(((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
}

template <int VEC>
__global__ __launch_bounds__(256) void k_axis0_summary(const uint8_t* __restrict__ mask, int n0,
                                                        int64_t M, int nseg,
                                                        uint16_t* __restrict__ first,
                                                        uint16_t* __restrict__ last,
                                                        uint64_t* __restrict__ bits) {
    const int64_t col = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    if (col >= M) return;
    const int i0 = s * kSegRows;
    const int i1 = min(n0, i0 + kSegRows);
    const uint8_t* src = mask + (int64_t)b * n0 * M + col;
    uint64_t bm[VEC];   // bit r: row i0 + r is background
#pragma unroll
    for (int v = 0; v < VEC; ++v) bm[v] = 0;
    if (VEC == 4 && i1 - i0 == kSegRows) {
        // A full segment, one 32-bit word (4 columns) per row: byte v of t
        // collects the zero flags of column v over 8 rows, which then fill
        // bits 8k .. 8k + 7 of that column's mask.
        const uint8_t* rp = src + (int64_t)i0 * M;
#pragma unroll
        for (int k = 0; k < kSegRows / 8; ++k) {
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)   // read once: keep it out of the caches
                w[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(rp + (int64_t)(8 * k + j) * M));
            uint32_t t = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) t |= (zero_bytes(w[j]) >> 7) << j;
#pragma unroll
            for (int v = 0; v < VEC; ++v) bm[v] |= (uint64_t)((t >> (8 * v)) & 0xFFu) << (8 * k);
        }
    } else {
#pragma unroll 4
        for (int i = i0; i < i1; ++i) {
            uint8_t x[VEC];
            load_bytes<VEC>(src + (int64_t)i * M, x);
#pragma unroll
            for (int v = 0; v < VEC; ++v) bm[v] |= (uint64_t)(x[v] == 0) << (i - i0);
        }
    }
    uint16_t f[VEC], l[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        f[v] = bm[v] ? (uint16_t)(i0 + __builtin_ctzll(bm[v])) : kNone16;
        l[v] = bm[v] ? (uint16_t)(i0 + 63 - __builtin_clzll(bm[v])) : kNone16;
    }
    const int64_t o = ((int64_t)b * nseg + s) * M + col;
    store_u16<VEC>(first + o, f);
    store_u16<VEC>(last + o, l);
#pragma unroll
    for (int v = 0; v < VEC; ++v) bits[o + v] = bm[v];
}

// After this kernel last[b][s][m] holds the nearest background row above
// segment s (kNone16 if none) and first[b][s][m] the nearest one below it.
// Q segment groups per column (threads along y): 16 for long columns; few
// segments are walked by fewer threads (one, for at most 8 segments).
template <int kScanQ>
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

// Row at which the answer switches from the background row above (p, < 0:
// none) to the one below (n, >= kFarRow: none): rows i with i - p <= n - i
// keep p (the smaller coordinate wins a tie).
constexpr int kFarRow = 1 << 20;
__device__ __forceinline__ int switch_row(int p, int n) {
    if (p < 0) return INT_MIN;
    if (n >= kFarRow) return INT_MAX;
    return ((p + n) >> 1) + 1;
}

template <int VEC>
__global__ __launch_bounds__(256) void k_axis0_resolve(const uint64_t* __restrict__ bits, int n0,
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
    const int64_t so = ((int64_t)b * nseg + s) * M + col;
    uint64_t bm[VEC];   // the segment's background rows, from the summary
#pragma unroll
    for (int v = 0; v < VEC; ++v) bm[v] = bits[so + v];
    uint16_t upc[VEC], dnc[VEC];
    if (nseg > 1) {
        load_u16<VEC>(up_carry + so, upc);
        load_u16<VEC>(dn_carry + so, dnc);
    } else {   // one segment: nothing above or below it (no scan ran)
#pragma unroll
        for (int v = 0; v < VEC; ++v) upc[v] = dnc[v] = kNone16;
    }

    // Per column: the background rows just above (prev) and at or below (next)
    // the current row, and the row where the answer switches from one to the
    // other; they change only when the row reaches next.
    int prev[VEC], next[VEC], sw[VEC];
    uint16_t pv[VEC], nv[VEC];   // prev / next as stored (kNone16: none)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        prev[v] = upc[v] == kNone16 ? -1 : (int)upc[v];
        next[v] = bm[v] ? i0 + __builtin_ctzll(bm[v]) : (dnc[v] == kNone16 ? kFarRow : (int)dnc[v]);
        sw[v] = switch_row(prev[v], next[v]);
        pv[v] = upc[v];
        nv[v] = next[v] >= kFarRow ? kNone16 : (uint16_t)next[v];
    }
    uint16_t* dst = c0 + (int64_t)b * n0 * M + col;
    for (int i = i0; i < i1; ++i) {
        bool ev = false;
#pragma unroll
        for (int v = 0; v < VEC; ++v) ev |= (i == next[v]);
        if (ev) {   // a background row: it becomes prev, the following one next
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                if (i == next[v]) {
                    const int r1 = i - i0 + 1;
                    const uint64_t rest = r1 < 64 ? bm[v] >> r1 : 0;
                    prev[v] = i;
                    next[v] = rest ? i + 1 + __builtin_ctzll(rest)
                                   : (dnc[v] == kNone16 ? kFarRow : (int)dnc[v]);
                    sw[v] = switch_row(prev[v], next[v]);
                    pv[v] = (uint16_t)i;
                    nv[v] = next[v] >= kFarRow ? kNone16 : (uint16_t)next[v];
                }
            }
        }
        uint16_t out[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) out[v] = i >= sw[v] ? nv[v] : pv[v];
        store_u16<VEC>(dst + (int64_t)i * M, out);
    }
}

hipError_t launch_axis0(const uint8_t* mask, int B, int n0, int64_t M, uint16_t* first,
                        uint16_t* last, uint64_t* bits, uint16_t* c0, hipStream_t s, KernelTimer* tm) {
    const int nseg = (n0 + kSegRows - 1) / kSegRows;
    int vec = 1;
    if (M % 16 == 0 && ((uintptr_t)mask & 15) == 0) vec = 16;
    else if (M % 4 == 0 && ((uintptr_t)mask & 3) == 0) vec = 4;
    dim3 block(256);
    auto grid_for = [&](int v) {
        const int64_t lanes = M / v + (M % v ? 1 : 0);
        return dim3((unsigned)((lanes + 255) / 256), (unsigned)nseg, (unsigned)B);
    };
    // the summary reads one 32-bit word per lane and row: more lanes in flight
    // than 16-byte reads give for the same bytes
    if (vec >= 4) {
        EDT_LAUNCH(tm, "axis0_summary", s, hipLaunchKernelGGL(k_axis0_summary<4>, grid_for(4), block, 0, s, mask, n0, M, nseg, first, last, bits));
    } else {
        EDT_LAUNCH(tm, "axis0_summary", s, hipLaunchKernelGGL(k_axis0_summary<1>, grid_for(1), block, 0, s, mask, n0, M, nseg, first, last, bits));
    }
    if (nseg > 1) {   // carries between segments (a single segment has none)
        dim3 sgrid((unsigned)((M + 63) / 64), (unsigned)B);
        if (nseg <= 8) {
            EDT_LAUNCH(tm, "axis0_scan", s, hipLaunchKernelGGL(k_axis0_scan<1>, sgrid, dim3(64, 1), 0, s, first, last, nseg, M));
        } else if (nseg <= 32) {
            EDT_LAUNCH(tm, "axis0_scan", s, hipLaunchKernelGGL(k_axis0_scan<4>, sgrid, dim3(64, 4), 0, s, first, last, nseg, M));
        } else {
            EDT_LAUNCH(tm, "axis0_scan", s, hipLaunchKernelGGL(k_axis0_scan<16>, sgrid, dim3(64, 16), 0, s, first, last, nseg, M));
        }
    }
    if (!c0) return hipSuccess;   // the summaries alone were asked for
    // the resolve keeps per-column state in registers: 4 columns per lane
    if (vec >= 4) {
        EDT_LAUNCH(tm, "axis0_resolve", s, hipLaunchKernelGGL(k_axis0_resolve<4>, grid_for(4), block, 0, s, bits, n0, M, nseg, last, first, c0));
    } else {
        EDT_LAUNCH(tm, "axis0_resolve", s, hipLaunchKernelGGL(k_axis0_resolve<1>, grid_for(1), block, 0, s, bits, n0, M, nseg, last, first, c0));
    }
    return hipSuccess;
}

// --------------------------------------------------------------------------
// Envelope passes.
//
// Every lane owns one chunk of K consecutive positions of one line.  Chunk
// values sit in LDS at slot * CS + t (t < K), slot being the lane's thread
// index; CS = K + pad makes the 32-bit word stride between slots odd, so when
// every lane reads position t of its own chunk the reads fall in distinct
// banks.  The owner marks use the same slot layout with 16-bit entries.  Per
// slot there are also the member mask, a 32-bit word (chunk minimum, then
// chunk-level owner marks) and two 16-bit scan words (last member + 1, first
// member).
//
// Phases of one line (all lanes of the line together):
//   1. chunk minima of F and the line's candidate bound U (see chunk_bound),
//      then the candidates that a pair of chunk minimisers dominates are
//      dropped (on each side the minimiser best at the chunk's nearer end);
//   2. local envelope of every chunk's remaining candidates;
//   3. each lane resolves its chunk alone from its own envelope and the few
//      members of other chunks that reach into it (chunk_owner_marks), writing
//      owner + 1 where each owned interval starts; if a chunk has more reaching
//      members than fit (or the layout skips this step), the block instead
//      takes the envelope of whole lines in rounds (boundary_dead), every
//      member marking the start of its interval, then a chunk-level scan;
//   4. each lane scans its chunk: the owner of position q is the latest mark at
//      or before q, so the outputs follow without any per-position search.
// --------------------------------------------------------------------------

template <class Val, int K>
struct Slots {
    static constexpr int CS = sizeof(Val) == 2 ? K + 2 : K + 1;   // value stride
    static constexpr int CM = K + 2;                               // mark stride (16-bit)
    using Mask = typename MaskOf<K>::T;
    // Occupancy words: ceil(Gp / 64) per line of Gp chunks.
    __host__ __device__ static int occ_words(int nslots, int Gp) { return (nslots / Gp) * ((Gp + 63) / 64); }
    // The per-line bound words share the storage of the two 16-bit scan arrays,
    // which are not live until later (lines per block <= slots).
    static size_t bytes(int nslots, int Gp) {
        return align16((size_t)nslots * CS * sizeof(Val)) + align16((size_t)nslots * CM * 2) +
               align16((size_t)nslots * sizeof(Mask)) + align16((size_t)nslots * 4) +
               2 * align16((size_t)nslots * 2) + align16((size_t)occ_words(nslots, Gp) * 8) + 16;
    }
};

constexpr uint16_t kNoFirst = 0xFFFFu;   // "no member" in the first-member scan
constexpr int kReach = 8;                // reaching members kept per chunk side
constexpr int kSparseCand = 12;          // above: a wave tests every position of its chunks
constexpr int kWitnessScan = 16;         // chunks scanned per side for the filter's witnesses
constexpr int kWitnessScanLinf = 32;     // the same under the chessboard metric (see resolve_line)
constexpr int kCascadeFrom = 2;          // first whole-line round with cascade steps

// LDS carve-up shared by both layouts.
template <class Val, int K>
struct SlotArrays {
    using Mask = typename MaskOf<K>::T;
    Val* val;
    uint16_t* mark;   // per position: owner + 1 of the interval starting there, else 0
    Mask* mask;
    int* own;         // chunk minimum of F (float32 bits), then chunk-level owner marks
    uint16_t* last;   // last member + 1 (0: none), then prefix maximum
    uint16_t* first;  // first member (kNoFirst: none), then suffix minimum
    unsigned* bound;  // per line: the candidate bound U (float32 bits); shares
                      // the storage of last/first, used before they are written
    uint64_t* occ;    // per line: bit c set while chunk c has a member
    unsigned* flag;   // per block: [0] some chunk needs whole lines; [1], [2]: a round of
                      // the whole-line envelope removed a member (alternating)
    __device__ SlotArrays(unsigned char* smem, int nslots, int Gp) {
        size_t off = 0;
        val = reinterpret_cast<Val*>(smem);
        off += align16((size_t)nslots * Slots<Val, K>::CS * sizeof(Val));
        mark = reinterpret_cast<uint16_t*>(smem + off);
        off += align16((size_t)nslots * Slots<Val, K>::CM * 2);
        mask = reinterpret_cast<Mask*>(smem + off);
        off += align16((size_t)nslots * sizeof(Mask));
        own = reinterpret_cast<int*>(smem + off);
        off += align16((size_t)nslots * 4);
        last = reinterpret_cast<uint16_t*>(smem + off);
        off += align16((size_t)nslots * 2);
        first = reinterpret_cast<uint16_t*>(smem + off);
        off += align16((size_t)nslots * 2);
        bound = reinterpret_cast<unsigned*>(last);
        occ = reinterpret_cast<uint64_t*>(smem + off);
        off += align16((size_t)Slots<Val, K>::occ_words(nslots, Gp) * 8);
        flag = reinterpret_cast<unsigned*>(smem + off);
    }
};

// One line as seen by the envelope helpers: chunk c of the line lives in slot
// slot0 + c * gs; occ points at the line's occupancy words; mt is the metric
// (L2Metric or LinfMetric), fof maps a stored value to the candidate's value.
// (LDS offsets are products of small slot indices and strides: 24-bit
// multiplies suffice.)
template <class Val, int K, class FOf, int GS, class Mt = L2Metric>
struct LineView {
    using Mask = typename MaskOf<K>::T;
    using Metric = Mt;
    using F = typename Mt::Val;
    static constexpr int CS = Slots<Val, K>::CS;
    const Val* vals;
    Mask* masks;
    uint64_t* occ;
    const int* own;   // chunk minima in the metric's 32-bit form
    int slot0;
    static constexpr int gs = GS;   // slot step between neighbouring chunks
    Mt mt;
    FOf fof;
    // a lower bound of the values of chunk c
    __device__ F fmin_lb(int c) const { return Mt::lower_from_bits((uint32_t)own[slot(c)]); }
    __device__ int last_nonempty(int lo, int hi) const {
        return occ_last([&](int w) { return occ[w]; }, lo, hi);
    }
    __device__ int first_nonempty(int lo, int hi) const {
        return occ_first([&](int w) { return occ[w]; }, lo, hi);
    }
    __device__ void mark_empty(int c) { atomicAnd(&occ[c >> 6], ~(uint64_t(1) << (c & 63))); }
    __device__ int slot(int c) const { return slot0 + c * gs; }
    __device__ Val val(int pos) const {
        return vals[__umul24((unsigned)slot((unsigned)pos / K), CS) + ((unsigned)pos % K)];
    }
    __device__ F f(int pos) const { return fof(val(pos)); }
    __device__ F Y(int pos) const { return mt.height(f(pos), pos); }
    __device__ Mask mask(int c) const { return masks[slot(c)]; }
    __device__ void set_mask(int c, Mask m) { masks[slot(c)] = m; }
};

// Inclusive scans over the Gp chunks of every line (slot step GS), in LDS:
// prefix maximum of a[], and (when b is non-null) suffix minimum of b[].
// Chunk g of a line sits GS lanes after chunk g - 1, so the S = min(Gp, 64/GS)
// chunks of a line that share a wave scan with lane shuffles; lines longer
// than one wave then add the totals of their earlier (later) waves.  Every
// thread of the block calls it; it starts and ends with a barrier.
template <int GS, class T>
__device__ void line_scans(T* a, uint16_t* b, int myslot, int g, int Gp) {
    constexpr int kLanes = 64 / GS > 0 ? 64 / GS : 1;   // chunks of a line per wave
    const int S = Gp < kLanes ? Gp : kLanes;
    const int pos = g & (S - 1);
    __syncthreads();
    int x = (int)a[myslot];
    int y = b ? (int)b[myslot] : 0;
    for (int d = 1; d < S; d <<= 1) {
        const int xu = __shfl_up(x, d * GS);
        if (pos >= d && xu > x) x = xu;
        if (b) {
            const int yd = __shfl_down(y, d * GS);
            if (pos + d < S && yd < y) y = yd;
        }
    }
    if (S < Gp) {
        a[myslot] = (T)x;
        if (b) b[myslot] = (uint16_t)y;
        __syncthreads();
        // totals of the other waves of the line: the last (first) chunk of each
        const int w0 = g - pos;   // first chunk of this wave
        for (int c = w0 - 1; c >= 0; c -= S) {
            const int v = (int)a[myslot - (g - c) * GS];
            if (v > x) x = v;
        }
        if (b) {
            for (int c = w0 + S; c < Gp; c += S) {
                const int v = (int)b[myslot + (c - g) * GS];
                if (v < y) y = v;
            }
        }
        __syncthreads();
    }
    a[myslot] = (T)x;
    if (b) b[myslot] = (uint16_t)y;
    __syncthreads();
}

// Phases 1-4 for the lane's chunk g of its line (local line index lslot).
// Fills the owner marks of the lane's chunk: the owner of a position is the
// largest mark at or before it within the chunk.  Every thread of the block
// must call it (it contains barriers).  PerChunk: try phase 3's per-chunk
// resolution first (otherwise whole lines in rounds straight away).
template <int K, bool PerChunk, class Val, class View, class IsValid, class FOfVal>
__device__ void resolve_line(View& view, SlotArrays<Val, K>& sa, const Val* mychunk,
                            uint16_t* mymarks, int g, int Gp, int L, bool active, int myslot,
                            int lslot, IsValid valid, FOfVal fval) {
    constexpr int gs = View::gs;
    using Mask = typename MaskOf<K>::T;
    constexpr int CM = Slots<Val, K>::CM;
    const int base = g * K;
    const int n = active ? min(K, L - base) : 0;
    const int G = (L + K - 1) / K;
    using Mt = typename View::Metric;
    using F = typename Mt::Val;
    const Mt& mt = view.mt;

    // 1. chunk minimum of F and its first minimiser, then the line's
    //    candidate bound.  The minimiser (+1, 0: none) is published in the mask
    //    slot, which the local envelope overwrites only after the second barrier.
    //    F of the chunk's positions stays in registers for the candidate pass
    //    when the chunk is short enough (+inf: no candidate there).
    constexpr bool kKeepF = K <= 32;
    F Fr[kKeepF ? K : 1];
    F fmin = Mt::kInf;
    int amin = -1;
    bool allzero = true;   // every position is background itself (F = 0)
    if constexpr (kKeepF) {
#pragma unroll
        for (int t = 0; t < K; ++t) {
            const Val v = mychunk[t];   // positions past the line hold "no background"
            const bool here = valid(v);
            Fr[t] = here ? fval(v) : F(Mt::kInf);
            if (Fr[t] != F(0)) allzero = false;
            if (Fr[t] < fmin) { fmin = Fr[t]; amin = t; }
        }
    } else {
#pragma unroll 8
        for (int t = 0; t < n; ++t) {
            const Val v = mychunk[t];
            const F f = fval(v);
            if (!valid(v) || f != F(0)) allzero = false;
            if (valid(v) && f < fmin) { fmin = f; amin = t; }
        }
    }
    // A chunk of background positions owns itself: F_q = 0 there, and any other
    // candidate j is s^2 (q - j)^2 > 0 away.
    const bool selfowned = n > 0 && allzero;
    const uint32_t fmin_bits = Mt::min_bits(fmin);
    sa.own[myslot] = (int)fmin_bits;
    sa.mask[myslot] = (Mask)(amin < 0 ? 0 : base + amin + 1);
    if (g == 0) sa.bound[lslot] = 0u;
    if ((g & 63) == 0) view.occ[g >> 6] = 0ull;
    if (myslot == 0) { sa.flag[0] = 0u; sa.flag[1] = 0u; }
    __syncthreads();
    // Witnesses for the filter of step 2: on each side, the chunk minimiser
    // with the smallest value at the chunk's nearer end, found by scanning
    // chunk minima outward until the distance term alone is no better, over
    // at most kWitnessScan chunks (lines far from their background -- large
    // objects -- have their useful witnesses many chunks away, often past
    // chunks without candidates).  Only on the whole-line route: the per-chunk
    // route looks past neighbouring chunks by itself (chunk_owner_marks), and
    // there the nearest chunk minimisers serve as witnesses.
    // The chessboard's distance term grows linearly, so its scans stop later
    // and its witnesses sit further out: 4096^2 disks 0.313 -> 0.275 ms with
    // 32 chunks instead of 16 (8: 0.39 ms).  The Euclidean transform keeps 16
    // (one background pixel in 4096^2: 0.050 ms with 8, 0.056 with 16, 0.067
    // with 32; disks 0.192, 0.189, 0.192 ms).
    constexpr int kScan = (PerChunk && 2 * kReach + K <= 64)
                              ? 1
                              : std::is_same<Mt, LinfMetric>::value ? kWitnessScanLinf : kWitnessScan;
    int aprev = -1, anext = -1;
    if (n > 0) {
        const F prev = g > 0 ? Mt::from_bits((uint32_t)sa.own[myslot - gs]) : F(Mt::kInf);
        const F next = g + 1 < G ? Mt::from_bits((uint32_t)sa.own[myslot + gs]) : F(Mt::kInf);
        atomicMax(&sa.bound[lslot], mt.bound_bits(Mt::from_bits(fmin_bits), prev, next, K));
        F best = F(Mt::kInf);
        for (int c2 = g - 1, sl = myslot - gs; c2 >= 0 && c2 >= g - kScan; --c2, sl -= gs) {
            if (!(mt.dist(base - (c2 * K + K - 1)) < best)) break;
            const int k = (int)sa.mask[sl] - 1;
            if (k < 0) continue;
            const F v = mt.combine(Mt::from_bits((uint32_t)sa.own[sl]), mt.dist(base - k));
            if (v < best) { best = v; aprev = k; }
        }
        best = F(Mt::kInf);
        const int e = base + n - 1;
        for (int c2 = g + 1, sl = myslot + gs; c2 < G && c2 <= g + kScan; ++c2, sl += gs) {
            if (!(mt.dist(c2 * K - e) < best)) break;
            const int k = (int)sa.mask[sl] - 1;
            if (k < 0) continue;
            const F v = mt.combine(Mt::from_bits((uint32_t)sa.own[sl]), mt.dist(k - e));
            if (v < best) { best = v; anext = k; }
        }
    }
    __syncthreads();
    const F U = Mt::from_bits(sa.bound[lslot]);

    // 2. local envelope of the chunk's candidates that can still own a
    //    position: F <= U, and not dominated by a chunk minimiser on either
    //    side (the chunk's own where it lies on that side, else the witness;
    //    a candidate that two others dominate never attains the minimum, and
    //    a witness that attains it somewhere passes F <= U there).
    const int acur = amin < 0 ? -1 : base + amin;
    const F Yprev = aprev >= 0 ? view.Y(aprev) : F(0);
    const F Ycur = acur >= 0 ? view.Y(acur) : F(0);
    const F Ynext = anext >= 0 ? view.Y(anext) : F(0);
    Mask m;
    if (selfowned) {
        m = n >= (int)(8 * sizeof(Mask)) ? ~Mask(0) : (Mask(1) << n) - Mask(1);   // positions 0 .. n-1
    } else {
        Mask cand = 0;
        // (U may be +inf when a chunk and both its neighbours hold no candidate)
        auto consider = [&](int t, F Yp, bool here) {
            const int p = base + t;
            const int lo = acur >= 0 && acur < p ? acur : aprev;
            const F Ylo = acur >= 0 && acur < p ? Ycur : Yprev;
            const int hi = acur > p ? acur : anext;
            const F Yhi = acur > p ? Ycur : Ynext;
            // (no short-circuit: the test is cheap, and a branch here keeps one
            // lane mask per position alive until the loop ends)
            const bool gone = (lo >= 0) & (hi >= 0) & mt.dominated(lo, Ylo, p, Yp, hi, Yhi);
            cand |= (Mask)(here & !gone) << t;
        };
        auto height = [&](Val v, int p) { return mt.height(fval(v), p); };
        if constexpr (kKeepF) {
            // Most positions of a line far from the background fail F <= U, so
            // the dominance test runs only on those that pass -- one at a time
            // unless some lane of the wave has many of them; then every
            // position's height comes from the registers of phase 1.
            // (F is the metric's kInf exactly where a position has no
            // background; U itself may be kInf, so the test runs against the
            // largest finite value)
            // The chessboard's per-chunk route always takes the one-at-a-time
            // form (512^3 transform 1.25 -> 1.21 ms; on its whole-line routes
            // the switch stays: 16 x 128^3 0.45 -> 0.47 ms without it).
            constexpr bool kOneAtATime = std::is_same<Mt, LinfMetric>::value && PerChunk && 2 * kReach + K <= 64;
            const F Ufin = U < Mt::kMaxFinite ? U : F(Mt::kMaxFinite);
            Mask pass = 0;
#pragma unroll
            for (int t = 0; t < K; ++t)
                if (Fr[t] <= Ufin) pass |= Mask(1) << t;
            if (!kOneAtATime && __any(__builtin_popcount(pass) > kSparseCand)) {
#pragma unroll
                for (int t = 0; t < K; ++t) {
                    Fr[t] = mt.height(Fr[t], base + t);   // now Y
                    consider(t, Fr[t], (pass >> t) & 1);
                }
                if constexpr (K <= 16)   // (for longer chunks the registers run out)
                    m = build_chunk_unrolled<K>(mt, base, cand, Fr, [&](int p) { return view.Y(p); });
                else
                    m = build_chunk<Mask>(mt, base, cand, [&](int t) { return mychunk[t]; }, height);
            } else {
                for (Mask rest = pass; rest; rest &= rest - 1) {
                    const int t = low_bit(rest);
                    consider(t, height(mychunk[t], base + t), true);
                }
                m = build_chunk<Mask>(mt, base, cand, [&](int t) { return mychunk[t]; }, height);
            }
        } else {
#pragma unroll 8
            for (int t = 0; t < n; ++t) {
                const Val v = mychunk[t];
                const F f = fval(v);
                consider(t, height(v, base + t), valid(v) && f <= U);
            }
            m = build_chunk<Mask>(mt, base, cand, [&](int t) { return mychunk[t]; }, height);
        }
    }
    sa.mask[myslot] = m;
    if (m) atomicOr(&view.occ[g >> 6], uint64_t(1) << (g & 63));

    __syncthreads();

    // 3. owners of the chunk from its own envelope and the members of other
    //    chunks that reach into it (chunk_owner_marks); only if some chunk of
    //    the block has more reaching members than the lists hold does the
    //    block take whole lines instead
    if constexpr (PerChunk && 2 * kReach + K <= 64) {
#pragma unroll
        for (int t = 0; t < K; t += 2) *reinterpret_cast<uint32_t*>(mymarks + t) = 0u;
        bool ok = true;
        if (selfowned) {
            for (int t = 0; t < n; ++t) mymarks[t] = (uint16_t)(base + t + 1);
        } else if (n > 0) {
            ok = chunk_owner_marks<K, kReach>(view, g, G, L, m,
                                              [&](int t, int o) { mymarks[t] = (uint16_t)(o + 1); });
        }
        if (!ok) atomicOr(sa.flag, 1u);
        __syncthreads();
        if (*sa.flag == 0u) return;
    }

    // 4. whole lines: the envelope from the chunk envelopes in rounds
    //    (boundary_dead: every chunk's first and last members tested against
    //    the nearest members around them, dominated ones removed together,
    //    until a round removes nothing), then marks from every member.
    //    From round kCascadeFrom on, a round that removed something goes on
    //    with a back and a front cascade step (back_cascade, front_cascade),
    //    which empty a chunk down to one member at once where only a far
    //    neighbour dominates its interior members (large objects); a round
    //    whose boundary step removes nothing leaves nothing to cascade.
    //    flag[1] was cleared with flag[0]; each round clears the other one.
    for (int r = 0;; ++r) {
        m = sa.mask[myslot];
        const Mask dead = active ? boundary_dead<K>(view, g, G, m) : Mask(0);
        __syncthreads();
        if (myslot == 0) sa.flag[1 + ((r + 1) & 1)] = 0u;   // the last round's flag, read by all
        if (dead) {
            m &= ~dead;
            sa.mask[myslot] = m;
            if (!m) view.mark_empty(g);
            atomicOr(&sa.flag[1 + (r & 1)], 1u);
        }
        __syncthreads();
        if (sa.flag[1 + (r & 1)] == 0u) break;
        if (r >= kCascadeFrom) {
            if (m & (m - 1)) {   // (inactive lanes hold no members)
                const int cn = view.first_nonempty(g + 1, G);
                if (cn >= 0) {
                    const Mask m2 = back_cascade<K>(view, g, m, cn * K + low_bit(view.mask(cn)));
                    if (m2 != m) {
                        m = m2;
                        sa.mask[myslot] = m;
                    }
                }
            }
            __syncthreads();
            if (m & (m - 1)) {
                const int cp = view.last_nonempty(0, g);
                if (cp >= 0) {
                    const Mask m2 = front_cascade<K>(view, g, m, cp * K + high_bit(view.mask(cp)));
                    if (m2 != m) {
                        m = m2;
                        sa.mask[myslot] = m;
                    }
                }
            }
            __syncthreads();
        }
    }

    // last member up to each chunk, first member from each chunk on; clear marks
    m = sa.mask[myslot];
    sa.last[myslot] = m ? (uint16_t)(base + high_bit(m) + 1) : (uint16_t)0;
    sa.first[myslot] = m ? (uint16_t)(base + low_bit(m)) : kNoFirst;
    sa.own[myslot] = 0;
#pragma unroll
    for (int t = 0; t < K; t += 2) *reinterpret_cast<uint32_t*>(mymarks + t) = 0u;
    line_scans<gs>(sa.last, sa.first, myslot, g, Gp);

    // owned intervals of the members: v owns [st, en), st against its
    // predecessor u, en where its successor w takes over
    if (m) {
        Mask mm = m;
        const int u = g > 0 ? (int)sa.last[myslot - gs] - 1 : -1;
        int v = base + low_bit(mm);
        mm &= mm - 1;
        F Yv = view.Y(v);
        int st = 0;
        if (u >= 0) st = mt.cross(u, view.Y(u), v, Yv, L);
        for (;;) {
            int w;
            if (mm) {
                w = base + low_bit(mm);
            } else {
                const uint16_t nf = g + 1 < Gp ? sa.first[myslot + gs] : kNoFirst;
                w = nf == kNoFirst ? -1 : (int)nf;
            }
            int en = L;
            F Yw = F(0);
            if (w >= 0) {
                Yw = view.Y(w);
                en = mt.cross(v, Yv, w, Yw, L);
            }
            if (st < en) {   // st < L follows from en <= L
                const int cs = (unsigned)st / K;
                sa.mark[__umul24((unsigned)view.slot(cs), CM) + ((unsigned)st % K)] = (uint16_t)(v + 1);
                atomicMax(&sa.own[view.slot(cs)], v + 1);
            }
            if (!mm) break;
            mm &= mm - 1;
            v = w;
            Yv = Yw;
            st = en;
        }
    }
    line_scans<gs>(sa.own, (uint16_t*)nullptr, myslot, g, Gp);
    // the owner entering the chunk becomes its first mark (marks only grow)
    const int enter = g > 0 ? sa.own[myslot - gs] : 0;
    if (n > 0 && enter > (int)mymarks[0]) mymarks[0] = (uint16_t)enter;
}

// --------------------------------------------------------------------------
// Row layout: lines contiguous in memory (the last axis).  A work-group holds
// LPW lines; lane g of a line owns chunk g.  The line is loaded with 16-byte
// coalesced reads.  Once every chunk's owners are in LDS, lane g writes the
// 4-position pieces g, g + Gp, ... of its line, so neighbouring lanes store
// neighbouring 16 bytes (a lane writing its own chunk would scatter each store
// over one cache line per lane).
// --------------------------------------------------------------------------

// Candidate values of the Euclidean passes: T = double (L2Metric), or int
// (L2IntMetric: every value and squared spacing times S = 2^shift, exact;
// the outputs divide by S again, exactly).
template <class T> struct L2Of { using type = L2Metric; };
template <> struct L2Of<int> { using type = L2IntMetric; };

template <class T>
struct Geo2DT {         // rows of B images of H x W; value = axis-0 coordinate
    using Val = uint16_t;
    static constexpr Val kNoneVal = kNone16;
    // Rows of an image follow the nearest background of one column each, so
    // their F varies freely along the row and many chunks see more reaching
    // members than the per-chunk lists hold: whole lines in rounds are faster
    // (16384^2: 0.90 against 1.07 ms; 4096^2 disks: 0.21 against 0.46 ms).
    static constexpr bool kPerChunk = false;
    static bool per_chunk(int) { return false; }
    using Metric = typename L2Of<T>::type;
    static constexpr bool kRootOut = true;   // float32 distances beside the squared ones
    static constexpr bool kScaled = !std::is_same<T, double>::value;
    T s2a, s2l;         // (S x) squared spacing of axis 0 and along the row
    int W;
    int H;              // rows per image: line ln is row ln % H of image ln / H
    int shift;          // S = 2^shift (scaled values only)
    float inv_s;        // 1 / S
    __device__ Metric metric() const { return Metric{s2l}; }
    struct Line { int row; };
    __device__ Line line(int64_t ln) const {
        return Line{ln < 0x100000000ll ? (int)((unsigned)ln % (unsigned)H) : (int)(ln % H)};
    }
    __device__ static bool valid(uint16_t v) { return v != kNone16; }
    __device__ T f(const Line& l, uint16_t v) const {
        const T t = (T)(l.row - (int)v);
        return s2a * t * t;
    }
    // v < 2^16 and W <= 32768: a 24-bit product is exact
    __device__ int32_t index(const Line&, uint16_t v, int pos) const {
        return (int32_t)__umul24((unsigned)v, (unsigned)W) + pos;
    }
    __device__ T virt_f(const Line& l) const {
        const T t = (T)(l.row + 1);
        return s2a * t * t;
    }
    __device__ int32_t virt_index() const { return -W; }
};
using Geo2D = Geo2DT<double>;

template <class T>
struct Geo3DT {         // rows along W of B x D x H x W volumes; value = packed (axis0, axis1)
    // Per-chunk resolution for rows longer than 128 (512^3: 0.66 ms against
    // 0.71 ms in whole-line rounds); rows of 128 or fewer go faster in rounds
    // (16 x 128^3: 0.288 against 0.310 ms).
    static constexpr bool kPerChunk = true;
    static bool per_chunk(int L) { return L > 128; }
    using Val = uint32_t;
    static constexpr Val kNoneVal = kNone32;
    using Metric = typename L2Of<T>::type;
    static constexpr bool kRootOut = true;
    static constexpr bool kScaled = !std::is_same<T, double>::value;
    T s2a, s2b, s2l;    // (S x) squared spacings
    int D, H, W;
    bool dh24;          // D * H < 2^24: the flat index needs only 24-bit products
    int shift;          // S = 2^shift (scaled values only)
    float inv_s;        // 1 / S
    __device__ Metric metric() const { return Metric{s2l}; }
    struct Line { int d, h; };
    __device__ Line line(int64_t ln) const {
        const unsigned DH = (unsigned)D * (unsigned)H;   // D * H * W < 2^31
        const unsigned dh = ln < 0x100000000ll ? (unsigned)ln % DH : (unsigned)(ln % DH);
        return Line{(int)(dh / (unsigned)H), (int)(dh % (unsigned)H)};
    }
    __device__ static bool valid(uint32_t v) { return v != kNone32; }
    __device__ T f(const Line& l, uint32_t v) const {
        const T t0 = (T)(l.d - (int)(v >> 16));
        const T t1 = (T)(l.h - (int)(v & 0xFFFFu));
        return s2a * t0 * t0 + s2b * t1 * t1;
    }
    __device__ int32_t index(const Line&, uint32_t v, int pos) const {
        // both factors are below 2^24, and d * H + h < 2^31 whenever int32
        // indices are asked for (D * H * W < 2^31)
        const unsigned dh = __umul24(v >> 16, (unsigned)H) + (v & 0xFFFFu);
        return (int32_t)(dh24 ? __umul24(dh, (unsigned)W) : dh * (unsigned)W) + pos;
    }
    __device__ T virt_f(const Line& l) const {
        const T t0 = (T)(l.d + 1);
        return s2a * t0 * t0 + s2b * (T)l.h * (T)l.h;
    }
    __device__ int32_t virt_index() const { return -(H * W); }
    // the same flat index for volumes over 2^31 - 1 elements
    __device__ int64_t index64(const Line&, uint32_t v, int pos) const {
        return ((int64_t)(v >> 16) * H + (v & 0xFFFFu)) * (int64_t)W + pos;
    }
};
using Geo3D = Geo3DT<double>;

// The chessboard (L-infinity) row passes (TorchMorph's chamfer transforms):
// the same lines and values, the candidate value g = the L-infinity distance
// over the earlier axes, f_j(q) = max(g_j, |q - j|), and int32 distances out
// (through the sqdist output).  The virtual element of an image without
// background sits one row before its first row, in column 0, as for the
// Euclidean transform.
struct GeoLinf2D {
    using Val = uint16_t;
    static constexpr Val kNoneVal = kNone16;
    static constexpr bool kPerChunk = false;
    static bool per_chunk(int) { return false; }
    using Metric = LinfMetric;
    static constexpr bool kRootOut = false;
    static constexpr bool kScaled = false;
    int W;
    int H;
    __device__ Metric metric() const { return LinfMetric{}; }
    struct Line { int row; };
    __device__ Line line(int64_t ln) const {
        return Line{ln < 0x100000000ll ? (int)((unsigned)ln % (unsigned)H) : (int)(ln % H)};
    }
    __device__ static bool valid(uint16_t v) { return v != kNone16; }
    __device__ int f(const Line& l, uint16_t v) const { return abs(l.row - (int)v); }
    __device__ int32_t index(const Line&, uint16_t v, int pos) const {
        return (int32_t)__umul24((unsigned)v, (unsigned)W) + pos;
    }
    __device__ int virt_f(const Line& l) const { return l.row + 1; }
    __device__ int32_t virt_index() const { return -W; }
};

struct GeoLinf3D {
    using Val = uint32_t;
    static constexpr Val kNoneVal = kNone32;
    static constexpr bool kPerChunk = true;
    static bool per_chunk(int L) { return L > 128; }
    using Metric = LinfMetric;
    static constexpr bool kRootOut = false;
    static constexpr bool kScaled = false;
    int D, H, W;
    bool dh24;
    __device__ Metric metric() const { return LinfMetric{}; }
    struct Line { int d, h; };
    __device__ Line line(int64_t ln) const {
        const unsigned DH = (unsigned)D * (unsigned)H;
        const unsigned dh = ln < 0x100000000ll ? (unsigned)ln % DH : (unsigned)(ln % DH);
        return Line{(int)(dh / (unsigned)H), (int)(dh % (unsigned)H)};
    }
    __device__ static bool valid(uint32_t v) { return v != kNone32; }
    __device__ int f(const Line& l, uint32_t v) const {
        return max(abs(l.d - (int)(v >> 16)), abs(l.h - (int)(v & 0xFFFFu)));
    }
    __device__ int32_t index(const Line&, uint32_t v, int pos) const {
        const unsigned dh = __umul24(v >> 16, (unsigned)H) + (v & 0xFFFFu);
        return (int32_t)(dh24 ? __umul24(dh, (unsigned)W) : dh * (unsigned)W) + pos;
    }
    __device__ int virt_f(const Line& l) const { return max(l.d + 1, l.h); }
    __device__ int32_t virt_index() const { return -(H * W); }
    __device__ int64_t index64(const Line&, uint32_t v, int pos) const {
        return ((int64_t)(v >> 16) * H + (v & 0xFFFFu)) * (int64_t)W + pos;
    }
};

template <int BYTES> struct RawVec;
template <> struct RawVec<16> { using T = uint4; };
template <> struct RawVec<8> { using T = uint2; };
template <> struct RawVec<4> { using T = uint32_t; };
template <> struct RawVec<2> { using T = uint16_t; };

// Load one line of L values (L % VW == 0) into its chunk slots: lane g of the
// line reads pieces g, g + Gp, ... of VW values each.
template <class Val, int K, int VW>
__device__ inline void load_row_line(const Val* __restrict__ src, int L, int g, int Gp, Val* dst) {
    constexpr int CS = Slots<Val, K>::CS;
    constexpr int NP = K / VW;               // pieces per lane at most (Gp * K >= L)
    constexpr int NB = NP < 16 ? NP : 16;    // loads kept in flight per batch
    using V = typename RawVec<VW * (int)sizeof(Val)>::T;
    const int PL = L / VW;
#pragma unroll
    for (int i0 = 0; i0 < NP; i0 += NB) {
        V buf[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int k = g + (i0 + i) * Gp;
            if (k < PL) buf[i] = reinterpret_cast<const V*>(src)[k];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int k = g + (i0 + i) * Gp;
            if (k < PL) {
                const int p = k * VW;
                Val* d = dst + __umul24((unsigned)p / K, CS) + ((unsigned)p % K);
                if constexpr (VW * sizeof(Val) == 16) {
                    uint32_t* d32 = reinterpret_cast<uint32_t*>(d);   // 4-byte aligned (CS even for uint16)
                    d32[0] = buf[i].x; d32[1] = buf[i].y; d32[2] = buf[i].z; d32[3] = buf[i].w;
                } else {
                    d[0] = buf[i];
                }
            }
        }
    }
}

template <class Geo, int K, int VW, class Ix = int32_t, bool PerChunk = Geo::kPerChunk>
__global__ __launch_bounds__(1024) void k_envelope_rows(const typename Geo::Val* __restrict__ in,
                                                        int L, int64_t nlines, int Gp, int LPW,
                                                        Geo geo, int32_t* __restrict__ sqdist,
                                                        float* __restrict__ dist,
                                                        Ix* __restrict__ indices, int vec_out) {
    using Val = typename Geo::Val;
    constexpr int CS = Slots<Val, K>::CS;
    constexpr int CM = Slots<Val, K>::CM;
    extern __shared__ __align__(16) unsigned char smem[];
    SlotArrays<Val, K> sa(smem, Gp * LPW, Gp);

    const int tid = threadIdx.x;
    const int g = tid & (Gp - 1);
    const int r = tid / Gp;
    const int slot0 = r * Gp;
    const int64_t line = (int64_t)blockIdx.x * LPW + r;
    const bool active = line < nlines;

    if (active) load_row_line<Val, K, VW>(in + line * (int64_t)L, L, g, Gp, sa.val + __umul24(slot0, CS));
    {   // positions past the end of the line (all of an inactive one) hold
        // "no background", so that validity alone marks the chunk's positions
        const int nv = active ? L - g * K : 0;
        Val* mc = sa.val + __umul24(tid, CS);
        for (int t = nv < 0 ? 0 : nv; t < K; ++t) mc[t] = Geo::kNoneVal;
    }
    __syncthreads();

    const typename Geo::Line gl = geo.line(active ? line : 0);
    auto fof = [&](Val v) { return geo.f(gl, v); };
    using Mt = typename Geo::Metric;
    LineView<Val, K, decltype(fof), 1, Mt> view{sa.val, sa.mask, sa.occ + (size_t)r * ((Gp + 63) / 64),
                                                sa.own, slot0, geo.metric(), fof};
    uint16_t* mymarks = sa.mark + __umul24(tid, CM);
    resolve_line<K, PerChunk>(view, sa, sa.val + __umul24(tid, CS), mymarks, g, Gp, L, active, tid, r,
                    [](Val v) { return Geo::valid(v); }, fof);

    // 5. outputs.  mk is owner + 1 of position q (0: the line has no
    //    background, the owner is the virtual element).
    const int n = active ? min(K, L - g * K) : 0;
    const Mt mt = geo.metric();
    const typename Mt::Val fvirt = geo.virt_f(gl);
    const int32_t ivirt = geo.virt_index();
    auto one = [&](int q, int mk, int32_t& osq, float& od, Ix& oix) {
        const int ow = mk - 1;
        const int oq = ow < 0 ? 0 : ow;   // the virtual element acts as one at position 0
        const Val vo = view.val(oq);
        const typename Mt::Val F = mt.combine(ow < 0 ? fvirt : fof(vo), mt.dist(q - oq));
        if constexpr (Geo::kScaled) {   // F = S x the squared distance, S = 2^shift
            osq = sqdist ? (int32_t)(F >> geo.shift) : 0;
            od = __builtin_amdgcn_sqrtf((float)F * geo.inv_s);   // (exact scaling)
        } else {
            osq = sqdist ? (int32_t)F : 0;
            if constexpr (Geo::kRootOut) od = __builtin_amdgcn_sqrtf((float)F);
            else od = 0.0f;
        }
        if constexpr (sizeof(Ix) == 8) oix = ow < 0 ? (Ix)ivirt : (Ix)geo.index64(gl, vo, ow);
        else oix = ow < 0 ? ivirt : geo.index(gl, vo, ow);
    };
    const int64_t lbase = line * (int64_t)L;
    int32_t osq[4];
    float od[4];
    Ix oix[4];
    auto store4 = [&](int64_t ob) {
        if (sqdist) *reinterpret_cast<int4*>(sqdist + ob) = make_int4(osq[0], osq[1], osq[2], osq[3]);
        if (dist) *reinterpret_cast<float4*>(dist + ob) = make_float4(od[0], od[1], od[2], od[3]);
        if (indices) {
            if constexpr (sizeof(Ix) == 8) {
                *reinterpret_cast<longlong2*>(indices + ob) = make_longlong2(oix[0], oix[1]);
                *reinterpret_cast<longlong2*>(indices + ob + 2) = make_longlong2(oix[2], oix[3]);
            } else {
                *reinterpret_cast<int4*>(indices + ob) = make_int4(oix[0], oix[1], oix[2], oix[3]);
            }
        }
    };
    // The marks of the own chunk become owners (running maximum, in place);
    // then lane g writes the 4-position pieces g, g + Gp, ... of the line, so
    // that neighbouring lanes store neighbouring 16-byte pieces.
    int o = 0;
    for (int t = 0; t < n; ++t) {
        const int mk = mymarks[t];
        o = mk > o ? mk : o;
        mymarks[t] = (uint16_t)o;
    }
    __syncthreads();
    if (!active) return;   // no barrier follows
    const uint16_t* marks = sa.mark + __umul24(slot0, CM);
    if (vec_out) {   // L % 4 == 0 and 16-byte aligned outputs
#pragma unroll 2
        for (int i = 0; i < K / 4; ++i) {
            const int p = 4 * (i * Gp + g);
            if (p >= L) break;
            const uint16_t* om = marks + __umul24((unsigned)p / K, CM) + (unsigned)p % K;
#pragma unroll
            for (int j = 0; j < 4; ++j) one(p + j, om[j], osq[j], od[j], oix[j]);
            store4(lbase + p);
        }
    } else {
        for (int p = g; p < L; p += Gp) {
            one(p, marks[__umul24((unsigned)p / K, CM) + (unsigned)p % K], osq[0], od[0], oix[0]);
            if (sqdist) sqdist[lbase + p] = osq[0];
            if (dist) dist[lbase + p] = od[0];
            if (indices) indices[lbase + p] = oix[0];
        }
    }
}

// --------------------------------------------------------------------------
// Rows of at most 1024 positions: one wave per line, lane l holding the P
// consecutive positions [P l, P l + P).  The candidates are filtered exactly as
// above (bound U and chunk-minimiser test over chunks of 16 positions), then
// the envelope of the survivors is found in rounds: every surviving candidate
// checks, against its current neighbours in the line, the dominance test of
// PR-EDT Figure 5, and all dominated ones leave together.  A point above the
// segment between two points of the set stays above the lower hull of what
// remains, so when a round removes nothing the survivors form a locally and
// hence globally convex chain: the envelope.  Every lane takes the same steps
// for its own few candidates, so the work follows the candidates, not the
// slowest chunk.  Each member then marks where it starts to own (against its
// predecessor), a prefix maximum gives each position its owner, and lane l
// writes its P outputs.
// --------------------------------------------------------------------------

template <class Geo, int P>
__global__ __launch_bounds__(64) void k_rows_wave(const typename Geo::Val* __restrict__ in, int L,
                                                  Geo geo, int32_t* __restrict__ sqdist,
                                                  float* __restrict__ dist,
                                                  int32_t* __restrict__ indices, int vec_io) {
    using Val = typename Geo::Val;
    static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "1 to 16 positions per lane");
    constexpr int NP = 64 * P;
    constexpr int KC = 16;          // chunk of the candidate bound and filter
    constexpr int GL = KC / P;      // lanes per chunk
    constexpr unsigned kNoneV = sizeof(Val) == 2 ? kNone16 : kNone32;
    __shared__ double Ys[NP];       // Y = F + s^2 q^2 of position q (+inf: no candidate)
    __shared__ Val vs[NP];          // the values, for the owners' outputs
    __shared__ unsigned marks[NP];  // owner + 1 where an owned interval starts
    __shared__ unsigned lanes_alive[64];

    const int lane = threadIdx.x;
    const int64_t line = blockIdx.x;
    const int base = lane * P;
    const double s2 = geo.s2l;
    const typename Geo::Line gl = geo.line(line);

    // 1. values and heights
    const Val* src = in + line * (int64_t)L;
    Val v[P];
    if (P >= 4 && vec_io) {   // L % 4 == 0, 4-value pieces aligned
#pragma unroll
        for (int t = 0; t < P; t += 4) {
            const int p = base + t;
            if (p < L) {
                if constexpr (sizeof(Val) == 4) {
                    const uint4 w = *reinterpret_cast<const uint4*>(src + p);
                    v[t] = w.x; v[t + 1] = w.y; v[t + 2] = w.z; v[t + 3] = w.w;
                } else {
                    const uint2 w = *reinterpret_cast<const uint2*>(src + p);
                    v[t] = (Val)w.x; v[t + 1] = (Val)(w.x >> 16); v[t + 2] = (Val)w.y; v[t + 3] = (Val)(w.y >> 16);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[t + j] = (Val)kNoneV;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < P; ++t) v[t] = base + t < L ? src[base + t] : (Val)kNoneV;
    }
    double F[P];
    unsigned vmask = 0;
    double fmin = __builtin_huge_val();
    int amin = -1;
#pragma unroll
    for (int t = 0; t < P; ++t) {
        const int p = base + t;
        const bool ok = p < L && Geo::valid(v[t]);
        F[t] = ok ? geo.f(gl, v[t]) : __builtin_huge_val();
        if (ok) vmask |= 1u << t;
        Ys[p] = ok ? F[t] + s2 * (double)p * (double)p : __builtin_huge_val();
        vs[p] = v[t];
        marks[p] = 0u;
        if (F[t] < fmin) { fmin = F[t]; amin = p; }
    }

    // 2. chunk minimum and first minimiser (GL lanes per chunk), the bound U
#pragma unroll
    for (int o = 1; o < GL; o <<= 1) {
        const double f2 = __shfl_xor(fmin, o);
        const int a2 = __shfl_xor(amin, o);
        if (f2 < fmin || (f2 == fmin && a2 >= 0 && (amin < 0 || a2 < amin))) { fmin = f2; amin = a2; }
    }
    double fpv = __shfl(fmin, (lane - GL) & 63), fnx = __shfl(fmin, (lane + GL) & 63);
    int apv = __shfl(amin, (lane - GL) & 63), anx = __shfl(amin, (lane + GL) & 63);
    if (lane < GL) { fpv = __builtin_huge_val(); apv = -1; }
    if (lane + GL >= 64) { fnx = __builtin_huge_val(); anx = -1; }
    double U = (lane / GL) * KC < L ? chunk_bound(fmin, fpv, fnx, s2, KC) : 0.0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) U = fmax(U, __shfl_xor(U, o));
    __syncthreads();

    // 3. candidates: valid, F <= U, not dominated by the nearest chunk minimisers
    const double Ycur = amin >= 0 ? Ys[amin] : 0.0;
    const double Yprev = apv >= 0 ? Ys[apv] : 0.0;
    const double Ynext = anx >= 0 ? Ys[anx] : 0.0;
    unsigned alive = 0;
#pragma unroll
    for (int t = 0; t < P; ++t) {
        const int p = base + t;
        const double Yp = F[t] + s2 * (double)p * (double)p;
        const int lo = amin >= 0 && amin < p ? amin : apv;
        const double Ylo = amin >= 0 && amin < p ? Ycur : Yprev;
        const int hi = amin > p ? amin : anx;
        const double Yhi = amin > p ? Ycur : Ynext;
        const bool gone = lo >= 0 && hi >= 0 && dominated(lo, Ylo, p, Yp, hi, Yhi);
        if (((vmask >> t) & 1u) && F[t] <= U && !gone) alive |= 1u << t;
    }

    // neighbours of the candidate at offset t among the alive set of the round
    // (nz: lanes with an alive candidate; lanes_alive: their sets)
    auto pred_of = [&](int t, uint64_t nz) -> int {
        const unsigned below = alive & ((1u << t) - 1u);
        if (below) return base + 31 - __builtin_clz(below);
        const uint64_t lm = nz & ((uint64_t(1) << lane) - 1);
        if (!lm) return -1;
        const int j = 63 - __builtin_clzll(lm);
        return j * P + 31 - __builtin_clz(lanes_alive[j]);
    };
    auto succ_of = [&](int t, uint64_t nz) -> int {
        const unsigned above = alive & ~((2u << t) - 1u);
        if (above) return base + __builtin_ctz(above);
        const uint64_t rm = lane == 63 ? 0 : nz & ~((uint64_t(2) << lane) - 1);
        if (!rm) return -1;
        const int j = __builtin_ctzll(rm);
        return j * P + __builtin_ctz(lanes_alive[j]);
    };

    // 4. envelope of the lane's own candidates (insertion sweep, stack as a
    //    bit mask), then rounds over the lane boundaries: only a lane's first
    //    and last members have neighbours outside it, and a member whose
    //    neighbours change by a removal becomes a first or last one, so each
    //    round tests those two per lane, removes the dominated ones together,
    //    and stops when a round removes nothing.
    {
        unsigned m = 0, cand = alive;
        int top = -1, sec = -1;
        double Ytop = 0.0, Ysec = 0.0;
        while (cand) {
            const int t = __builtin_ctz(cand);
            cand &= cand - 1u;
            const int p = base + t;
            const double Y = Ys[p];
            while (sec >= 0 && dominated(sec, Ysec, top, Ytop, p, Y)) {
                m &= ~(1u << (top - base));
                top = sec;
                Ytop = Ysec;
                const unsigned below = m & ((1u << (top - base)) - 1u);
                if (below) {
                    sec = base + 31 - __builtin_clz(below);
                    Ysec = Ys[sec];
                } else {
                    sec = -1;
                }
            }
            m |= 1u << t;
            sec = top;
            Ysec = Ytop;
            top = p;
            Ytop = Y;
        }
        alive = m;
    }
    for (;;) {
        lanes_alive[lane] = alive;
        const uint64_t nz = __ballot(alive != 0u);
        __syncthreads();
        unsigned dead = 0;
        if (alive) {
            const int t0 = __builtin_ctz(alive), t1 = 31 - __builtin_clz(alive);
            {
                const int p = base + t0, pp = pred_of(t0, nz), pn = succ_of(t0, nz);
                if (pp >= 0 && pn >= 0 && dominated(pp, Ys[pp], p, Ys[p], pn, Ys[pn])) dead |= 1u << t0;
            }
            if (t1 != t0) {
                const int p = base + t1, pp = pred_of(t1, nz), pn = succ_of(t1, nz);
                if (pp >= 0 && pn >= 0 && dominated(pp, Ys[pp], p, Ys[p], pn, Ys[pn])) dead |= 1u << t1;
            }
        }
        alive &= ~dead;
        const bool more = __ballot(dead != 0u) != 0;
        __syncthreads();
        if (!more) break;
    }
    lanes_alive[lane] = alive;
    __syncthreads();

    // 5. every member marks the first position it owns (strictly nearer than
    //    its predecessor there; ties stay with the smaller coordinate)
    {
        const uint64_t nz = __ballot(alive != 0u);   // lanes_alive already holds alive
        unsigned rest = alive;
        while (rest) {
            const int t = __builtin_ctz(rest);
            rest &= rest - 1u;
            const int p = base + t;
            const int pp = pred_of(t, nz);
            const int st = pp < 0 ? 0 : first_index_beating(Ys[p] - Ys[pp], 2.0 * s2 * (double)(p - pp), L);
            if (st < L) atomicMax(&marks[st], (unsigned)(p + 1));
        }
    }
    __syncthreads();

    // 6. owner of each position: prefix maximum of the marks along the line
    unsigned own[P];
    unsigned run = 0;
#pragma unroll
    for (int t = 0; t < P; ++t) {
        const unsigned mk = marks[base + t];
        run = mk > run ? mk : run;
        own[t] = run;
    }
    unsigned incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned x = __shfl_up(incl, o);
        if (lane >= o) incl = x > incl ? x : incl;
    }
    unsigned excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0;

    // 7. outputs (owner + 1 == 0: the line has no background, the virtual element)
    const double fvirt = geo.virt_f(gl);
    const int32_t ivirt = geo.virt_index();
    const int64_t lbase = line * (int64_t)L;
    int32_t osq[P];
    float od[P];
    int32_t oix[P];
#pragma unroll
    for (int t = 0; t < P; ++t) {
        const int q = base + t;
        const int ow = (int)(own[t] > excl ? own[t] : excl) - 1;
        const Val vo = vs[ow < 0 ? 0 : ow];
        const double qq = (double)q;
        const double dq = (double)(q - ow);
        const double Fq = ow < 0 ? fvirt + s2 * qq * qq : geo.f(gl, vo) + s2 * dq * dq;
        osq[t] = sqdist ? (int32_t)Fq : 0;
        od[t] = __builtin_amdgcn_sqrtf((float)Fq);
        oix[t] = ow < 0 ? ivirt : geo.index(gl, vo, ow);
    }
    if (P >= 4 && vec_io) {
#pragma unroll
        for (int t = 0; t < P; t += 4) {
            const int q = base + t;
            if (q < L) {
                if (sqdist) *reinterpret_cast<int4*>(sqdist + lbase + q) = make_int4(osq[t], osq[t + 1], osq[t + 2], osq[t + 3]);
                if (dist) *reinterpret_cast<float4*>(dist + lbase + q) = make_float4(od[t], od[t + 1], od[t + 2], od[t + 3]);
                if (indices) *reinterpret_cast<int4*>(indices + lbase + q) = make_int4(oix[t], oix[t + 1], oix[t + 2], oix[t + 3]);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < P; ++t) {
            const int q = base + t;
            if (q < L) {
                if (sqdist) sqdist[lbase + q] = osq[t];
                if (dist) dist[lbase + q] = od[t];
                if (indices) indices[lbase + q] = oix[t];
            }
        }
    }
}

template <class Geo, int P>
static hipError_t launch_rows_wave_t(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                                     int32_t* sqdist, float* dist, int32_t* indices, hipStream_t s,
                                     KernelTimer* tm, const char* kname) {
    constexpr int VB = (int)sizeof(typename Geo::Val);
    const bool vec = L % 4 == 0 && (((uintptr_t)in & (4 * VB - 1)) == 0) &&
                     ((((uintptr_t)sqdist | (uintptr_t)dist | (uintptr_t)indices) & 15) == 0);
    EDT_LAUNCH(tm, kname, s,
               hipLaunchKernelGGL((k_rows_wave<Geo, P>), dim3((unsigned)nlines), dim3(64), 0, s, in, L,
                                  geo, sqdist, dist, indices, vec ? 1 : 0));
    return hipSuccess;
}

// Few lines of at most 1024 positions take the one-wave kernel: it launches
// one wave per line where the chunk kernel would leave most CUs idle (for
// many lines the two run at about the same speed, the chunk kernel slightly
// ahead on 512-position lines).  Returns false when the chunk kernel is used.
template <class Geo>
static bool launch_rows_wave(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                             int32_t* sqdist, float* dist, int32_t* indices, hipStream_t s,
                             KernelTimer* tm, const char* kname, hipError_t* err) {
    if (L > 1024 || nlines > 65536) return false;
    if (L <= 64) *err = launch_rows_wave_t<Geo, 1>(in, L, nlines, geo, sqdist, dist, indices, s, tm, kname);
    else if (L <= 128) *err = launch_rows_wave_t<Geo, 2>(in, L, nlines, geo, sqdist, dist, indices, s, tm, kname);
    else if (L <= 256) *err = launch_rows_wave_t<Geo, 4>(in, L, nlines, geo, sqdist, dist, indices, s, tm, kname);
    else if (L <= 512) *err = launch_rows_wave_t<Geo, 8>(in, L, nlines, geo, sqdist, dist, indices, s, tm, kname);
    else *err = launch_rows_wave_t<Geo, 16>(in, L, nlines, geo, sqdist, dist, indices, s, tm, kname);
    return true;
}

struct RowPlan {
    int K, Gp, LPW, VW;
    size_t lds;
};

// Chunk size: 32 positions for 16-bit values, 16 for 32-bit values (their
// larger slots would otherwise leave too few lanes resident per CU).  Lines
// shorter than a wave share one, 64 threads per block: small blocks let the
// phases of several blocks overlap on a CU, so one block waiting at a barrier
// for its slowest lane leaves the SIMDs to the others.
static RowPlan plan_rows(int L, int value_bytes) {
    RowPlan p{};
    p.K = value_bytes == 2 ? 32 : 16;
    const int chunks = (L + p.K - 1) / p.K;
    p.Gp = 1;
    while (p.Gp < chunks) p.Gp <<= 1;
    p.LPW = p.Gp >= 64 ? 1 : 64 / p.Gp;
    const int nslots = p.Gp * p.LPW;
    const int vw16 = 16 / value_bytes;
    p.VW = (L % vw16 == 0) ? vw16 : 1;
    p.lds = value_bytes == 2 ? Slots<uint16_t, 32>::bytes(nslots, p.Gp) : Slots<uint32_t, 16>::bytes(nslots, p.Gp);
    return p;
}

size_t rows_lds_bytes(int L, int value_bytes) {
    const RowPlan p = plan_rows(L, value_bytes);
    if (p.Gp > 1024 || p.lds > 160 * 1024) return 0;
    return p.lds;
}

template <class Geo, int K, int VW, class Ix, bool PerChunk>
static hipError_t launch_rows_t(const typename Geo::Val* in, int L, int64_t nlines, const RowPlan& p,
                                const Geo& geo, int32_t* sqdist, float* dist, Ix* indices,
                                hipStream_t s, KernelTimer* tm, const char* kname) {
    static unsigned long long lds_done = 0;
    hipError_t le = large_lds_once((const void*)k_envelope_rows<Geo, K, VW, Ix, PerChunk>, &lds_done);
    if (le != hipSuccess) return le;
    const int64_t nblocks = (nlines + p.LPW - 1) / p.LPW;
    const bool aligned16 = (((uintptr_t)sqdist | (uintptr_t)dist | (uintptr_t)indices) & 15) == 0;
    const int vec_out = (L % 4 == 0 && aligned16) ? 1 : 0;
    EDT_LAUNCH(tm, kname, s,
               hipLaunchKernelGGL((k_envelope_rows<Geo, K, VW, Ix, PerChunk>), dim3((unsigned)nblocks),
                                  dim3(p.Gp * p.LPW), p.lds, s, in, L, nlines, p.Gp, p.LPW, geo,
                                  sqdist, dist, indices, vec_out));
    return hipSuccess;
}

template <class Geo, int K, class Ix>
static hipError_t launch_rows_any(const typename Geo::Val* in, int L, int64_t nlines, const Geo& geo,
                                  int32_t* sqdist, float* dist, Ix* indices, hipStream_t s,
                                  KernelTimer* tm, const char* kname) {
    constexpr int VB = (int)sizeof(typename Geo::Val);
    constexpr int V16 = 16 / VB;
    const RowPlan p = plan_rows(L, VB);
    if (Geo::kPerChunk && !Geo::per_chunk(L)) {   // (only Geo3D takes both)
        if (p.VW == V16)
            return launch_rows_t<Geo, K, V16, Ix, false>(in, L, nlines, p, geo, sqdist, dist, indices, s, tm, kname);
        return launch_rows_t<Geo, K, 1, Ix, false>(in, L, nlines, p, geo, sqdist, dist, indices, s, tm, kname);
    }
    if (p.VW == V16)
        return launch_rows_t<Geo, K, V16, Ix, Geo::kPerChunk>(in, L, nlines, p, geo, sqdist, dist, indices, s, tm, kname);
    return launch_rows_t<Geo, K, 1, Ix, Geo::kPerChunk>(in, L, nlines, p, geo, sqdist, dist, indices, s, tm, kname);
}

// Exact integer values for a pass (L2IntMetric): the smallest S = 2^k,
// k <= 10, with every S * s2[i] an integer (at most 2^20), provided that
// S * sum_i s2[i] * ext[i]^2 stays below 2^29, ext[i] bounding the offsets
// the pass forms along axis i (the virtual element's and the chunk bound's
// included).  -1: the pass keeps double values.  (A larger S only raises the
// sum, so the smallest one decides.)
static int int_scale_shift(const double* s2, const double* ext, int n) {
    for (int k = 0; k <= 10; ++k) {
        const double S = (double)(1 << k);
        bool whole = true;
        double ymax = 0.0;
        for (int i = 0; i < n; ++i) {
            const double x = S * s2[i];
            if (!(x >= 0.0 && x <= 1048576.0 && x == rint(x))) whole = false;   // (NaN: false)
            ymax += x * ext[i] * ext[i];
        }
        if (whole) return ymax < 536870912.0 ? k : -1;
    }
    return -1;
}

hipError_t launch_rows_2d(const uint16_t* c0, int B, int H, int W, double s2_0, double s2_1,
                          int32_t* sqdist, float* dist, int32_t* indices, hipStream_t s,
                          KernelTimer* tm) {
    Geo2D geo{s2_0, s2_1, W, H};
    const int64_t nlines = (int64_t)B * H;
    hipError_t e = hipSuccess;
    if (launch_rows_wave<Geo2D>(c0, W, nlines, geo, sqdist, dist, indices, s, tm, "envelope_rows_2d", &e))
        return e;
    const double s2[2] = {s2_0, s2_1}, ext[2] = {(double)H, (double)std::max(W - 1, 63)};
    const int k = int_scale_shift(s2, ext, 2);
    if (k >= 0) {
        const int S = 1 << k;
        const Geo2DT<int> gi{(int)(S * s2_0), (int)(S * s2_1), W, H, k, 1.0f / (float)S};
        return launch_rows_any<Geo2DT<int>, 32>(c0, W, nlines, gi, sqdist, dist, indices, s, tm,
                                                "envelope_rows_2d");
    }
    return launch_rows_any<Geo2D, 32>(c0, W, nlines, geo, sqdist, dist, indices, s, tm, "envelope_rows_2d");
}

// --------------------------------------------------------------------------
// Flat indices -> per-axis coordinates (the layout SciPy's feature transform
// returns: per image an array of ndim planes, plane k holding the axis-k
// coordinate of every element's nearest background element).  Division
// rounds toward minus infinity, so the virtual element's negative flat index
// -(n1 * ... * n_{d-1}) becomes (-1, 0, ..., 0).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_unravel(const int32_t* __restrict__ flat, int64_t total,
                                                 int64_t per_image, int ndim, int n1, int n2,
                                                 int32_t* __restrict__ coords) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t b = e / per_image;
    const int64_t i = e - b * per_image;
    int f = flat[e];
    int c[3] = {0, 0, 0};
    auto divmod = [](int x, int d, int& q, int& r) {   // floor division, 0 <= r < d
        q = x / d;
        r = x - q * d;
        if (r < 0) { r += d; --q; }
    };
    if (ndim == 1) {
        c[0] = f;
    } else if (ndim == 2) {
        divmod(f, n1, c[0], c[1]);
    } else {
        int t;
        divmod(f, n2, t, c[2]);
        divmod(t, n1, c[0], c[1]);
    }
    int32_t* dst = coords + b * (int64_t)ndim * per_image + i;
    for (int k = 0; k < ndim; ++k) dst[(int64_t)k * per_image] = c[k];
}

hipError_t launch_unravel(const int32_t* flat, int64_t images, int64_t per_image, int ndim, int n1,
                          int n2, int32_t* coords, hipStream_t s) {
    const int64_t total = images * per_image;
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(k_unravel, dim3(blocks), dim3(256), 0, s, flat, total, per_image, ndim, n1, n2,
                       coords);
    return hipGetLastError();
}

hipError_t launch_rows_3d(const uint32_t* c01, int B, int D, int H, int W, double s2_0,
                          double s2_1, double s2_2, int32_t* sqdist, float* dist,
                          int32_t* indices, int64_t* indices64, hipStream_t s, KernelTimer* tm) {
    const bool dh24 = (int64_t)D * H < (1 << 24);
    Geo3D geo{s2_0, s2_1, s2_2, D, H, W, dh24};
    const int64_t nlines = (int64_t)B * D * H;
    const double s2[3] = {s2_0, s2_1, s2_2}, ext[3] = {(double)D, (double)H, (double)std::max(W - 1, 31)};
    const int k = int_scale_shift(s2, ext, 3);
    const int S = 1 << (k < 0 ? 0 : k);
    const Geo3DT<int> gi{(int)(S * s2_0), (int)(S * s2_1), (int)(S * s2_2), D, H, W, dh24, k, 1.0f / (float)S};
    if (indices64) {   // int64 indices: the chunk kernel for any number of lines
        if (k >= 0)
            return launch_rows_any<Geo3DT<int>, 16>(c01, W, nlines, gi, sqdist, dist, indices64, s, tm,
                                                    "envelope_rows_3d");
        return launch_rows_any<Geo3D, 16>(c01, W, nlines, geo, sqdist, dist, indices64, s, tm,
                                          "envelope_rows_3d");
    }
    hipError_t e = hipSuccess;
    if (launch_rows_wave<Geo3D>(c01, W, nlines, geo, sqdist, dist, indices, s, tm, "envelope_rows_3d", &e)) return e;
    if (k >= 0)
        return launch_rows_any<Geo3DT<int>, 16>(c01, W, nlines, gi, sqdist, dist, indices, s, tm,
                                                "envelope_rows_3d");
    return launch_rows_any<Geo3D, 16>(c01, W, nlines, geo, sqdist, dist, indices, s, tm, "envelope_rows_3d");
}

// Chessboard row passes on the envelope kernel (lines that fit its LDS).
hipError_t launch_rows_linf_2d(const uint16_t* c0, int B, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm) {
    const GeoLinf2D geo{W, H};
    return launch_rows_any<GeoLinf2D, 32>(c0, W, (int64_t)B * H, geo, dist, (float*)nullptr, indices, s, tm,
                                          "chessboard_rows");
}

hipError_t launch_rows_linf_3d(const uint32_t* c01, int B, int D, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm) {
    const GeoLinf3D geo{D, H, W, (int64_t)D * H < (1 << 24)};
    return launch_rows_any<GeoLinf3D, 16>(c01, W, (int64_t)B * D * H, geo, dist, (float*)nullptr, indices, s,
                                          tm, "chessboard_rows");
}

// --------------------------------------------------------------------------
// Column layout: the middle axis of a volume, lines strided by W.  A
// work-group takes TW neighbouring lines (lane x = line) and Gp chunk groups
// (chunk g of all TW lines), so every global load and store moves TW
// consecutive elements.  Each lane loads its own chunk.
// --------------------------------------------------------------------------

struct ColPlan {
    int K, TW, Gp;
    size_t lds;
};

// H <= 128: chunks of 16 (16 x 128^3: 0.28 -> 0.26 ms against chunks of 32;
// at H = 512 they cost 0.48 -> 0.65 ms); H <= 512: chunks of 32.  Both with
// 64 / Gp lines per block (at least 8).  Longer lines: chunks of 64 and 512 /
// Gp lines per block (32 lines up to H = 1024,
// one line at H = 32768), so that a block's 512 slots of values and marks
// stay within the LDS (narrower tiles mean smaller blocks, more of them
// resident per CU).
static ColPlan plan_cols(int H) {
    ColPlan p{};
    p.K = H <= 128 ? 16 : H <= 512 ? 32 : 64;
    p.Gp = 1;
    while (p.Gp * p.K < H) p.Gp <<= 1;
    // the narrowest tile that still fills one wave (8 lines at the least)
    p.TW = p.K == 64 ? (512 / p.Gp > 0 ? 512 / p.Gp : 0) : (64 / p.Gp > 8 ? 64 / p.Gp : 8);
    const int n = p.Gp * p.TW;
    p.lds = p.K == 16 ? Slots<uint16_t, 16>::bytes(n, p.Gp)
            : p.K == 32 ? Slots<uint16_t, 32>::bytes(n, p.Gp) : Slots<uint16_t, 64>::bytes(n, p.Gp);
    return p;
}

size_t cols_lds_bytes(int H) {
    const ColPlan p = plan_cols(H);
    return (p.TW < 1 || p.Gp * p.TW > 1024 || p.lds > 160 * 1024) ? 0 : p.lds;
}

// Candidate values of the middle-axis pass from the axis-0 coordinate v at
// plane d: the Euclidean one (s2a (d - v)^2, lines of squared spacing s2l; in
// double, or scaled integers) and the chessboard one (|d - v|).
template <class T>
struct ColL2T {
    using Metric = typename L2Of<T>::type;
    static constexpr bool kPerChunk = true;   // per-chunk owners first (step 4)
    T s2a, s2l;   // (S x) squared spacings
    __device__ Metric metric() const { return Metric{s2l}; }
    __device__ T f(int d, uint16_t v) const {
        const T t = (T)(d - (int)v);
        return s2a * t * t;
    }
};
using ColL2 = ColL2T<double>;
struct ColLinf {
    using Metric = LinfMetric;
    // whole-line rounds: 512^3 middle axis 1.25 -> 1.23 ms, 16 x 128^3 0.49 ->
    // 0.45 ms against per-chunk owners
    static constexpr bool kPerChunk = false;
    __device__ Metric metric() const { return LinfMetric{}; }
    __device__ int f(int d, uint16_t v) const { return abs(d - (int)v); }
};

template <int K, int TW, class CG>
__global__ __launch_bounds__(1024) void k_envelope_cols(const uint16_t* __restrict__ c0,
                                                        uint32_t* __restrict__ out, int D, int H,
                                                        int W, int Gp, CG cg) {
    constexpr int CS = Slots<uint16_t, K>::CS;
    constexpr int CM = Slots<uint16_t, K>::CM;
    extern __shared__ __align__(16) unsigned char smem[];
    SlotArrays<uint16_t, K> sa(smem, Gp * TW, Gp);

    const int x = threadIdx.x;
    const int g = threadIdx.y;
    const int tid = g * TW + x;
    // Work-groups are dealt to the eight XCDs in turn.  The SH tiles that
    // share 128-byte lines of a row go to one XCD (one L2 fetches each line
    // once), and consecutive groups of them still go round the XCDs, so cheap
    // and costly planes stay spread over all of them.
    constexpr unsigned SH = TW * 2 >= 128 ? 1 : 128 / (TW * 2);
    unsigned tile_id = blockIdx.x;
    if (SH > 1 && blockIdx.x < gridDim.x / (8 * SH) * (8 * SH)) {
        const unsigned xcd = blockIdx.x % 8, k = blockIdx.x / 8;
        tile_id = ((k / SH) * 8 + xcd) * SH + k % SH;
    }
    const int tiles = (W + TW - 1) / TW;
    const int64_t plane = tile_id / tiles;
    const int w0 = (int)(tile_id % tiles) * TW;
    const bool active = (w0 + x) < W;
    const int d = (int)(plane % D);
    const int base = g * K;
    const int n = active ? min(K, H - base) : 0;

    // own chunk: rows base .. base + n - 1 of column w0 + x (all loads issued
    // before any is used; rows past the end read row n - 1 and are discarded)
    uint16_t* mine = sa.val + __umul24(tid, CS);
    if (n > 0) {
        const uint16_t* src = c0 + plane * (int64_t)H * W + (int64_t)base * W + w0 + x;
        uint16_t buf[K];
#pragma unroll
        for (int t = 0; t < K; ++t) buf[t] = src[(int64_t)min(t, n - 1) * W];
#pragma unroll
        for (int t = 0; t < K; t += 2) {
            const uint32_t lo = t < n ? buf[t] : kNone16;
            const uint32_t hi = t + 1 < n ? buf[t + 1] : kNone16;
            *reinterpret_cast<uint32_t*>(mine + t) = lo | (hi << 16);
        }
    } else {   // no rows: every position holds "no background"
#pragma unroll
        for (int t = 0; t < K; t += 2) *reinterpret_cast<uint32_t*>(mine + t) = kNone16 | (kNone16 << 16);
    }

    auto fof = [&](uint16_t v) { return cg.f(d, v); };
    // (line x's occupancy words follow those of lines 0 .. x - 1)
    LineView<uint16_t, K, decltype(fof), TW, typename CG::Metric> view{
        sa.val, sa.mask, sa.occ + (size_t)x * ((Gp + 63) / 64), sa.own, x, cg.metric(), fof};
    uint16_t* mymarks = sa.mark + __umul24(tid, CM);
    resolve_line<K, CG::kPerChunk>(view, sa, mine, mymarks, g, Gp, H, active, tid, x,
                    [](uint16_t v) { return v != kNone16; }, fof);
    int o = 0;

    if (n <= 0) return;   // no barrier follows
    uint32_t* dst = out + plane * (int64_t)H * W + (int64_t)base * W + w0 + x;
#pragma unroll 4
    for (int t = 0; t < n; ++t) {
        const int mk = mymarks[t];
        o = mk > o ? mk : o;
        const int ow = o - 1;
        const uint32_t hi = (uint32_t)view.val(ow < 0 ? 0 : ow) << 16;
        dst[(int64_t)t * W] = ow < 0 ? kNone32 : (hi | (uint32_t)ow);
    }
}

template <int K, int TW, class CG>
static hipError_t launch_cols_t(const uint16_t* c0, int B, int D, int H, int W, const CG& cg,
                                uint32_t* c01, const ColPlan& p, hipStream_t s, KernelTimer* tm,
                                const char* kname) {
    static unsigned long long lds_done = 0;
    hipError_t le = large_lds_once((const void*)k_envelope_cols<K, TW, CG>, &lds_done);
    if (le != hipSuccess) return le;
    const int tiles = (W + TW - 1) / TW;
    const int64_t nblocks = (int64_t)B * D * tiles;
    EDT_LAUNCH(tm, kname, s,
               hipLaunchKernelGGL((k_envelope_cols<K, TW, CG>), dim3((unsigned)nblocks), dim3(TW, p.Gp),
                                  p.lds, s, c0, c01, D, H, W, p.Gp, cg));
    return hipSuccess;
}

template <class CG>
static hipError_t launch_cols_any(const uint16_t* c0, int B, int D, int H, int W, const CG& cg,
                                  uint32_t* c01, hipStream_t s, KernelTimer* tm, const char* kname) {
    const ColPlan p = plan_cols(H);
    if (p.K == 64) {
        switch (p.TW) {
            case 32: return launch_cols_t<64, 32>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 16: return launch_cols_t<64, 16>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 8: return launch_cols_t<64, 8>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 4: return launch_cols_t<64, 4>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 2: return launch_cols_t<64, 2>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 1: return launch_cols_t<64, 1>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            default: return hipErrorInvalidValue;
        }
    }
    if (p.K == 16) {
        switch (p.TW) {
            case 8: return launch_cols_t<16, 8>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 16: return launch_cols_t<16, 16>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            case 32: return launch_cols_t<16, 32>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
            default: return launch_cols_t<16, 64>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
        }
    }
    switch (p.TW) {
        case 8: return launch_cols_t<32, 8>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
        case 16: return launch_cols_t<32, 16>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
        case 32: return launch_cols_t<32, 32>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
        default: return launch_cols_t<32, 64>(c0, B, D, H, W, cg, c01, p, s, tm, kname);
    }
}

hipError_t launch_cols_3d(const uint16_t* c0, int B, int D, int H, int W, double s2_0,
                          double s2_1, uint32_t* c01, hipStream_t s, KernelTimer* tm) {
    const double s2[2] = {s2_0, s2_1}, ext[2] = {(double)D, (double)std::max(H - 1, 127)};
    const int k = int_scale_shift(s2, ext, 2);
    if (k >= 0) {
        const int S = 1 << k;
        return launch_cols_any(c0, B, D, H, W, ColL2T<int>{(int)(S * s2_0), (int)(S * s2_1)}, c01, s, tm,
                               "envelope_cols_3d");
    }
    return launch_cols_any(c0, B, D, H, W, ColL2{s2_0, s2_1}, c01, s, tm, "envelope_cols_3d");
}

hipError_t launch_cols_linf_3d(const uint16_t* c0, int B, int D, int H, int W, uint32_t* c01,
                               hipStream_t s, KernelTimer* tm) {
    return launch_cols_any(c0, B, D, H, W, ColLinf{}, c01, s, tm, "chessboard_cols");
}

}  // namespace edt
