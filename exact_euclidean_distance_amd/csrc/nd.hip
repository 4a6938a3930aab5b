// nd.hip -- the transform for any spatial rank (1..8), strided masks, lines of
// any length and extents beyond 16 bits.
//
// The same separable method as the LDS kernels ("TorchMorph: CUDA-accelerated
// Morphological Transforms", the separable lower-envelope EDT paragraph), with
// its state in the caller's workspace instead of LDS -- TorchMorph's fallback
// for lines too long for on-chip memory, which spills the envelope to a
// global buffer:
//   axis 0   one thread per line along the first spatial axis: the nearest
//            background element above and at-or-below ("GPU-Based Parallel
//            Euclidean Distance Transform Algorithm", §3.2: the upper and lower
//            candidates), the nearer kept (a tie goes to the smaller
//            coordinate); F = s0^2 d^2 and the flat index of that element.
//   axis k   one thread per line along spatial axis k: the lower envelope of
//            the parabolas s_k^2 (q - j)^2 + F_j by the insertion sweep of
//            PR-EDT Algorithm 1 (§3.3.1; a middle member is dropped when the
//            bisectors of its two neighbours cross the line in the wrong
//            order, equality included), then the 1-D Voronoi query of §3.4
//            (the owner advances while the next member is strictly nearer).
// A line's stack of members lives in the workspace slots of the line's own
// elements, so neighbouring threads (neighbouring lines) touch neighbouring
// addresses.  F is float64 and features int64 between passes (exact for
// integer coordinates and dyadic spacings); the last pass writes the outputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace edt {

namespace {

constexpr double kInfF = __builtin_huge_val();

__device__ __forceinline__ void write_out(int64_t e, double F, int64_t feat, int32_t* sqdist, float* dist,
                                          void* indices, int idx_bytes) {
    if (sqdist) sqdist[e] = (int32_t)F;
    if (dist) dist[e] = (float)sqrt(F);
    if (indices) {
        if (idx_bytes == 8) reinterpret_cast<int64_t*>(indices)[e] = feat;
        else reinterpret_cast<int32_t*>(indices)[e] = (int32_t)feat;
    }
}

// The virtual background element (-1, 0, ..., 0) of an image without
// background: F and index at element p (flat within its image).
__device__ __forceinline__ void virtual_at(const NdDesc& d, int64_t p, double* F, int64_t* feat) {
    double f = 0.0;
    int64_t rem = p;
    for (int a = d.nd - 1; a >= 0; --a) {
        const int64_t n = d.ext[d.nb + a];
        const int64_t c = rem % n;
        rem /= n;
        const double t = (double)(a == 0 ? c + 1 : c);
        f += d.s2[a] * t * t;
    }
    *F = f;
    *feat = -(d.N / d.ext[d.nb]);
}

// Mask offset (elements) of line t of the axis-0 pass: t = b * S0 + i, b the
// image (batch axes, row-major), i the index over spatial axes 1.. .
__device__ __forceinline__ int64_t mask_line_offset(const NdDesc& d, int64_t b, int64_t i) {
    int64_t off = 0;
    for (int a = d.nb - 1; a >= 0; --a) {
        off += (b % d.ext[a]) * d.mstride[a];
        b /= d.ext[a];
    }
    for (int a = d.nb + d.nd - 1; a > d.nb; --a) {
        off += (i % d.ext[a]) * d.mstride[a];
        i /= d.ext[a];
    }
    return off;
}

__global__ __launch_bounds__(256) void k_nd_axis0(const uint8_t* __restrict__ mask, NdDesc d,
                                                  double* __restrict__ F, int64_t* __restrict__ feat,
                                                  int final_pass, int32_t* __restrict__ sqdist,
                                                  float* __restrict__ dist, void* __restrict__ indices,
                                                  int idx_bytes) {
    const int64_t n0 = d.ext[d.nb];
    const int64_t S0 = d.N / n0;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= d.B * S0) return;
    const int64_t b = t / S0, i = t - b * S0;
    const uint8_t* m = mask + mask_line_offset(d, b, i);
    const int64_t st = d.mstride[d.nb];
    const int64_t e0 = b * d.N + i;   // element j of the line: e0 + j * S0
    // forward: the last background at or above j (kept in the feature slots)
    int64_t last = -1;
    for (int64_t j = 0; j < n0; ++j) {
        if (m[j * st] == 0) last = j;
        feat[e0 + j * S0] = last;
    }
    // backward: the first background at or below j; the nearer of the two
    int64_t next = -1;
    const double s2 = d.s2[0];
    for (int64_t j = n0 - 1; j >= 0; --j) {
        const int64_t e = e0 + j * S0;
        const int64_t up = feat[e];
        if (up == j) next = j;
        int64_t c;
        if (up < 0) c = next;
        else if (next < 0) c = up;
        else c = (j - up <= next - j) ? up : next;
        double f;
        int64_t ft;
        if (c < 0) {
            f = kInfF;
            ft = -1;
        } else {
            const double dd = (double)(j - c);
            f = s2 * dd * dd;
            ft = c * S0 + i;
        }
        if (final_pass) {
            if (c < 0) virtual_at(d, e - b * d.N, &f, &ft);
            write_out(e, f, ft, sqdist, dist, indices, idx_bytes);
        } else {
            F[e] = f;
            feat[e] = ft;
        }
    }
}

// The same pass for few long lines, in segments of kNdSeg positions so that
// the GPU has work (few lines of at least 4 segments: fewer than 16384 lines):
// per (segment, line) the first and last background in the
// segment; per line, over its segments, the last background strictly before
// and the first strictly after each segment; then each segment resolved from
// those carries.  Thread u takes line u % lines of segment u / lines.
constexpr int64_t kNdSeg = 64;

__global__ __launch_bounds__(256) void k_nd_axis0_seg_summary(const uint8_t* __restrict__ mask, NdDesc d,
                                                              int64_t nseg, int64_t* __restrict__ sfirst,
                                                              int64_t* __restrict__ slast) {
    const int64_t n0 = d.ext[d.nb];
    const int64_t S0 = d.N / n0, lines = d.B * S0;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= lines * nseg) return;
    const int64_t t = u % lines, sg = u / lines;
    const int64_t b = t / S0, i = t - b * S0;
    const uint8_t* m = mask + mask_line_offset(d, b, i);
    const int64_t st = d.mstride[d.nb];
    const int64_t j0 = sg * kNdSeg, j1 = min(n0, j0 + kNdSeg);
    int64_t f = -1, l = -1;
    for (int64_t j = j0; j < j1; ++j) {
        if (m[j * st] == 0) {
            if (f < 0) f = j;
            l = j;
        }
    }
    sfirst[u] = f;
    slast[u] = l;
}

// per line (one block of kNdScanThreads each): above[sg * lines + t] = the
// last background before segment sg, below[...] = the first after it (-1:
// none), written in place of slast / sfirst.  Each thread takes a run of
// consecutive segments; the block scans the runs' totals (prefix maximum of
// the last, suffix minimum of the first), then each thread sweeps its run.
constexpr int kNdScanThreads = 1024;
constexpr int64_t kNdNoFirst = INT64_MAX;

__global__ __launch_bounds__(kNdScanThreads) void k_nd_axis0_seg_scan(NdDesc d, int64_t nseg,
                                                                       int64_t* __restrict__ sfirst,
                                                                       int64_t* __restrict__ slast) {
    __shared__ int64_t pmax[kNdScanThreads];
    __shared__ int64_t smin[kNdScanThreads];
    const int64_t lines = d.B * (d.N / d.ext[d.nb]);
    const int64_t t = blockIdx.x;
    const int k = threadIdx.x;
    const int64_t run = (nseg + kNdScanThreads - 1) / kNdScanThreads;
    const int64_t s0 = min(nseg, (int64_t)k * run), s1 = min(nseg, s0 + run);
    int64_t lmax = -1, fmin = kNdNoFirst;
    for (int64_t sg = s0; sg < s1; ++sg) {
        const int64_t l = slast[sg * lines + t], f = sfirst[sg * lines + t];
        if (l > lmax) lmax = l;
        if (f >= 0 && f < fmin) fmin = f;
    }
    pmax[k] = lmax;
    smin[k] = fmin;
    __syncthreads();
    for (int o = 1; o < kNdScanThreads; o <<= 1) {   // inclusive scans over the runs
        const int64_t a = k >= o ? pmax[k - o] : -1;
        const int64_t b = k + o < kNdScanThreads ? smin[k + o] : kNdNoFirst;
        __syncthreads();
        if (a > pmax[k]) pmax[k] = a;
        if (b < smin[k]) smin[k] = b;
        __syncthreads();
    }
    int64_t above = k > 0 ? pmax[k - 1] : -1;   // from the runs before / after this one
    int64_t below = k + 1 < kNdScanThreads ? smin[k + 1] : kNdNoFirst;
    for (int64_t sg = s0; sg < s1; ++sg) {
        const int64_t l = slast[sg * lines + t];
        slast[sg * lines + t] = above;
        if (l >= 0) above = l;
    }
    for (int64_t sg = s1 - 1; sg >= s0; --sg) {
        const int64_t f = sfirst[sg * lines + t];
        sfirst[sg * lines + t] = below == kNdNoFirst ? -1 : below;
        if (f >= 0) below = f;
    }
}

__global__ __launch_bounds__(256) void k_nd_axis0_seg_resolve(const uint8_t* __restrict__ mask, NdDesc d,
                                                              int64_t nseg, const int64_t* __restrict__ below,
                                                              const int64_t* __restrict__ above,
                                                              double* __restrict__ F, int64_t* __restrict__ feat,
                                                              int final_pass, int32_t* __restrict__ sqdist,
                                                              float* __restrict__ dist, void* __restrict__ indices,
                                                              int idx_bytes) {
    const int64_t n0 = d.ext[d.nb];
    const int64_t S0 = d.N / n0, lines = d.B * S0;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= lines * nseg) return;
    const int64_t t = u % lines, sg = u / lines;
    const int64_t b = t / S0, i = t - b * S0;
    const uint8_t* m = mask + mask_line_offset(d, b, i);
    const int64_t st = d.mstride[d.nb];
    const int64_t e0 = b * d.N + i;
    const int64_t j0 = sg * kNdSeg, j1 = min(n0, j0 + kNdSeg);
    int64_t last = above[u];   // forward: the last background at or above j
    for (int64_t j = j0; j < j1; ++j) {
        if (m[j * st] == 0) last = j;
        feat[e0 + j * S0] = last;
    }
    int64_t next = below[u];   // backward: the first background at or below j
    const double s2 = d.s2[0];
    for (int64_t j = j1 - 1; j >= j0; --j) {
        const int64_t e = e0 + j * S0;
        const int64_t up = feat[e];
        if (up == j) next = j;
        int64_t c;
        if (up < 0) c = next;
        else if (next < 0) c = up;
        else c = (j - up <= next - j) ? up : next;
        double f;
        int64_t ft;
        if (c < 0) {
            f = kInfF;
            ft = -1;
        } else {
            const double dd = (double)(j - c);
            f = s2 * dd * dd;
            ft = c * S0 + i;
        }
        if (final_pass) {
            if (c < 0) virtual_at(d, e - b * d.N, &f, &ft);
            write_out(e, f, ft, sqdist, dist, indices, idx_bytes);
        } else {
            F[e] = f;
            feat[e] = ft;
        }
    }
}

// b between a and c leaves the envelope (equality included)
__device__ __forceinline__ bool nd_dominated(int64_t a, double Ya, int64_t b, double Yb, int64_t c, double Yc) {
    return (Yb - Ya) * (double)(c - b) >= (Yc - Yb) * (double)(b - a);
}

__global__ __launch_bounds__(256) void k_nd_envelope(const double* __restrict__ Fin,
                                                     const int64_t* __restrict__ fin,
                                                     double* __restrict__ Fout,
                                                     int64_t* __restrict__ fout,
                                                     int64_t* __restrict__ stk, NdDesc d, int k,
                                                     int final_pass, int32_t* __restrict__ sqdist,
                                                     float* __restrict__ dist,
                                                     void* __restrict__ indices, int idx_bytes) {
    const int64_t nk = d.ext[d.nb + k];
    int64_t Sk = 1;
    for (int a = k + 1; a < d.nd; ++a) Sk *= d.ext[d.nb + a];
    const int64_t lines = d.B * (d.N / nk);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= lines) return;
    const int64_t o = t / Sk, i = t - o * Sk;
    const int64_t base = o * nk * Sk + i;   // element j: base + j * Sk
    const double s2 = d.s2[k];
    auto Fat = [&](int64_t j) { return Fin[base + j * Sk]; };
    auto Yat = [&](int64_t j) { return Fat(j) + s2 * (double)j * (double)j; };
    // 1. envelope: members in stk[base + m * Sk], m = 0 .. n-1
    int64_t n = 0, top = -1, sec = -1;
    double Ytop = 0.0, Ysec = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const double Fj = Fat(j);
        if (!(Fj < kInfF)) continue;
        const double Y = Fj + s2 * (double)j * (double)j;
        while (n >= 2 && nd_dominated(sec, Ysec, top, Ytop, j, Y)) {
            --n;
            top = sec;
            Ytop = Ysec;
            if (n >= 2) {
                sec = stk[base + (n - 2) * Sk];
                Ysec = Yat(sec);
            }
        }
        stk[base + n * Sk] = j;
        ++n;
        sec = top;
        Ysec = Ytop;
        top = j;
        Ytop = Y;
    }
    // 2. query
    int64_t m = 0, cur = n > 0 ? stk[base] : -1, nxt = n > 1 ? stk[base + Sk] : -1;
    double Fc = cur >= 0 ? Fat(cur) : kInfF, Fn = nxt >= 0 ? Fat(nxt) : kInfF;
    for (int64_t q = 0; q < nk; ++q) {
        while (m + 1 < n) {
            const double dc = (double)(q - cur), dn = (double)(q - nxt);
            if (!(Fn + s2 * dn * dn < Fc + s2 * dc * dc)) break;
            ++m;
            cur = nxt;
            Fc = Fn;
            if (m + 1 < n) {
                nxt = stk[base + (m + 1) * Sk];
                Fn = Fat(nxt);
            }
        }
        const int64_t e = base + q * Sk;
        double f = kInfF;
        int64_t ft = -1;
        if (cur >= 0) {
            const double dq = (double)(q - cur);
            f = Fc + s2 * dq * dq;
            ft = fin[base + cur * Sk];
        }
        if (final_pass) {
            if (cur < 0) virtual_at(d, e % d.N, &f, &ft);
            write_out(e, f, ft, sqdist, dist, indices, idx_bytes);
        } else {
            Fout[e] = f;
            fout[e] = ft;
        }
    }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

struct Ext8 {
    int64_t n[8];
};

template <class Ix>
__global__ __launch_bounds__(256) void k_unravel_nd(const Ix* __restrict__ flat, int64_t total,
                                                    int64_t per_image, int nd, Ext8 ext,
                                                    Ix* __restrict__ coords) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t b = e / per_image;
    const int64_t i = e - b * per_image;
    int64_t f = (int64_t)flat[e];
    int64_t c[8];
    // floor division, so that the virtual element -(n1 * ... ) becomes (-1, 0, ...)
    for (int k = nd - 1; k >= 1; --k) {
        int64_t q = f / ext.n[k], r = f - q * ext.n[k];
        if (r < 0) {
            r += ext.n[k];
            --q;
        }
        c[k] = r;
        f = q;
    }
    c[0] = f;
    Ix* dst = coords + b * (int64_t)nd * per_image + i;
    for (int k = 0; k < nd; ++k) dst[(int64_t)k * per_image] = (Ix)c[k];
}

}  // namespace

hipError_t launch_unravel_nd(const void* flat, int idx_bytes, int64_t images, int nd,
                             const int64_t* ext, void* coords, hipStream_t s) {
    int64_t per = 1;
    Ext8 e{};
    for (int k = 0; k < nd; ++k) {
        e.n[k] = ext[k];
        per *= ext[k];
    }
    const int64_t total = images * per;
    if (total == 0) return hipSuccess;
    if (idx_bytes == 8)
        hipLaunchKernelGGL(k_unravel_nd<int64_t>, dim3(blocks_for(total)), dim3(256), 0, s,
                           static_cast<const int64_t*>(flat), total, per, nd, e, static_cast<int64_t*>(coords));
    else
        hipLaunchKernelGGL(k_unravel_nd<int32_t>, dim3(blocks_for(total)), dim3(256), 0, s,
                           static_cast<const int32_t*>(flat), total, per, nd, e, static_cast<int32_t*>(coords));
    return hipGetLastError();
}

// workspace: F (2 x float64) and features (2 x int64) per element for the
// ping-pong between passes, and the members' positions (int64) per element
// ---------------------------------------------------------------------------
// Reordered runs of the LDS kernels.  The transform is separable, so its
// result does not depend on the order in which the axes are taken: a 1-, 2- or
// 3-D image the LDS kernels refuse as laid out (a strided mask, rows too long
// for them) is gathered into a contiguous buffer with its spatial axes in
// another order (perm: permuted axis k is original axis perm[k]), transformed
// there with the spacings reordered alike, and the outputs are put back in
// the original order.  An image without background used the virtual element
// (-1, 0, ...) of the permuted axis 0, so its outputs are recomputed in the
// original frame (the virtual element on the original axis 0).
// ---------------------------------------------------------------------------

namespace {

struct PermDesc {
    int nd;
    int perm[3];
    int64_t pext[3];   // extents in permuted order
};

// original coordinates of the element with flat index r of one image (row-major)
__device__ __forceinline__ void unravel3(const NdDesc& d, int64_t r, int64_t oc[3]) {
    for (int a = d.nd - 1; a >= 0; --a) {
        const int64_t n = d.ext[d.nb + a];
        oc[a] = r % n;
        r /= n;
    }
}

}  // namespace

// dst[b][permuted image] = mask at the original coordinates; one thread per element
__global__ __launch_bounds__(256) void k_nd_gather(const uint8_t* __restrict__ mask, NdDesc d, PermDesc pd,
                                                   uint8_t* __restrict__ dst) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= d.B * d.N) return;
    const int64_t b = e / d.N;
    int64_t r = e - b * d.N;
    int64_t oc[3] = {0, 0, 0};
    for (int k = pd.nd - 1; k >= 0; --k) {   // permuted coordinates -> original axes
        oc[pd.perm[k]] = r % pd.pext[k];
        r /= pd.pext[k];
    }
    int64_t off = 0, bb = b;
    for (int a = d.nb - 1; a >= 0; --a) {
        off += (bb % d.ext[a]) * d.mstride[a];
        bb /= d.ext[a];
    }
    for (int a = 0; a < pd.nd; ++a) off += oc[a] * d.mstride[d.nb + a];
    dst[e] = mask[off];
}

// Outputs in the original order from the permuted run's int32 index (always)
// and sqdist / dist (when asked for); one thread per output element.
__global__ __launch_bounds__(256) void k_nd_unpermute(NdDesc d, PermDesc pd, const int32_t* __restrict__ pidx,
                                                      const int32_t* __restrict__ psq,
                                                      const float* __restrict__ pdist,
                                                      int32_t* __restrict__ sqdist, float* __restrict__ dist,
                                                      void* __restrict__ indices, int idx_bytes) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= d.B * d.N) return;
    const int64_t b = e / d.N, r = e - b * d.N;
    int64_t oc[3] = {0, 0, 0};
    unravel3(d, r, oc);
    int64_t pr = 0;   // flat index of the same element in the permuted image
    for (int k = 0; k < pd.nd; ++k) pr = pr * pd.pext[k] + oc[pd.perm[k]];
    const int64_t pe = b * d.N + pr;
    const int32_t pi = pidx[pe];
    if (pi < 0) {   // no background in the image: the virtual element of the original axis 0
        double f;
        int64_t ft;
        virtual_at(d, r, &f, &ft);
        write_out(e, f, ft, sqdist, dist, indices, idx_bytes);
        return;
    }
    if (sqdist) sqdist[e] = psq[pe];
    if (dist) dist[e] = pdist[pe];
    if (indices) {
        int64_t q = pi, pc[3] = {0, 0, 0};
        for (int k = pd.nd - 1; k >= 0; --k) {
            pc[k] = q % pd.pext[k];
            q /= pd.pext[k];
        }
        int64_t oo[3] = {0, 0, 0};
        for (int k = 0; k < pd.nd; ++k) oo[pd.perm[k]] = pc[k];
        int64_t flat = 0;
        for (int a = 0; a < pd.nd; ++a) flat = flat * d.ext[d.nb + a] + oo[a];
        if (idx_bytes == 8) reinterpret_cast<int64_t*>(indices)[e] = flat;
        else reinterpret_cast<int32_t*>(indices)[e] = (int32_t)flat;
    }
}

hipError_t launch_nd_gather(const uint8_t* mask, const NdDesc& d, const int* perm, uint8_t* dst, hipStream_t s) {
    PermDesc pd{};
    pd.nd = d.nd;
    for (int k = 0; k < d.nd; ++k) {
        pd.perm[k] = perm[k];
        pd.pext[k] = d.ext[d.nb + perm[k]];
    }
    const int64_t total = d.B * d.N;
    hipLaunchKernelGGL(k_nd_gather, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, mask, d, pd, dst);
    return hipGetLastError();
}

hipError_t launch_nd_unpermute(const NdDesc& d, const int* perm, const int32_t* pidx, const int32_t* psq,
                               const float* pdist, int32_t* sqdist, float* dist, void* indices, int idx_bytes,
                               hipStream_t s) {
    PermDesc pd{};
    pd.nd = d.nd;
    for (int k = 0; k < d.nd; ++k) {
        pd.perm[k] = perm[k];
        pd.pext[k] = d.ext[d.nb + perm[k]];
    }
    const int64_t total = d.B * d.N;
    hipLaunchKernelGGL(k_nd_unpermute, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, d, pd, pidx, psq,
                       pdist, sqdist, dist, indices, idx_bytes);
    return hipGetLastError();
}

size_t nd_workspace_bytes(int64_t total) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    return 2 * al((size_t)total * 8) + 2 * al((size_t)total * 8) + al((size_t)total * 8);
}

hipError_t launch_nd(const uint8_t* mask, const NdDesc& d, void* ws, int32_t* sqdist, float* dist,
                     void* indices, int idx_bytes, hipStream_t s) {
    const int64_t total = d.B * d.N;
    if (total == 0) return hipSuccess;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    char* p = static_cast<char*>(ws);
    double* F[2] = {reinterpret_cast<double*>(p), reinterpret_cast<double*>(p + al((size_t)total * 8))};
    p += 2 * al((size_t)total * 8);
    int64_t* feat[2] = {reinterpret_cast<int64_t*>(p), reinterpret_cast<int64_t*>(p + al((size_t)total * 8))};
    p += 2 * al((size_t)total * 8);
    int64_t* stk = reinterpret_cast<int64_t*>(p);
    const int64_t S0 = d.N / d.ext[d.nb];
    const int64_t lines0 = d.B * S0, n0 = d.ext[d.nb];
    hipError_t e;
    if (lines0 < 16384 && n0 >= 4 * kNdSeg) {
        // few long lines: segments; the summaries use the stack region, idle
        // until the envelope passes (4 * nseg * lines0 <= total words)
        const int64_t nseg = (n0 + kNdSeg - 1) / kNdSeg;
        int64_t* sfirst = stk;
        int64_t* slast = stk + nseg * lines0;
        hipLaunchKernelGGL(k_nd_axis0_seg_summary, dim3(blocks_for(nseg * lines0)), dim3(256), 0, s, mask, d, nseg,
                           sfirst, slast);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_nd_axis0_seg_scan, dim3((unsigned)lines0), dim3(kNdScanThreads), 0, s, d, nseg, sfirst,
                           slast);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_nd_axis0_seg_resolve, dim3(blocks_for(nseg * lines0)), dim3(256), 0, s, mask, d, nseg,
                           sfirst, slast, F[0], feat[0], d.nd == 1 ? 1 : 0, sqdist, dist, indices, idx_bytes);
    } else {
        hipLaunchKernelGGL(k_nd_axis0, dim3(blocks_for(d.B * S0)), dim3(256), 0, s, mask, d, F[0], feat[0],
                           d.nd == 1 ? 1 : 0, sqdist, dist, indices, idx_bytes);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    int cur = 0;
    for (int k = 1; k < d.nd; ++k) {
        const int64_t lines = d.B * (d.N / d.ext[d.nb + k]);
        const int fin = k == d.nd - 1;
        hipLaunchKernelGGL(k_nd_envelope, dim3(blocks_for(lines)), dim3(256), 0, s, F[cur], feat[cur],
                           F[1 - cur], feat[1 - cur], stk, d, k, fin, sqdist, dist, indices, idx_bytes);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        cur = 1 - cur;
    }
    return hipSuccess;
}

}  // namespace edt
