// kernels.h -- internal launch interface between the host planner (abi.hip)
// and the gfx950 kernels (kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace edt {

constexpr uint16_t kNone16 = 0xFFFFu;
constexpr uint32_t kNone32 = 0xFFFFFFFFu;
constexpr int kSegRows = 64;   // rows per segment of the axis-0 scan

// Records a HIP event pair around each kernel when non-null (measurement only).
struct KernelTimer {
    static constexpr int kMax = 8;
    hipEvent_t ev[2 * kMax];
    const char* name[kMax];
    int n = 0;         // completed event pairs
    int created = 0;   // event pairs created (destroy all of them)
    int capacity = 0;
    bool ok = true;
    hipError_t begin(const char* kname, hipStream_t s);
    hipError_t end(hipStream_t s);
};

// Launch bracket: optional timing events, then the launch error check.
#define EDT_LAUNCH(tm, kname, stream, ...)                                   \
    do {                                                                     \
        if (tm) { hipError_t e_ = (tm)->begin(kname, stream); if (e_ != hipSuccess) return e_; } \
        __VA_ARGS__;                                                         \
        hipError_t e2_ = hipGetLastError();                                  \
        if (e2_ != hipSuccess) return e2_;                                   \
        if (tm) { hipError_t e_ = (tm)->end(stream); if (e_ != hipSuccess) return e_; } \
    } while (0)

// Axis-0 pass: for every line along axis 0 (B images of n0 x M elements), the
// axis-0 coordinate of the nearest background element on that line (kNone16 if
// the line has none).  first/last: workspace of B * nseg * M uint16 each;
// bits: B * nseg * M uint64 (nseg = ceil(n0 / kSegRows)).  With c0 null only
// the summaries are made (first / last then hold the nearest background row
// strictly below / above each segment when nseg > 1).
hipError_t launch_axis0(const uint8_t* mask, int B, int n0, int64_t M,
                        uint16_t* first, uint16_t* last, uint64_t* bits, uint16_t* c0,
                        hipStream_t s, KernelTimer* tm);

// Envelope pass along the last axis of B 2-D images (lines = rows of length W).
hipError_t launch_rows_2d(const uint16_t* c0, int B, int H, int W, double s2_0, double s2_1,
                          int32_t* sqdist, float* dist, int32_t* indices,
                          hipStream_t s, KernelTimer* tm);

// Envelope pass along axis 1 of B volumes (lines of length H at fixed (d, w));
// writes the packed nearest coordinates (axis0 << 16 | axis1), kNone32 if none.
hipError_t launch_cols_3d(const uint16_t* c0, int B, int D, int H, int W,
                          double s2_0, double s2_1, uint32_t* c01,
                          hipStream_t s, KernelTimer* tm);

// Envelope pass along axis 2 of B volumes (lines of length W) with the epilogue;
// flat indices as int32 (indices) or int64 (indices64), at most one of them.
hipError_t launch_rows_3d(const uint32_t* c01, int B, int D, int H, int W,
                          double s2_0, double s2_1, double s2_2,
                          int32_t* sqdist, float* dist, int32_t* indices, int64_t* indices64,
                          hipStream_t s, KernelTimer* tm);

// Flat per-image indices of `images` images of per_image elements -> per-axis
// coordinates, image-major: coords[b][k][i] (ndim 1..3; n1, n2: the extents of
// axes 1 and 2 of an image, unused beyond ndim).
hipError_t launch_unravel(const int32_t* flat, int64_t images, int64_t per_image, int ndim, int n1,
                          int n2, int32_t* coords, hipStream_t s);

// The transform by its definition (brute force), B images of ndim (1..3)
// extents n[]: list / counts / block_off are workspace (B * elements,
// B and B * brute_list_block_count(elements) int32).
size_t brute_list_block_count(int64_t per);
hipError_t launch_brute(const uint8_t* mask, int B, int ndim, const int* n, const double* s2,
                        int32_t* list, int32_t* counts, int32_t* block_off, int32_t* sqdist,
                        float* dist, int32_t* indices, hipStream_t s);
// Integer metrics of the brute force (the squared one is launch_brute's at
// unit spacing); launch_brute_metric takes the city block or the chessboard.
constexpr int kBruteSquared = 0;
constexpr int kBruteTaxicab = 1;
constexpr int kBruteChessboard = 2;
hipError_t launch_brute_metric(const uint8_t* mask, int B, int ndim, const int* n, int metric,
                               int32_t* list, int32_t* counts, int32_t* block_off, int32_t* dist,
                               int32_t* indices, hipStream_t s);

// City-block (taxicab) transform (chamfer.hip): last-axis pass with int32
// distances / indices for B images or volumes, and the middle-axis pass of
// volumes (packed owners, as launch_cols_3d).
hipError_t launch_l1_rows_2d(const uint16_t* c0, int B, int H, int W, int32_t* dist,
                             int32_t* indices, hipStream_t s, KernelTimer* tm);
hipError_t launch_l1_cols_3d(const uint16_t* c0, int B, int D, int H, int W, uint32_t* c01,
                             hipStream_t s, KernelTimer* tm);
hipError_t launch_l1_rows_3d(const uint32_t* c01, int B, int D, int H, int W, int32_t* dist,
                             int32_t* indices, hipStream_t s, KernelTimer* tm);
// Chessboard (L-infinity) transform (kernels.hip, the envelope kernels under
// the chessboard metric): last axis with int32 distances / indices for B
// images or volumes, and the middle axis of volumes (packed owners, as
// launch_cols_3d).  Lines must fit the kernels' LDS (rows_lds_bytes /
// cols_lds_bytes non-zero).
hipError_t launch_rows_linf_2d(const uint16_t* c0, int B, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm);
hipError_t launch_rows_linf_3d(const uint32_t* c01, int B, int D, int H, int W, int32_t* dist,
                               int32_t* indices, hipStream_t s, KernelTimer* tm);
hipError_t launch_cols_linf_3d(const uint16_t* c0, int B, int D, int H, int W, uint32_t* c01,
                               hipStream_t s, KernelTimer* tm);

// The transform for any spatial rank (nd.hip): nb leading batch axes and nd
// (1..8) spatial axes; ext[] the extents (batch first), mstride[] the mask's
// element strides, s2[] the squared spacings of the spatial axes; B the
// number of images, N the elements per image.  Outputs C-contiguous.
struct NdDesc {
    int nb, nd;
    int64_t ext[16];
    int64_t mstride[16];
    double s2[8];
    int64_t B, N;
};
size_t nd_workspace_bytes(int64_t total);
hipError_t launch_nd(const uint8_t* mask, const NdDesc& d, void* ws, int32_t* sqdist, float* dist,
                     void* indices, int idx_bytes, hipStream_t s);
// Reordered runs (nd.hip): gather the mask of d (1..3 spatial axes) into a
// contiguous [B][permuted image] buffer (permuted axis k = original axis
// perm[k]); put the permuted run's outputs back in the original order
// (pidx: its int32 indices, always; psq / pdist when sqdist / dist are asked
// for; images without background get the original frame's virtual element).
hipError_t launch_nd_gather(const uint8_t* mask, const NdDesc& d, const int* perm, uint8_t* dst, hipStream_t s);
hipError_t launch_nd_unpermute(const NdDesc& d, const int* perm, const int32_t* pidx, const int32_t* psq,
                               const float* pdist, int32_t* sqdist, float* dist, void* indices, int idx_bytes,
                               hipStream_t s);
// Flat per-image indices (int32 or int64) of `images` images of shape
// ext[0..nd) -> per-axis coordinates of the same type, coords[b][k][i].
hipError_t launch_unravel_nd(const void* flat, int idx_bytes, int64_t images, int nd,
                             const int64_t* ext, void* coords, hipStream_t s);

// PR-EDT's row-recursive proximate-point row pass (prox.hip) for B images
// H x W (W <= prox_max_width()), from the axis-0 summary: above / below the
// nearest background row strictly above / below each 64-row segment, bits
// its background rows; tmpF / tmpI: workspace of B * H * W float64 / int32.
hipError_t launch_prox_rows_2d(const uint16_t* above, const uint16_t* below, const uint64_t* bits,
                               int B, int H, int W, double s2r, double s2c, double* tmpF,
                               int32_t* tmpI, int32_t* sqdist, float* dist, int32_t* indices,
                               hipStream_t s, KernelTimer* tm);
size_t prox_lds_bytes();
int prox_max_width();

// Raise a kernel's dynamic-LDS ceiling to the gfx950 LDS size on the current
// device, once per device (done[] holds one bit per device id, set
// atomically; devices past 63 set it on every call).  A failure is not fatal
// here: a launch that really needs more LDS fails on its own.
hipError_t large_lds_once(const void* fn, unsigned long long* done);

// Dynamic LDS each envelope launch needs (0 if the line is too long).
size_t rows_lds_bytes(int L, int value_bytes);
size_t cols_lds_bytes(int H);

}  // namespace edt
