// abi.hip -- host planner and C ABI of libedt_mi355x.so (declared in include/edt.h).
//
// Argument conventions are resolved here and only here (as TorchMorph keeps
// argument handling in one validation layer); every check runs before the
// first HIP call, so a rejected call touches no buffer.  The planner carves
// the caller's workspace and enqueues the passes on the caller's stream:
//   2-D:  axis-0 scan (3 kernels) -> row envelope + epilogue (B images at once;
//         a 1-D line of n elements is an n x 1 image)
//   3-D:  axis-0 scan (3 kernels) -> axis-1 envelope -> axis-2 envelope + epilogue
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/edt.h"
#include "kernels.h"

namespace {

constexpr int32_t kMaxExtent = 65535;
constexpr int32_t kMaxW2D = 32768;
constexpr int32_t kMaxH3D = 32768;
constexpr int32_t kMaxW3D = 16384;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t c0 = 0, c01 = 0, first = 0, last = 0, bits = 0, total = 0;
};

bool shape2d_ok(int32_t B, int32_t H, int32_t W) {
    if (B < 1 || H < 1 || W < 1 || B > kMaxExtent || H > kMaxExtent || W > kMaxExtent) return false;
    if (W > kMaxW2D) return false;
    if ((int64_t)H * W > INT32_MAX) return false;
    return edt::rows_lds_bytes(W, 2) != 0;
}

// Volumes over 2^31 - 1 elements are accepted here (offsets are 64-bit
// throughout); only their int32 flat indices cannot be returned (run3d).
bool shape3d_ok(int32_t B, int32_t D, int32_t H, int32_t W) {
    if (B < 1 || D < 1 || H < 1 || W < 1) return false;
    if (B > kMaxExtent || D > kMaxExtent || H > kMaxExtent || W > kMaxExtent) return false;
    if (H > kMaxH3D || W > kMaxW3D) return false;
    if (H > 1 && edt::cols_lds_bytes(H) == 0) return false;
    return edt::rows_lds_bytes(W, 4) != 0;
}

Layout layout2d(int32_t B, int32_t H, int32_t W) {
    Layout L;
    const size_t n = (size_t)B * H * W;
    const size_t nseg = (size_t)B * ((H + edt::kSegRows - 1) / edt::kSegRows);
    L.c0 = 0;
    L.first = round_up(n * 2);
    L.last = L.first + round_up(nseg * W * 2);
    L.bits = L.last + round_up(nseg * W * 2);
    L.total = L.bits + round_up(nseg * W * 8);
    return L;
}

Layout layout3d(int32_t B, int32_t D, int32_t H, int32_t W) {
    Layout L;
    const size_t n = (size_t)B * D * H * W;
    const size_t nseg = (size_t)(D + edt::kSegRows - 1) / edt::kSegRows;
    const size_t summ = (size_t)B * nseg * H * W * 2;
    L.c0 = 0;
    L.c01 = round_up(n * 2);
    L.first = L.c01 + round_up(n * 4);
    L.last = L.first + round_up(summ);
    L.bits = L.last + round_up(summ);
    L.total = L.bits + round_up(summ * 4);
    return L;
}

// Returns EDT_OK and the squared spacings, or the error for bad spacing.
edt_status read_sampling(const float* sampling, int ndim, double* s2, bool* unit) {
    *unit = true;
    for (int k = 0; k < ndim; ++k) {
        double s = 1.0;
        if (sampling) {
            const float f = sampling[k];
            if (!(f > 0.0f) || !isfinite(f)) return EDT_ERR_INVALID_ARGUMENT;
            s = (double)f;
        }
        if (s != 1.0) *unit = false;
        s2[k] = s * s;
    }
    return EDT_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Common checks on outputs and workspace; n = total element count.
// indices: int32 (idx_bytes 4) or int64 (idx_bytes 8) per element.
// check_ws false: the workspace is the library's own scratch, not checked here.
edt_status check_buffers(const uint8_t* mask, size_t n, int32_t* sqdist, float* dist,
                         void* indices, void* ws, size_t ws_bytes, size_t ws_need,
                         size_t idx_bytes = 4, bool check_ws = true) {
    if (!mask) return EDT_ERR_INVALID_ARGUMENT;
    if (!sqdist && !dist && !indices) return EDT_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)sqdist & 3) || ((uintptr_t)dist & 3) || ((uintptr_t)indices & (idx_bytes - 1)))
        return EDT_ERR_INVALID_ARGUMENT;
    if (!check_ws) {
        ws = nullptr;
        ws_need = 0;
    } else {
        if (!ws || ((uintptr_t)ws & (kAlign - 1))) return EDT_ERR_INVALID_ARGUMENT;
        if (ws_bytes < ws_need) return EDT_ERR_WORKSPACE_TOO_SMALL;
    }
    const void* bufs[5] = {mask, sqdist, dist, indices, ws};
    const size_t sizes[5] = {n, sqdist ? n * 4 : 0, dist ? n * 4 : 0, indices ? n * idx_bytes : 0, ws_need};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(bufs[i], sizes[i], bufs[j], sizes[j])) return EDT_ERR_INVALID_ARGUMENT;
    return EDT_OK;
}

// Workspace of edt2d_u8_batched_noalloc, for callers that cannot allocate:
// one copy per device, held from the first use until the process ends.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (nullptr on a HIP error).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// use_scratch: the workspace is this device's copy of `scratch` (ws and
// ws_bytes are ignored); it is looked up only after every argument check.
edt_status run2d(const uint8_t* mask, int32_t B, int32_t H, int32_t W, const float* sampling,
                 int32_t* sqdist, float* dist, int32_t* indices, void* ws, size_t ws_bytes,
                 hipStream_t stream, edt::KernelTimer* tm, bool use_scratch = false) {
    if (B < 1 || H < 1 || W < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (!shape2d_ok(B, H, W)) return EDT_ERR_UNSUPPORTED_SHAPE;
    double s2[2];
    bool unit;
    edt_status st = read_sampling(sampling, 2, s2, &unit);
    if (st != EDT_OK) return st;
    if (sqdist && !unit) return EDT_ERR_INVALID_ARGUMENT;
    if (sqdist && (double)H * H + (double)W * W > (double)INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    const Layout L = layout2d(B, H, W);
    if (use_scratch && L.total > kScratchBytes) return EDT_ERR_WORKSPACE_TOO_SMALL;
    st = check_buffers(mask, (size_t)B * H * W, sqdist, dist, indices, ws, ws_bytes, L.total, 4,
                       !use_scratch);
    if (st != EDT_OK) return st;
    if (use_scratch) {   // the first HIP calls of this entry point
        ws = scratch_address();
        if (!ws) return EDT_ERR_HIP;
    }

    char* base = static_cast<char*>(ws);
    uint16_t* c0 = reinterpret_cast<uint16_t*>(base + L.c0);
    uint16_t* first = reinterpret_cast<uint16_t*>(base + L.first);
    uint16_t* last = reinterpret_cast<uint16_t*>(base + L.last);
    uint64_t* bits = reinterpret_cast<uint64_t*>(base + L.bits);
    if (edt::launch_axis0(mask, B, H, W, first, last, bits, c0, stream, tm) != hipSuccess) return EDT_ERR_HIP;
    if (edt::launch_rows_2d(c0, B, H, W, s2[0], s2[1], sqdist, dist, indices, stream, tm) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

// PR-EDT's row-recursive pass: the axis-0 summaries, then the proximate-point
// sets of each 64-row sub-block; workspace = summaries + each pixel's upper
// answer (float64 + int32).
bool prox_shape_ok(int32_t B, int32_t H, int32_t W) {
    if (B < 1 || H < 1 || W < 1 || B > kMaxExtent || H > kMaxExtent) return false;
    if (W > edt::prox_max_width()) return false;
    return (int64_t)H * W <= INT32_MAX;
}

size_t prox_workspace(int32_t B, int32_t H, int32_t W, size_t* off_f, size_t* off_i) {
    const Layout L = layout2d(B, H, W);
    const size_t n = (size_t)B * H * W;
    const size_t summ = L.total - L.first;   // first, last, bits (no c0)
    *off_f = round_up(summ);
    *off_i = *off_f + round_up(n * 8);
    return *off_i + round_up(n * 4);
}

edt_status run_prox2d(const uint8_t* mask, int32_t B, int32_t H, int32_t W, const float* sampling,
                      int32_t* sqdist, float* dist, int32_t* indices, void* ws, size_t ws_bytes,
                      hipStream_t stream, edt::KernelTimer* tm) {
    if (B < 1 || H < 1 || W < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (!prox_shape_ok(B, H, W)) return EDT_ERR_UNSUPPORTED_SHAPE;
    double s2[2];
    bool unit;
    edt_status st = read_sampling(sampling, 2, s2, &unit);
    if (st != EDT_OK) return st;
    if (sqdist && !unit) return EDT_ERR_INVALID_ARGUMENT;
    if (sqdist && (double)H * H + (double)W * W > (double)INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    size_t off_f, off_i;
    const size_t need = prox_workspace(B, H, W, &off_f, &off_i);
    st = check_buffers(mask, (size_t)B * H * W, sqdist, dist, indices, ws, ws_bytes, need);
    if (st != EDT_OK) return st;
    const Layout L = layout2d(B, H, W);
    char* base = static_cast<char*>(ws);
    // the summaries at the front of the workspace (the same relative layout
    // as the separable path's, without its per-pixel coordinates)
    uint16_t* first = reinterpret_cast<uint16_t*>(base);
    uint16_t* last = reinterpret_cast<uint16_t*>(base + (L.last - L.first));
    uint64_t* bits = reinterpret_cast<uint64_t*>(base + (L.bits - L.first));
    if (edt::launch_axis0(mask, B, H, W, first, last, bits, nullptr, stream, tm) != hipSuccess)
        return EDT_ERR_HIP;
    if (edt::launch_prox_rows_2d(last, first, bits, B, H, W, s2[0], s2[1],
                                 reinterpret_cast<double*>(base + off_f),
                                 reinterpret_cast<int32_t*>(base + off_i), sqdist, dist, indices, stream,
                                 tm) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

edt_status run3d(const uint8_t* mask, int32_t B, int32_t D, int32_t H, int32_t W,
                 const float* sampling, int32_t* sqdist, float* dist, int32_t* indices,
                 void* ws, size_t ws_bytes, hipStream_t stream, edt::KernelTimer* tm,
                 int64_t* indices64 = nullptr) {
    if (B < 1 || D < 1 || H < 1 || W < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (!shape3d_ok(B, D, H, W)) return EDT_ERR_UNSUPPORTED_SHAPE;
    double s2[3];
    bool unit;
    edt_status st = read_sampling(sampling, 3, s2, &unit);
    if (st != EDT_OK) return st;
    if (sqdist && !unit) return EDT_ERR_INVALID_ARGUMENT;
    if (sqdist && (double)D * D + (double)H * H + (double)W * W > (double)INT32_MAX)
        return EDT_ERR_UNSUPPORTED_SHAPE;
    if (indices && (int64_t)D * H * W > INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    const Layout L = layout3d(B, D, H, W);
    st = indices64 ? check_buffers(mask, (size_t)B * D * H * W, sqdist, dist, indices64, ws, ws_bytes,
                                   L.total, 8)
                   : check_buffers(mask, (size_t)B * D * H * W, sqdist, dist, indices, ws, ws_bytes,
                                   L.total);
    if (st != EDT_OK) return st;

    char* base = static_cast<char*>(ws);
    uint16_t* c0 = reinterpret_cast<uint16_t*>(base + L.c0);
    uint32_t* c01 = reinterpret_cast<uint32_t*>(base + L.c01);
    uint16_t* first = reinterpret_cast<uint16_t*>(base + L.first);
    uint16_t* last = reinterpret_cast<uint16_t*>(base + L.last);
    uint64_t* bits = reinterpret_cast<uint64_t*>(base + L.bits);
    if (edt::launch_axis0(mask, B, D, (int64_t)H * W, first, last, bits, c0, stream, tm) != hipSuccess)
        return EDT_ERR_HIP;
    if (edt::launch_cols_3d(c0, B, D, H, W, s2[0], s2[1], c01, stream, tm) != hipSuccess)
        return EDT_ERR_HIP;
    if (edt::launch_rows_3d(c01, B, D, H, W, s2[0], s2[1], s2[2], sqdist, dist, indices, indices64,
                            stream, tm) !=
        hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

bool brute_shape_ok(int32_t B, int32_t ndim, const int32_t* shape, int64_t* per) {
    if (!shape || ndim < 1 || ndim > 3 || B < 1 || B > kMaxExtent) return false;
    int64_t p = 1;
    for (int k = 0; k < ndim; ++k) {
        if (shape[k] < 1 || shape[k] > kMaxExtent) return false;
        p *= shape[k];
    }
    if (p > INT32_MAX) return false;
    *per = p;
    return true;
}

// Workspace of the brute force: the background list, the per-image counts
// and the per-block offsets of the list kernels.
struct BruteLayout {
    size_t list, counts, block_off, total;
};
BruteLayout brute_layout(int32_t B, int64_t per) {
    BruteLayout L{};
    L.list = 0;
    L.counts = round_up((size_t)B * (size_t)per * 4);
    L.block_off = L.counts + round_up((size_t)B * 4);
    L.total = L.block_off + round_up((size_t)B * edt::brute_list_block_count(per) * 4);
    return L;
}

edt_status finish_timed(edt_status st, edt::KernelTimer& tm, hipStream_t stream, float* kernel_ms,
                        const char** kernel_names, int32_t* count) {
    if (st == EDT_OK && hipStreamSynchronize(stream) != hipSuccess) st = EDT_ERR_HIP;
    for (int i = 0; i < tm.n; ++i) {
        float ms = 0.0f;
        if (st == EDT_OK && hipEventElapsedTime(&ms, tm.ev[2 * i], tm.ev[2 * i + 1]) != hipSuccess)
            st = EDT_ERR_HIP;
        if (st == EDT_OK) {
            kernel_ms[i] = ms;
            if (kernel_names) kernel_names[i] = tm.name[i];
        }
    }
    for (int i = 0; i < tm.created; ++i) {
        (void)hipEventDestroy(tm.ev[2 * i]);
        (void)hipEventDestroy(tm.ev[2 * i + 1]);
    }
    if (st == EDT_OK && !tm.ok) st = EDT_ERR_INVALID_ARGUMENT;
    if (count) *count = (st == EDT_OK) ? tm.n : 0;
    return st;
}

}  // namespace

extern "C" {

size_t edt2d_workspace_size(int32_t H, int32_t W) {
    return edt2d_batched_workspace_size(1, H, W);
}

size_t edt2d_batched_workspace_size(int32_t B, int32_t H, int32_t W) {
    if (!shape2d_ok(B, H, W)) return 0;
    return layout2d(B, H, W).total;
}

size_t edt1d_workspace_size(int32_t B, int32_t N) {
    return edt2d_batched_workspace_size(B, N, 1);
}

size_t edt3d_workspace_size(int32_t B, int32_t D, int32_t H, int32_t W) {
    if (!shape3d_ok(B, D, H, W)) return 0;
    return layout3d(B, D, H, W).total;
}

edt_status edt2d_u8(const uint8_t* mask, int32_t H, int32_t W, const float* sampling,
                    int32_t* sqdist, float* dist, int32_t* indices, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    return run2d(mask, 1, H, W, sampling, sqdist, dist, indices, workspace, workspace_bytes, stream,
                 nullptr);
}

edt_status edt2d_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                            const float* sampling, int32_t* sqdist, float* dist, int32_t* indices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return run2d(mask, B, H, W, sampling, sqdist, dist, indices, workspace, workspace_bytes, stream,
                 nullptr);
}

size_t edt2d_noalloc_max_workspace(void) { return kScratchBytes; }

size_t edt2d_proximate_workspace_size(int32_t B, int32_t H, int32_t W) {
    if (!prox_shape_ok(B, H, W)) return 0;
    size_t a, b;
    return prox_workspace(B, H, W, &a, &b);
}

edt_status edt2d_proximate_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                      const float* sampling, int32_t* sqdist, float* dist,
                                      int32_t* indices, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    return run_prox2d(mask, B, H, W, sampling, sqdist, dist, indices, workspace, workspace_bytes,
                      stream, nullptr);
}

edt_status edt2d_proximate_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                            const float* sampling, int32_t* sqdist, float* dist,
                                            int32_t* indices, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream,
                                            float* kernel_ms, const char** kernel_names,
                                            int32_t capacity, int32_t* count) {
    if (!kernel_ms || capacity < 1) return EDT_ERR_INVALID_ARGUMENT;
    edt::KernelTimer tm;
    tm.capacity = capacity;
    edt_status st = run_prox2d(mask, B, H, W, sampling, sqdist, dist, indices, workspace,
                               workspace_bytes, stream, &tm);
    return finish_timed(st, tm, stream, kernel_ms, kernel_names, count);
}

edt_status edt2d_u8_batched_noalloc(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                    const float* sampling, int32_t* sqdist, float* dist,
                                    int32_t* indices, hipStream_t stream) {
    return run2d(mask, B, H, W, sampling, sqdist, dist, indices, nullptr, 0, stream, nullptr, true);
}

edt_status edt1d_u8_batched(const uint8_t* mask, int32_t B, int32_t N, const float* sampling,
                            int32_t* sqdist, float* dist, int32_t* indices, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    // a line of N elements is an N x 1 image: the axis-0 pass alone decides,
    // and the virtual element (-1, 0) gives (p + 1)^2 and index -1
    const float s2d[2] = {sampling ? sampling[0] : 1.0f, 1.0f};
    return run2d(mask, B, N, 1, s2d, sqdist, dist, indices, workspace, workspace_bytes, stream,
                 nullptr);
}

edt_status edt_unravel_indices(const int32_t* indices, int32_t images, int32_t ndim,
                               const int32_t* shape, int32_t* coords, hipStream_t stream) {
    if (!indices || !coords || !shape || images < 1 || ndim < 1 || ndim > 3)
        return EDT_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)indices & 3) || ((uintptr_t)coords & 3)) return EDT_ERR_INVALID_ARGUMENT;
    int64_t per = 1;
    for (int k = 0; k < ndim; ++k) {
        if (shape[k] < 1 || shape[k] > kMaxExtent) return EDT_ERR_INVALID_ARGUMENT;
        per *= shape[k];
    }
    if (per > INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    const size_t nin = (size_t)images * (size_t)per * 4;
    if (overlap(indices, nin, coords, nin * (size_t)ndim)) return EDT_ERR_INVALID_ARGUMENT;
    const int n1 = ndim >= 2 ? shape[1] : 1;
    const int n2 = ndim >= 3 ? shape[2] : 1;
    if (edt::launch_unravel(indices, images, per, ndim, n1, n2, coords, stream) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

edt_status edt3d_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H, int32_t W,
                            const float* sampling, int32_t* sqdist, float* dist, int32_t* indices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return run3d(mask, B, D, H, W, sampling, sqdist, dist, indices, workspace, workspace_bytes,
                 stream, nullptr);
}

edt_status edt3d_u8_batched_idx64(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                  int32_t W, const float* sampling, int32_t* sqdist, float* dist,
                                  int64_t* indices, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    return run3d(mask, B, D, H, W, sampling, sqdist, dist, nullptr, workspace, workspace_bytes,
                 stream, nullptr, indices);
}

edt_status edt2d_u8_timed(const uint8_t* mask, int32_t H, int32_t W, const float* sampling,
                          int32_t* sqdist, float* dist, int32_t* indices, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, float* kernel_ms,
                          const char** kernel_names, int32_t capacity, int32_t* count) {
    if (!kernel_ms || capacity < 1) return EDT_ERR_INVALID_ARGUMENT;
    edt::KernelTimer tm;
    tm.capacity = capacity;
    edt_status st = run2d(mask, 1, H, W, sampling, sqdist, dist, indices, workspace, workspace_bytes,
                          stream, &tm);
    return finish_timed(st, tm, stream, kernel_ms, kernel_names, count);
}

edt_status edt2d_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                  const float* sampling, int32_t* sqdist, float* dist,
                                  int32_t* indices, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, float* kernel_ms, const char** kernel_names,
                                  int32_t capacity, int32_t* count) {
    if (!kernel_ms || capacity < 1) return EDT_ERR_INVALID_ARGUMENT;
    edt::KernelTimer tm;
    tm.capacity = capacity;
    edt_status st = run2d(mask, B, H, W, sampling, sqdist, dist, indices, workspace,
                          workspace_bytes, stream, &tm);
    return finish_timed(st, tm, stream, kernel_ms, kernel_names, count);
}

edt_status edt3d_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                  int32_t W, const float* sampling, int32_t* sqdist, float* dist,
                                  int32_t* indices, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, float* kernel_ms, const char** kernel_names,
                                  int32_t capacity, int32_t* count) {
    if (!kernel_ms || capacity < 1) return EDT_ERR_INVALID_ARGUMENT;
    edt::KernelTimer tm;
    tm.capacity = capacity;
    edt_status st = run3d(mask, B, D, H, W, sampling, sqdist, dist, indices, workspace,
                          workspace_bytes, stream, &tm);
    return finish_timed(st, tm, stream, kernel_ms, kernel_names, count);
}

size_t edt_brute_workspace_size(int32_t B, int32_t ndim, const int32_t* shape) {
    int64_t per = 0;
    if (!brute_shape_ok(B, ndim, shape, &per)) return 0;
    return brute_layout(B, per).total;
}

edt_status edt_brute_u8(const uint8_t* mask, int32_t B, int32_t ndim, const int32_t* shape,
                        const float* sampling, int32_t* sqdist, float* dist, int32_t* indices,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!shape || ndim < 1 || ndim > 3 || B < 1) return EDT_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < ndim; ++k)
        if (shape[k] < 1) return EDT_ERR_INVALID_ARGUMENT;
    int64_t per = 0;
    if (!brute_shape_ok(B, ndim, shape, &per)) return EDT_ERR_UNSUPPORTED_SHAPE;
    double s2[3];
    bool unit;
    edt_status st = read_sampling(sampling, ndim, s2, &unit);
    if (st != EDT_OK) return st;
    if (sqdist) {
        if (!unit) return EDT_ERR_INVALID_ARGUMENT;
        double mx = 0.0;
        for (int k = 0; k < ndim; ++k) mx += (double)shape[k] * shape[k];
        if (mx > (double)INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    }
    const BruteLayout L = brute_layout(B, per);
    st = check_buffers(mask, (size_t)B * per, sqdist, dist, indices, workspace, workspace_bytes, L.total);
    if (st != EDT_OK) return st;
    char* base = static_cast<char*>(workspace);
    int n[3];
    for (int k = 0; k < ndim; ++k) n[k] = shape[k];
    if (edt::launch_brute(mask, B, ndim, n, s2, reinterpret_cast<int32_t*>(base + L.list),
                          reinterpret_cast<int32_t*>(base + L.counts),
                          reinterpret_cast<int32_t*>(base + L.block_off), sqdist, dist, indices,
                          stream) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

edt_status edt_brute_metric_u8(const uint8_t* mask, int32_t B, int32_t ndim, const int32_t* shape,
                               int32_t metric, int32_t* dist, int32_t* indices, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (!shape || ndim < 1 || ndim > 3 || B < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (metric != EDT_METRIC_TAXICAB && metric != EDT_METRIC_CHESSBOARD) return EDT_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < ndim; ++k)
        if (shape[k] < 1) return EDT_ERR_INVALID_ARGUMENT;
    int64_t per = 0;
    if (!brute_shape_ok(B, ndim, shape, &per)) return EDT_ERR_UNSUPPORTED_SHAPE;
    const BruteLayout L = brute_layout(B, per);
    // the int32 distance buffer goes in the sqdist slot of the common check
    edt_status st = check_buffers(mask, (size_t)B * per, dist, nullptr, indices, workspace,
                                  workspace_bytes, L.total);
    if (st != EDT_OK) return st;
    char* base = static_cast<char*>(workspace);
    int n[3];
    for (int k = 0; k < ndim; ++k) n[k] = shape[k];
    if (edt::launch_brute_metric(mask, B, ndim, n,
                                 metric == EDT_METRIC_TAXICAB ? edt::kBruteTaxicab : edt::kBruteChessboard,
                                 reinterpret_cast<int32_t*>(base + L.list),
                                 reinterpret_cast<int32_t*>(base + L.counts),
                                 reinterpret_cast<int32_t*>(base + L.block_off), dist, indices,
                                 stream) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

}  // extern "C"

namespace {
// ---------------------------------------------------------------- any rank

constexpr int kMaxSpatial = 8;
constexpr int kMaxBatchAxes = 8;

// How edt_nd_u8 runs a shape: the LDS kernels for C-contiguous 1-, 2- and 3-D
// images within their limits; otherwise, for 1-, 2- and 3-D images whose
// spatial axes in some order fit those kernels, a reordered run (the mask
// gathered into the workspace in that order, the outputs put back); the
// workspace path of nd.hip for the rest.
enum class NdRoute { kEmpty, k1D, k2D, k3D, kPermuted, kGenericPermuted, kGeneric };

struct NdPlan {
    NdRoute route = NdRoute::kGeneric;
    edt::NdDesc d{};
    int64_t total = 0;          // elements over all images
    int64_t mask_span = 0;      // bytes from the mask pointer to its last element + 1
    int32_t fB = 0, fD = 0, fH = 0, fW = 0;   // the fast path's shape (permuted order for kPermuted)
    int perm[3] = {0, 1, 2};    // kPermuted: permuted axis k is spatial axis perm[k]
    size_t ws = 0;
    // kPermuted workspace: gathered mask, permuted int32 index / sqdist /
    // dist, then the LDS kernels' own workspace
    size_t off_idx = 0, off_sq = 0, off_dist = 0, off_inner = 0;
};

// Shape checks and routing (no buffer is looked at).  idx_bytes: 4 or 8.
edt_status plan_nd(int32_t nbatch, int32_t ndim, const int64_t* shape, const int64_t* strides,
                   int idx_bytes, NdPlan* out) {
    if (!shape || ndim < 1 || ndim > kMaxSpatial || nbatch < 0 || nbatch > kMaxBatchAxes)
        return EDT_ERR_INVALID_ARGUMENT;
    if (idx_bytes != 4 && idx_bytes != 8) return EDT_ERR_INVALID_ARGUMENT;
    NdPlan P;
    P.d.nb = nbatch;
    P.d.nd = ndim;
    const int na = nbatch + ndim;
    int64_t B = 1, N = 1;
    bool contiguous = true;
    int64_t expect = 1;
    for (int a = na - 1; a >= 0; --a) {
        const int64_t n = shape[a];
        if (n < 0) return EDT_ERR_INVALID_ARGUMENT;
        const int64_t st = strides ? strides[a] : expect;
        if (st < 0) return EDT_ERR_INVALID_ARGUMENT;
        if (n > 1 && st != expect) contiguous = false;
        if (n > 0 && expect > ((int64_t)1 << 62) / n) return EDT_ERR_UNSUPPORTED_SHAPE;
        expect *= n > 0 ? n : 1;
        P.d.ext[a] = n;
        P.d.mstride[a] = st;
    }
    for (int a = 0; a < nbatch; ++a) B *= shape[a];
    for (int a = nbatch; a < na; ++a) N *= shape[a];
    P.d.B = B;
    P.d.N = N;
    P.total = B * N;
    if (P.total == 0) {
        P.route = NdRoute::kEmpty;
        *out = P;
        return EDT_OK;
    }
    int64_t span = 1;
    for (int a = 0; a < na; ++a) {
        const int64_t reach = (shape[a] - 1) * P.d.mstride[a];
        if (P.d.mstride[a] > 0 && shape[a] - 1 > (((int64_t)1 << 62) - span) / P.d.mstride[a])
            return EDT_ERR_UNSUPPORTED_SHAPE;
        span += reach;
    }
    P.mask_span = span;
    // the LDS kernels: C-contiguous, at most 65535 images, int32 indices
    // (int64 for volumes), shapes within their limits
    if (contiguous && B <= kMaxExtent) {
        const int32_t b32 = (int32_t)B;
        auto fits = [](int64_t x) { return x >= 1 && x <= kMaxExtent; };
        if (ndim == 1 && fits(shape[nbatch]) && idx_bytes == 4 && shape2d_ok(b32, (int32_t)shape[nbatch], 1)) {
            P.route = NdRoute::k1D;
            P.fB = b32;
            P.fH = (int32_t)shape[nbatch];
            P.fW = 1;
            P.ws = layout2d(b32, P.fH, 1).total;
        } else if (ndim == 2 && fits(shape[nbatch]) && fits(shape[nbatch + 1]) && idx_bytes == 4 &&
                   shape2d_ok(b32, (int32_t)shape[nbatch], (int32_t)shape[nbatch + 1])) {
            P.route = NdRoute::k2D;
            P.fB = b32;
            P.fH = (int32_t)shape[nbatch];
            P.fW = (int32_t)shape[nbatch + 1];
            P.ws = layout2d(b32, P.fH, P.fW).total;
        } else if (ndim == 3 && fits(shape[nbatch]) && fits(shape[nbatch + 1]) && fits(shape[nbatch + 2]) &&
                   shape3d_ok(b32, (int32_t)shape[nbatch], (int32_t)shape[nbatch + 1], (int32_t)shape[nbatch + 2]) &&
                   (idx_bytes == 8 || N <= INT32_MAX)) {
            P.route = NdRoute::k3D;
            P.fB = b32;
            P.fD = (int32_t)shape[nbatch];
            P.fH = (int32_t)shape[nbatch + 1];
            P.fW = (int32_t)shape[nbatch + 2];
            P.ws = layout3d(b32, P.fD, P.fH, P.fW).total;
        }
    }
    // a reordered run: the first order of the spatial axes (identity first)
    // whose shape the LDS kernels take; int32 indices inside
    if (P.route == NdRoute::kGeneric && ndim <= 3 && B <= kMaxExtent && N <= INT32_MAX) {
        static const int kPerms2[2][3] = {{0, 1, 2}, {1, 0, 2}};
        static const int kPerms3[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
        const int np = ndim == 1 ? 1 : ndim == 2 ? 2 : 6;
        bool fitsall = true;
        for (int k = 0; k < ndim; ++k) fitsall = fitsall && shape[nbatch + k] >= 1 && shape[nbatch + k] <= kMaxExtent;
        const int32_t b32 = (int32_t)B;
        for (int pi = 0; fitsall && pi < np && P.route == NdRoute::kGeneric; ++pi) {
            const int* pm = ndim == 3 ? kPerms3[pi] : kPerms2[pi];
            int32_t e[3] = {1, 1, 1};
            for (int k = 0; k < ndim; ++k) e[k] = (int32_t)shape[nbatch + pm[k]];
            size_t inner = 0;
            bool ok = false;
            if (ndim == 1) {
                ok = shape2d_ok(b32, e[0], 1);
                if (ok) inner = layout2d(b32, e[0], 1).total;
            } else if (ndim == 2) {
                ok = shape2d_ok(b32, e[0], e[1]);
                if (ok) inner = layout2d(b32, e[0], e[1]).total;
            } else {
                ok = shape3d_ok(b32, e[0], e[1], e[2]);
                if (ok) inner = layout3d(b32, e[0], e[1], e[2]).total;
            }
            if (!ok) continue;
            P.route = NdRoute::kPermuted;
            for (int k = 0; k < 3; ++k) P.perm[k] = k < ndim ? pm[k] : k;
            P.fB = b32;
            P.fD = e[0];
            P.fH = e[1];
            P.fW = e[2];
            const size_t n = (size_t)P.total;
            P.off_idx = round_up(n);
            P.off_sq = P.off_idx + round_up(n * 4);
            P.off_dist = P.off_sq + round_up(n * 4);
            P.off_inner = P.off_dist + round_up(n * 4);
            P.ws = P.off_inner + inner;
        }
    }
    // the workspace path gives each line one thread on every axis but the
    // first (which runs in segments when its lines are few): a longest axis
    // with few lines goes first, in a reordered run of the workspace path
    if (P.route == NdRoute::kGeneric && (ndim == 2 || ndim == 3) && N <= INT32_MAX) {
        int amax = 0;
        for (int k = 1; k < ndim; ++k)
            if (shape[nbatch + k] > shape[nbatch + amax]) amax = k;
        if (amax != 0 && B * (N / shape[nbatch + amax]) < 16384) {
            P.route = NdRoute::kGenericPermuted;
            P.perm[0] = amax;
            for (int k = 0, o = 1; k < ndim; ++k)
                if (k != amax) P.perm[o++] = k;
            const size_t n = (size_t)P.total;
            P.off_idx = round_up(n);
            P.off_sq = P.off_idx + round_up(n * 4);
            P.off_dist = P.off_sq + round_up(n * 4);
            P.off_inner = P.off_dist + round_up(n * 4);
            P.ws = P.off_inner + edt::nd_workspace_bytes(P.total);
        }
    }
    if (P.route == NdRoute::kGeneric) P.ws = edt::nd_workspace_bytes(P.total);
    *out = P;
    return EDT_OK;
}

}  // namespace

extern "C" {
size_t edt_nd_workspace_size(int32_t nbatch, int32_t ndim, const int64_t* shape,
                             const int64_t* strides, int32_t index_bytes) {
    NdPlan P;
    if (plan_nd(nbatch, ndim, shape, strides, index_bytes == 8 ? 8 : 4, &P) != EDT_OK) return 0;
    return P.ws > 0 ? P.ws : 256;
}

edt_status edt_nd_u8(const uint8_t* mask, int32_t nbatch, int32_t ndim, const int64_t* shape,
                     const int64_t* strides, const float* sampling, int32_t* sqdist, float* dist,
                     void* indices, int32_t index_bytes, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (indices && index_bytes != 4 && index_bytes != 8) return EDT_ERR_INVALID_ARGUMENT;
    const int ib = indices ? index_bytes : 4;
    NdPlan P;
    edt_status st = plan_nd(nbatch, ndim, shape, strides, ib, &P);
    if (st != EDT_OK) return st;
    double s2[kMaxSpatial];
    bool unit;
    st = read_sampling(sampling, ndim, s2, &unit);
    if (st != EDT_OK) return st;
    if (!mask) return EDT_ERR_INVALID_ARGUMENT;
    if (!sqdist && !dist && !indices) return EDT_ERR_INVALID_ARGUMENT;
    if (sqdist) {
        if (!unit) return EDT_ERR_INVALID_ARGUMENT;
        double mx = 0.0;
        for (int k = 0; k < ndim; ++k) mx += (double)shape[nbatch + k] * (double)shape[nbatch + k];
        if (mx > (double)INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    }
    if (indices && ib == 4 && P.d.N > INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    // outputs, mask span and workspace: alignment and overlap
    if (((uintptr_t)sqdist & 3) || ((uintptr_t)dist & 3) || ((uintptr_t)indices & (ib - 1)))
        return EDT_ERR_INVALID_ARGUMENT;
    if (P.route == NdRoute::kEmpty) return EDT_OK;
    if (!workspace || ((uintptr_t)workspace & (kAlign - 1))) return EDT_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < P.ws) return EDT_ERR_WORKSPACE_TOO_SMALL;
    const size_t n = (size_t)P.total;
    const void* bufs[5] = {mask, sqdist, dist, indices, workspace};
    const size_t sizes[5] = {(size_t)P.mask_span, sqdist ? n * 4 : 0, dist ? n * 4 : 0,
                             indices ? n * (size_t)ib : 0, P.ws};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(bufs[i], sizes[i], bufs[j], sizes[j])) return EDT_ERR_INVALID_ARGUMENT;
    float samp[kMaxSpatial];
    for (int k = 0; k < ndim; ++k) samp[k] = sampling ? sampling[k] : 1.0f;
    switch (P.route) {
        case NdRoute::k1D: {
            const float s1[2] = {samp[0], 1.0f};
            return run2d(mask, P.fB, P.fH, 1, s1, sqdist, dist, static_cast<int32_t*>(indices), workspace,
                         workspace_bytes, stream, nullptr);
        }
        case NdRoute::k2D:
            return run2d(mask, P.fB, P.fH, P.fW, samp, sqdist, dist, static_cast<int32_t*>(indices),
                         workspace, workspace_bytes, stream, nullptr);
        case NdRoute::k3D:
            if (ib == 8)
                return run3d(mask, P.fB, P.fD, P.fH, P.fW, samp, sqdist, dist, nullptr, workspace,
                             workspace_bytes, stream, nullptr, static_cast<int64_t*>(indices));
            return run3d(mask, P.fB, P.fD, P.fH, P.fW, samp, sqdist, dist, static_cast<int32_t*>(indices),
                         workspace, workspace_bytes, stream, nullptr);
        case NdRoute::kPermuted: {
            char* base = static_cast<char*>(workspace);
            uint8_t* pm = reinterpret_cast<uint8_t*>(base);
            int32_t* pidx = reinterpret_cast<int32_t*>(base + P.off_idx);
            int32_t* psq = sqdist ? reinterpret_cast<int32_t*>(base + P.off_sq) : nullptr;
            float* pdist = dist ? reinterpret_cast<float*>(base + P.off_dist) : nullptr;
            void* inner = base + P.off_inner;
            const size_t inner_bytes = workspace_bytes - P.off_inner;
            for (int k = 0; k < ndim; ++k) P.d.s2[k] = s2[k];
            if (edt::launch_nd_gather(mask, P.d, P.perm, pm, stream) != hipSuccess) return EDT_ERR_HIP;
            float ps[3] = {1.0f, 1.0f, 1.0f};
            for (int k = 0; k < ndim; ++k) ps[k] = samp[P.perm[k]];
            edt_status rs;
            if (ndim == 1) {
                const float s1[2] = {ps[0], 1.0f};
                rs = run2d(pm, P.fB, P.fD, 1, s1, psq, pdist, pidx, inner, inner_bytes, stream, nullptr);
            } else if (ndim == 2) {
                rs = run2d(pm, P.fB, P.fD, P.fH, ps, psq, pdist, pidx, inner, inner_bytes, stream, nullptr);
            } else {
                rs = run3d(pm, P.fB, P.fD, P.fH, P.fW, ps, psq, pdist, pidx, inner, inner_bytes, stream,
                           nullptr);
            }
            if (rs != EDT_OK) return rs;
            if (edt::launch_nd_unpermute(P.d, P.perm, pidx, psq, pdist, sqdist, dist, indices, ib, stream) !=
                hipSuccess)
                return EDT_ERR_HIP;
            return EDT_OK;
        }
        case NdRoute::kGenericPermuted: {
            char* base = static_cast<char*>(workspace);
            uint8_t* pm = reinterpret_cast<uint8_t*>(base);
            int32_t* pidx = reinterpret_cast<int32_t*>(base + P.off_idx);
            int32_t* psq = sqdist ? reinterpret_cast<int32_t*>(base + P.off_sq) : nullptr;
            float* pdist = dist ? reinterpret_cast<float*>(base + P.off_dist) : nullptr;
            for (int k = 0; k < ndim; ++k) P.d.s2[k] = s2[k];
            if (edt::launch_nd_gather(mask, P.d, P.perm, pm, stream) != hipSuccess) return EDT_ERR_HIP;
            edt::NdDesc q = P.d;   // the gathered array: C-contiguous, spatial axes permuted
            for (int k = 0; k < ndim; ++k) {
                q.ext[nbatch + k] = P.d.ext[nbatch + P.perm[k]];
                q.s2[k] = s2[P.perm[k]];
            }
            int64_t st = 1;
            for (int a = nbatch + ndim - 1; a >= 0; --a) {
                q.mstride[a] = st;
                st *= q.ext[a];
            }
            if (edt::launch_nd(pm, q, base + P.off_inner, psq, pdist, pidx, 4, stream) != hipSuccess)
                return EDT_ERR_HIP;
            if (edt::launch_nd_unpermute(P.d, P.perm, pidx, psq, pdist, sqdist, dist, indices, ib, stream) !=
                hipSuccess)
                return EDT_ERR_HIP;
            return EDT_OK;
        }
        default:
            break;
    }
    for (int k = 0; k < ndim; ++k) P.d.s2[k] = s2[k];
    if (edt::launch_nd(mask, P.d, workspace, sqdist, dist, indices, ib, stream) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

edt_status edt_unravel_indices_nd(const void* indices, int32_t index_bytes, int64_t images,
                                  int32_t ndim, const int64_t* shape, void* coords,
                                  hipStream_t stream) {
    if (!indices || !coords || !shape || images < 0 || ndim < 1 || ndim > kMaxSpatial)
        return EDT_ERR_INVALID_ARGUMENT;
    if (index_bytes != 4 && index_bytes != 8) return EDT_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)indices & (index_bytes - 1)) || ((uintptr_t)coords & (index_bytes - 1)))
        return EDT_ERR_INVALID_ARGUMENT;
    int64_t per = 1;
    for (int k = 0; k < ndim; ++k) {
        if (shape[k] < 1) return EDT_ERR_INVALID_ARGUMENT;
        if (per > ((int64_t)1 << 62) / shape[k]) return EDT_ERR_UNSUPPORTED_SHAPE;
        per *= shape[k];
    }
    if (index_bytes == 4 && per > INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    if (images > 0 && per > (((int64_t)1 << 62) / ndim) / images) return EDT_ERR_UNSUPPORTED_SHAPE;
    const size_t nin = (size_t)images * (size_t)per * (size_t)index_bytes;
    if (overlap(indices, nin, coords, nin * (size_t)ndim)) return EDT_ERR_INVALID_ARGUMENT;
    if (edt::launch_unravel_nd(indices, index_bytes, images, ndim, shape, coords, stream) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

namespace {

enum class Chamfer { kTaxicab, kChessboard };

edt_status chamfer2d(Chamfer metric, const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                     int32_t* dist, int32_t* indices, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (B < 1 || H < 1 || W < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (!shape2d_ok(B, H, W)) return EDT_ERR_UNSUPPORTED_SHAPE;
    const Layout L = layout2d(B, H, W);
    edt_status st = check_buffers(mask, (size_t)B * H * W, dist, nullptr, indices, workspace,
                                  workspace_bytes, L.total);
    if (st != EDT_OK) return st;
    char* base = static_cast<char*>(workspace);
    uint16_t* c0 = reinterpret_cast<uint16_t*>(base + L.c0);
    if (edt::launch_axis0(mask, B, H, W, reinterpret_cast<uint16_t*>(base + L.first),
                          reinterpret_cast<uint16_t*>(base + L.last),
                          reinterpret_cast<uint64_t*>(base + L.bits), c0, stream, nullptr) != hipSuccess)
        return EDT_ERR_HIP;
    const hipError_t e = metric == Chamfer::kTaxicab
                             ? edt::launch_l1_rows_2d(c0, B, H, W, dist, indices, stream, nullptr)
                             : edt::launch_rows_linf_2d(c0, B, H, W, dist, indices, stream, nullptr);
    return e == hipSuccess ? EDT_OK : EDT_ERR_HIP;
}

edt_status chamfer3d(Chamfer metric, const uint8_t* mask, int32_t B, int32_t D, int32_t H, int32_t W,
                     int32_t* dist, int32_t* indices, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (B < 1 || D < 1 || H < 1 || W < 1) return EDT_ERR_INVALID_ARGUMENT;
    if (!shape3d_ok(B, D, H, W)) return EDT_ERR_UNSUPPORTED_SHAPE;
    if (indices && (int64_t)D * H * W > INT32_MAX) return EDT_ERR_UNSUPPORTED_SHAPE;
    const Layout L = layout3d(B, D, H, W);
    edt_status st = check_buffers(mask, (size_t)B * D * H * W, dist, nullptr, indices, workspace,
                                  workspace_bytes, L.total);
    if (st != EDT_OK) return st;
    char* base = static_cast<char*>(workspace);
    uint16_t* c0 = reinterpret_cast<uint16_t*>(base + L.c0);
    uint32_t* c01 = reinterpret_cast<uint32_t*>(base + L.c01);
    if (edt::launch_axis0(mask, B, D, (int64_t)H * W, reinterpret_cast<uint16_t*>(base + L.first),
                          reinterpret_cast<uint16_t*>(base + L.last),
                          reinterpret_cast<uint64_t*>(base + L.bits), c0, stream, nullptr) != hipSuccess)
        return EDT_ERR_HIP;
    const bool l1 = metric == Chamfer::kTaxicab;
    if ((l1 ? edt::launch_l1_cols_3d(c0, B, D, H, W, c01, stream, nullptr)
            : edt::launch_cols_linf_3d(c0, B, D, H, W, c01, stream, nullptr)) != hipSuccess)
        return EDT_ERR_HIP;
    if ((l1 ? edt::launch_l1_rows_3d(c01, B, D, H, W, dist, indices, stream, nullptr)
            : edt::launch_rows_linf_3d(c01, B, D, H, W, dist, indices, stream, nullptr)) != hipSuccess)
        return EDT_ERR_HIP;
    return EDT_OK;
}

}  // namespace

edt_status edt2d_taxicab_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                    int32_t* dist, int32_t* indices, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return chamfer2d(Chamfer::kTaxicab, mask, B, H, W, dist, indices, workspace, workspace_bytes,
                     stream);
}

edt_status edt3d_taxicab_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                    int32_t W, int32_t* dist, int32_t* indices, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    return chamfer3d(Chamfer::kTaxicab, mask, B, D, H, W, dist, indices, workspace, workspace_bytes,
                     stream);
}

edt_status edt2d_chessboard_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                       int32_t* dist, int32_t* indices, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return chamfer2d(Chamfer::kChessboard, mask, B, H, W, dist, indices, workspace, workspace_bytes,
                     stream);
}

edt_status edt3d_chessboard_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                       int32_t W, int32_t* dist, int32_t* indices, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return chamfer3d(Chamfer::kChessboard, mask, B, D, H, W, dist, indices, workspace,
                     workspace_bytes, stream);
}

const char* edt_status_string(edt_status status) {
    switch (status) {
        case EDT_OK: return "EDT_OK";
        case EDT_ERR_INVALID_ARGUMENT: return "EDT_ERR_INVALID_ARGUMENT";
        case EDT_ERR_UNSUPPORTED_SHAPE: return "EDT_ERR_UNSUPPORTED_SHAPE";
        case EDT_ERR_WORKSPACE_TOO_SMALL: return "EDT_ERR_WORKSPACE_TOO_SMALL";
        case EDT_ERR_HIP: return "EDT_ERR_HIP";
    }
    return "EDT_ERR_UNKNOWN";
}

const char* edt_version(void) { return "0.1.0"; }

}  // extern "C"
