/*
 * edt.h -- exact Euclidean distance transform for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libedt_mi355x.so.  Plain pointers and sizes only.
 *
 * The transform ("GPU-Based Parallel Euclidean Distance Transform Algorithm",
 * Mathematics 14(4), §1 Introduction): every element of a binary image gets
 * the Euclidean distance to its nearest background element and, on request,
 * the index of that element (the discrete Voronoi / feature transform).  It is
 * computed exactly by the separable lower-envelope-of-parabolas method
 * (TorchMorph, the paragraph on the separable lower-envelope EDT): one
 * nearest-background scan along axis 0, then one lower-envelope pass per
 * remaining axis.  Keyword semantics (grid spacing `sampling`, distances
 * and/or indices, caller-preallocated outputs) follow TorchMorph's
 * SciPy-compatible distance-transform interface.
 *
 * Conventions shared by every entry point
 *   mask       device pointer, uint8, C-contiguous; 0 = background, any other
 *              value = foreground.  Any alignment.
 *   sampling   HOST pointer to one positive float per axis (axis order of the
 *              array), or NULL for unit spacing.  sampling[k] scales axis k.
 *   sqdist     device int32 [N] or NULL: exact squared distance.  Only with
 *              unit spacing (sampling NULL or all 1.0f).
 *   dist       device float [N] or NULL: sqrt of the squared distance,
 *              rounded to float32 (error <= 1 ulp of the float32 result).
 *   indices    device int32 [N] or NULL: row-major flat index, within the same
 *              image/volume, of a nearest background element.  Where several
 *              are equally near, any one of them may be returned.
 *   At least one of sqdist / dist / indices must be non-NULL.  Outputs are
 *   4-byte aligned, C-contiguous, and alias neither the mask, each other, nor
 *   the workspace.
 *   workspace  device buffer of at least *_workspace_size() bytes, 256-byte
 *              aligned, owned by the caller; its contents on entry do not
 *              matter and on return are unspecified.
 *   stream     HIP stream the kernels are enqueued on (NULL = default stream).
 *              The call returns after enqueueing; it never synchronizes.
 *
 * No background.  An image/volume without any background element is handled
 * with a virtual background element at coordinates (-1, 0, ..., 0), the
 * convention SciPy follows (TorchMorph defers to it): its squared distance is
 * s0^2 (p0+1)^2 + sum_k sk^2 pk^2 and its index is -(n1 * ... * n_{d-1}).
 *
 * Ownership and threading.  The library allocates no device memory and keeps
 * no state between calls; concurrent calls with distinct buffers are safe.
 * The one exception is edt2d_u8_batched_noalloc, whose workspace is a device
 * array of the library's own (one per device, see its declaration).
 *
 * Errors.  Argument errors are detected on the host before any HIP call and
 * return without touching any buffer.  EDT_ERR_HIP means a kernel launch was
 * rejected (hipGetLastError after the launch); outputs are then unspecified.
 *
 * Limits (of the entry points with int32 extents; edt_nd_u8 below lifts
 * them).  Every extent and every batch size B in [1, 65535]; elements per
 * image <= 2^31-1, and per volume too when indices are requested (a volume of
 * more elements, which HBM holds easily, is transformed when only sqdist
 * and/or dist are asked for);
 * when sqdist is requested the largest possible squared distance
 * (sum of extent^2) must fit in int32.  The lower envelope of a line is kept in
 * LDS, which bounds the line lengths of the envelope passes:
 *   2-D: W <= 32768;  3-D: H <= 32768 and W <= 16384.
 * Shapes beyond the limits return EDT_ERR_UNSUPPORTED_SHAPE.
 */
#ifndef EDT_MI355X_H
#define EDT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum edt_status {
    EDT_OK = 0,
    EDT_ERR_INVALID_ARGUMENT = 1,    /* NULL mask, no output, bad spacing, sqdist with
                                        non-unit spacing, misaligned output/workspace */
    EDT_ERR_UNSUPPORTED_SHAPE = 2,   /* extent or element count beyond the limits */
    EDT_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < *_workspace_size(...) */
    EDT_ERR_HIP = 4                  /* a kernel launch failed */
} edt_status;

/* Bytes of workspace edt2d_u8 needs for an H x W image (0 if the shape is
   outside the limits). */
size_t edt2d_workspace_size(int32_t H, int32_t W);

/* 2-D transform of one H x W image (row-major, axis 0 = rows).  sampling is
   {s_rows, s_cols} or NULL. */
edt_status edt2d_u8(const uint8_t* mask, int32_t H, int32_t W,
                    const float* sampling,
                    int32_t* sqdist, float* dist, int32_t* indices,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace edt2d_u8_batched needs for B images of H x W (0 if the
   shape is outside the limits; B <= 65535). */
size_t edt2d_batched_workspace_size(int32_t B, int32_t H, int32_t W);

/* 2-D transform of B independent H x W images stored back to back
   ([B][H][W]): the per-image result of edt2d_u8 for each, in one set of
   launches (the batched tensors of TorchMorph's transforms).  indices are flat
   within each image (r*W + c); an image without background gets the virtual
   element on its own, whatever the other images hold. */
edt_status edt2d_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                            const float* sampling,
                            int32_t* sqdist, float* dist, int32_t* indices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* edt2d_u8_batched for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   hipMalloc): the same transform, but the workspace is the library's own
   device array of edt2d_noalloc_max_workspace() bytes (64 MiB; one copy per
   device, held from the first call on that device until the process ends).
   The call allocates nothing; the caller still passes the mask and outputs,
   with the conventions of edt2d_u8_batched.  A shape whose workspace
   (edt2d_batched_workspace_size) exceeds the array returns
   EDT_ERR_WORKSPACE_TOO_SMALL before any HIP call.  Every call on one device
   shares that device's array: calls that overlap in time on one device (two
   streams, or two threads) race on it and must be serialized by the caller;
   the array keeps the last call's contents, and nothing in it needs to be
   cleared between calls.  EDT_ERR_HIP also covers a failure to look up the
   array's device address on the first call on a device. */
edt_status edt2d_u8_batched_noalloc(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                    const float* sampling,
                                    int32_t* sqdist, float* dist, int32_t* indices,
                                    hipStream_t stream);

/* Size in bytes of the device array edt2d_u8_batched_noalloc works in. */
size_t edt2d_noalloc_max_workspace(void);

/* Bytes of workspace edt2d_proximate_u8_batched needs for B images of H x W
   (0 outside its limits: B, H <= 65535, W <= 16384, H * W <= 2^31-1). */
size_t edt2d_proximate_workspace_size(int32_t B, int32_t H, int32_t W);

/* The same 2-D transform as edt2d_u8_batched, by the row pass of "GPU-Based
   Parallel Euclidean Distance Transform Algorithm" instead of the separable
   envelope: sub-blocks of 64 rows, each row's upper and lower proximate-point
   sets built by Algorithm 1 for the sub-block's first row and updated row by
   row by Algorithms 2-3 (masked points removed, the row's background pixels
   merged in, prefix-sum compaction), every pixel answered from both sets
   (§3.3-§3.4).  A second implementation of the same result, kept for
   comparison with the page's own method: arguments, outputs, indices and the
   virtual element exactly as edt2d_u8_batched; any nearest background
   element may be returned where several are equally near. */
edt_status edt2d_proximate_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                      const float* sampling,
                                      int32_t* sqdist, float* dist, int32_t* indices,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* edt2d_proximate_u8_batched with per-kernel HIP event timings, as
   edt2d_u8_timed. */
edt_status edt2d_proximate_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                            const float* sampling,
                                            int32_t* sqdist, float* dist, int32_t* indices,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream, float* kernel_ms,
                                            const char** kernel_names, int32_t capacity,
                                            int32_t* count);

/* Bytes of workspace edt1d_u8_batched needs for B lines of N elements. */
size_t edt1d_workspace_size(int32_t B, int32_t N);

/* 1-D transform of B independent lines of N elements ([B][N]): for each
   element the distance along the line to the nearest background element of
   its own line.  sampling is {s} or NULL.  indices are the position within the
   line; a line without background gets the virtual element at -1, so
   sqdist = s^2 (p + 1)^2 and index -1.  (Computed as B images of N x 1.) */
edt_status edt1d_u8_batched(const uint8_t* mask, int32_t B, int32_t N,
                            const float* sampling,
                            int32_t* sqdist, float* dist, int32_t* indices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-axis coordinates of flat indices, the layout SciPy's feature transform
   returns (TorchMorph's `return_indices` follows SciPy's interface).
   indices: device int32 [images][n] as returned by the transforms above for
   images of shape shape[0..ndim) (ndim 1..3, n = product of the extents).
   coords:  device int32 [images][ndim][n]: plane k of image b holds the axis-k
   coordinate.  A virtual index -(shape[1] * ... ) becomes (-1, 0, ..., 0).
   Both buffers are caller-owned, 4-byte aligned and must not overlap; shape
   is a HOST pointer.  Asynchronous on `stream`; argument errors return before
   any HIP call. */
edt_status edt_unravel_indices(const int32_t* indices, int32_t images, int32_t ndim,
                               const int32_t* shape, int32_t* coords, hipStream_t stream);

/* Bytes of workspace edt_brute_u8 needs (0 if the shape is outside its
   limits).  shape is a HOST pointer to ndim extents. */
size_t edt_brute_workspace_size(int32_t B, int32_t ndim, const int32_t* shape);

/* The same transform by its definition, for checking on the device: every
   element against every background element of its image (TorchMorph keeps a
   brute-force transform beside its EDT as an exactness oracle).  B images of
   ndim = 1..3 axes, extents shape[0..ndim) (HOST pointer), mask [B][...];
   sampling {s_0, ..} or NULL; outputs, indices and the virtual element as for
   the transforms above.  Among equally near background elements the smallest
   flat index is returned.  Cost O(elements x background elements): meant for
   small images.  Limits: B and every extent in [1, 65535], elements per image
   <= 2^31-1; sqdist as above. */
edt_status edt_brute_u8(const uint8_t* mask, int32_t B, int32_t ndim, const int32_t* shape,
                        const float* sampling,
                        int32_t* sqdist, float* dist, int32_t* indices,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Metric codes of edt_brute_metric_u8. */
#define EDT_METRIC_TAXICAB 1
#define EDT_METRIC_CHESSBOARD 2

/* The chamfer transforms by their definition, the checker beside the taxicab
   and chessboard entry points below (TorchMorph ships both chamfer transforms
   and a brute-force oracle beside its EDT): for every element the minimum
   over the background elements of its image of sum_k |p_k - b_k|
   (EDT_METRIC_TAXICAB) or max_k |p_k - b_k| (EDT_METRIC_CHESSBOARD), as
   int32, and the smallest flat index attaining it.  B images of ndim = 1..3
   axes, extents shape[0..ndim) (HOST pointer), mask [B][...]; dist and/or
   indices (int32, device, 4-byte aligned, [B][...]); the virtual element for
   images without background as for the taxicab and chessboard entry points;
   workspace of edt_brute_workspace_size(B, ndim, shape) bytes.  Limits as
   for edt_brute_u8; an unknown metric is EDT_ERR_INVALID_ARGUMENT.  Cost
   O(elements x background elements). */
edt_status edt_brute_metric_u8(const uint8_t* mask, int32_t B, int32_t ndim, const int32_t* shape,
                               int32_t metric, int32_t* dist, int32_t* indices,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* City-block (taxicab, L1) distance transform, one of the chamfer
   transforms TorchMorph ships beside its EDT (read as the L1 metric, like
   SciPy's "taxicab"): for every element, min over background elements of
   sum_k |p_k - b_k|, as int32 (unit spacing), and optionally the flat index of
   such an element (ties: any).  B images H x W ([B][H][W]) or B volumes
   D x H x W; an image/volume without background uses the virtual element at
   (-1, 0, ...) (distance (p0 + 1) + sum_{k>0} p_k, index as above).  dist
   and/or indices (int32, device, 4-byte aligned); workspace of
   edt2d_batched_workspace_size / edt3d_workspace_size bytes; the same shape
   limits as the EDT entry points (volumes with indices: <= 2^31-1 elements);
   errors as above. */
edt_status edt2d_taxicab_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                    int32_t* dist, int32_t* indices,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);
edt_status edt3d_taxicab_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                    int32_t W, int32_t* dist, int32_t* indices,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Chessboard (L-infinity) distance transform, the other chamfer transform
   TorchMorph ships beside its EDT (read as the L-infinity metric, like SciPy's
   "chessboard"): for every element, min over background elements of
   max_k |p_k - b_k|, as int32, and optionally the flat index of such an
   element (ties: any).  Layouts, the virtual element (distance
   max(p0 + 1, p1, ...)), buffers, workspace, limits and errors exactly as for
   the taxicab entry points above.  Computed as the EDT is, one lower
   envelope per line and axis (the functions max(g_j, |q - j|) change places
   once, as parabolas do), with exact integer crossings. */
edt_status edt2d_chessboard_u8_batched(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                       int32_t* dist, int32_t* indices,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);
edt_status edt3d_chessboard_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                       int32_t W, int32_t* dist, int32_t* indices,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace edt3d_u8_batched needs for B volumes of D x H x W. */
size_t edt3d_workspace_size(int32_t B, int32_t D, int32_t H, int32_t W);

/* 3-D transform of B independent volumes, each D x H x W, stored back to back
   ([B][D][H][W]).  sampling is {s_D, s_H, s_W} or NULL.  indices are flat
   within each volume (d*H*W + h*W + w). */
edt_status edt3d_u8_batched(const uint8_t* mask, int32_t B, int32_t D, int32_t H, int32_t W,
                            const float* sampling,
                            int32_t* sqdist, float* dist, int32_t* indices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* edt3d_u8_batched with int64 flat indices (int64_t [B*D*H*W], 8-byte
   aligned; NULL for none), for volumes of more than 2^31 - 1 elements, which
   the int32 form refuses indices for; same workspace, limits and errors
   otherwise. */
edt_status edt3d_u8_batched_idx64(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                  int32_t W, const float* sampling,
                                  int32_t* sqdist, float* dist, int64_t* indices,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Same as edt2d_u8 / edt2d_u8_batched / edt3d_u8_batched, for measurement: records a HIP event
   pair around every kernel it enqueues, waits for the stream, and returns each
   kernel's duration in milliseconds (launch order) in kernel_ms[0..*count) and
   its name in kernel_names[] (static strings; may be NULL).  Fails with
   EDT_ERR_INVALID_ARGUMENT if capacity is smaller than the number of kernels
   (at most 8).  Results are identical to the untimed call. */
edt_status edt2d_u8_timed(const uint8_t* mask, int32_t H, int32_t W,
                          const float* sampling,
                          int32_t* sqdist, float* dist, int32_t* indices,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          float* kernel_ms, const char** kernel_names,
                          int32_t capacity, int32_t* count);

edt_status edt2d_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t H, int32_t W,
                                  const float* sampling,
                                  int32_t* sqdist, float* dist, int32_t* indices,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, float* kernel_ms,
                                  const char** kernel_names, int32_t capacity,
                                  int32_t* count);

edt_status edt3d_u8_batched_timed(const uint8_t* mask, int32_t B, int32_t D, int32_t H,
                                  int32_t W, const float* sampling,
                                  int32_t* sqdist, float* dist, int32_t* indices,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, float* kernel_ms,
                                  const char** kernel_names, int32_t capacity,
                                  int32_t* count);

/* Bytes of workspace edt_nd_u8 needs for the given shape and mask strides
   (NULL: C-contiguous) and index width (4 or 8); 0 if the arguments are
   invalid.  The size depends on the path the shape takes (see edt_nd_u8). */
size_t edt_nd_workspace_size(int32_t nbatch, int32_t ndim, const int64_t* shape,
                             const int64_t* strides, int32_t index_bytes);

/* The transform for any spatial rank: TorchMorph's batched (B, C, Spatial...)
   tensors with a spatial rank from 1 to 8 (the separable method applies one
   pass per axis, whatever the rank).
     shape    HOST int64 [nbatch + ndim]: nbatch leading batch axes (0..8; each
              image is transformed on its own), then ndim (1..8) spatial axes.
              Extents >= 0 (any extent 0: nothing to do, EDT_OK).
     strides  HOST int64 [nbatch + ndim] element strides of the mask (>= 0;
              views such as slices and transposes), or NULL for C-contiguous.
     sampling HOST float [ndim] (spatial axes) or NULL.
     outputs  C-contiguous over the full shape: sqdist int32 / dist float32 as
              for the entry points above; indices int32 (index_bytes 4) or
              int64 (8), flat within each image (row-major over the spatial
              axes), the virtual element -(n1 * ... * n_{ndim-1}).
   C-contiguous 1-, 2- and 3-D images within the limits of edt1d_u8_batched,
   edt2d_u8_batched and edt3d_u8_batched (int64 indices: 3-D only) run those
   kernels.  Every other shape -- rank 4 and above, strided masks, rows longer
   than the LDS envelope holds (2-D W > 32768, 3-D W > 16384 or H > 32768),
   extents over 65535, more than 65535 images -- runs the workspace path: the
   envelope of each line in the caller's workspace instead of LDS (TorchMorph's
   fallback for long lines), 40 bytes of workspace per element.  Limits:
   elements of all images < 2^62; int32 indices need elements per image
   <= 2^31-1; sqdist needs unit spacing and sum of extent^2 <= 2^31-1.  Errors
   as above; the mask's span (from its pointer to its last element) must not
   overlap the outputs or the workspace. */
edt_status edt_nd_u8(const uint8_t* mask, int32_t nbatch, int32_t ndim, const int64_t* shape,
                     const int64_t* strides, const float* sampling,
                     int32_t* sqdist, float* dist, void* indices, int32_t index_bytes,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Per-axis coordinates of flat indices of any rank (1..8) and width:
   indices int32 (index_bytes 4) or int64 (8), [images][n]; coords of the same
   type, [images][ndim][n] (the layout of edt_unravel_indices); shape HOST
   int64 [ndim].  The virtual index becomes (-1, 0, ..., 0).  Buffers
   caller-owned, aligned to the index width, not overlapping; asynchronous on
   stream; argument errors return before any HIP call. */
edt_status edt_unravel_indices_nd(const void* indices, int32_t index_bytes, int64_t images,
                                  int32_t ndim, const int64_t* shape, void* coords,
                                  hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* edt_status_string(edt_status status);

/* Library version, as "major.minor.patch". */
const char* edt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EDT_MI355X_H */
