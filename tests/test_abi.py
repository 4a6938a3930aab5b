"""CPU tests of the C ABI boundary: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(so these run without a GPU; the pointers below are never dereferenced)."""

import ctypes
import os
import re

import numpy as np
import pytest

from exact_euclidean_distance_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "edt.h")

OK, INVALID, SHAPE, SMALL, HIP = 0, 1, 2, 3, 4
# fake, aligned device addresses in disjoint ranges (never dereferenced)
MASK, SQ, DIST, IDX, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
BIG = 1 << 40


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The argument tests pass fake device addresses: a call that validation let
# through by mistake would launch kernels on them, so they run only where no
# HIP device exists (the GPU tests cover the same entry points with buffers).
fake_pointers = pytest.mark.skipif(_has_gpu(), reason="fake device pointers; CPU-only checks")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(edt\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.edt_status_string(code).decode() == name
    assert lib.edt_version().decode().count(".") == 2


def test_workspace_sizes(lib):
    assert lib.edt2d_workspace_size(512, 512) >= 512 * 512 * 2
    assert lib.edt3d_workspace_size(16, 128, 128, 128) >= 16 * 128 ** 3 * 6
    assert lib.edt2d_workspace_size(0, 5) == 0
    assert lib.edt2d_workspace_size(5, 40000) == 0
    assert lib.edt2d_workspace_size(70000, 5) == 0
    assert lib.edt3d_workspace_size(1, 8, 40000, 8) == 0   # H over the column-pass limit
    assert lib.edt3d_workspace_size(1, 8, 8, 20000) == 0
    # > 2^31-1 elements: a workspace for distances (indices are refused by the call)
    assert lib.edt3d_workspace_size(1, 2100, 1024, 1000) >= 2100 * 1024 * 1000 * 6


def call2d(lib, mask=MASK, H=64, W=64, sampling=None, sq=SQ, dist=DIST, idx=IDX, ws=WS,
           ws_bytes=BIG):
    samp = None if sampling is None else (ctypes.c_float * 2)(*sampling)
    return lib.edt2d_u8(mask, H, W, samp, sq, dist, idx, ws, ws_bytes, None)


def call3d(lib, mask=MASK, B=2, D=8, H=8, W=8, sampling=None, sq=SQ, dist=DIST, idx=IDX, ws=WS,
           ws_bytes=BIG):
    samp = None if sampling is None else (ctypes.c_float * 3)(*sampling)
    return lib.edt3d_u8_batched(mask, B, D, H, W, samp, sq, dist, idx, ws, ws_bytes, None)


@fake_pointers
def test_2d_argument_errors(lib):
    assert call2d(lib, mask=None) == INVALID
    assert call2d(lib, H=0) == INVALID
    assert call2d(lib, W=-3) == INVALID
    assert call2d(lib, H=70000) == SHAPE
    assert call2d(lib, W=40000) == SHAPE
    assert call2d(lib, H=65535, W=32768) == SHAPE           # > 2^31-1 elements
    assert call2d(lib, sq=None, dist=None, idx=None) == INVALID
    assert call2d(lib, sampling=(2.0, 1.0)) == INVALID      # sqdist needs unit spacing
    assert call2d(lib, sampling=(0.0, 1.0), sq=None) == INVALID
    assert call2d(lib, sampling=(-1.0, 1.0), sq=None) == INVALID
    assert call2d(lib, sampling=(float("nan"), 1.0), sq=None) == INVALID
    assert call2d(lib, sampling=(float("inf"), 1.0), sq=None) == INVALID
    assert call2d(lib, ws=None) == INVALID
    assert call2d(lib, ws=WS + 16) == INVALID               # workspace not 256-byte aligned
    assert call2d(lib, ws_bytes=lib.edt2d_workspace_size(64, 64) - 1) == SMALL
    assert call2d(lib, sq=SQ + 2) == INVALID                # misaligned output
    assert call2d(lib, dist=WS + 256) == INVALID            # output inside the workspace
    assert call2d(lib, idx=SQ) == INVALID                   # outputs alias each other
    assert call2d(lib, sq=MASK) == INVALID                  # output aliases the mask
    assert call2d(lib, H=50000, W=50000, sampling=None, dist=None, idx=None) == SHAPE


@fake_pointers
def test_3d_argument_errors(lib):
    assert call3d(lib, mask=None) == INVALID
    assert call3d(lib, B=0) == INVALID
    assert call3d(lib, D=0) == INVALID
    assert call3d(lib, H=40000) == SHAPE
    assert call3d(lib, W=20000) == SHAPE
    assert call3d(lib, D=70000) == SHAPE
    assert call3d(lib, sq=None, dist=None, idx=None) == INVALID
    assert call3d(lib, sampling=(2.5, 1.0, 1.0)) == INVALID
    assert call3d(lib, sampling=(2.5, 0.0, 1.0), sq=None) == INVALID
    assert call3d(lib, ws=None) == INVALID
    assert call3d(lib, ws_bytes=lib.edt3d_workspace_size(2, 8, 8, 8) - 1) == SMALL
    assert call3d(lib, idx=IDX + 1) == INVALID
    assert call3d(lib, dist=WS) == INVALID
    # a volume over 2^31-1 elements cannot return int32 indices
    assert call3d(lib, B=1, D=2100, H=1024, W=1000, sq=None, dist=None) == SHAPE


@fake_pointers
def test_timed_entry_rejects_without_buffer(lib):
    cnt = ctypes.c_int32(0)
    st = lib.edt2d_u8_timed(MASK, 8, 8, None, SQ, DIST, IDX, WS, BIG, None,
                            None, None, 8, ctypes.byref(cnt))
    assert st == INVALID


def test_python_binding_refuses_cpu_tensors():
    import torch
    from exact_euclidean_distance_amd import edt2d
    with pytest.raises(ValueError):
        edt2d(torch.zeros((4, 4), dtype=torch.uint8))
    with pytest.raises(TypeError):
        edt2d(torch.zeros((4, 4), dtype=torch.float32))


def call2db(lib, mask=MASK, B=3, H=64, W=64, sampling=None, sq=SQ, dist=DIST, idx=IDX, ws=WS,
            ws_bytes=BIG):
    samp = None if sampling is None else (ctypes.c_float * 2)(*sampling)
    return lib.edt2d_u8_batched(mask, B, H, W, samp, sq, dist, idx, ws, ws_bytes, None)


def call1d(lib, mask=MASK, B=3, N=64, sampling=None, sq=SQ, dist=DIST, idx=IDX, ws=WS,
           ws_bytes=BIG):
    samp = None if sampling is None else (ctypes.c_float * 1)(*sampling)
    return lib.edt1d_u8_batched(mask, B, N, samp, sq, dist, idx, ws, ws_bytes, None)


@fake_pointers
def test_batched_2d_and_1d_argument_errors(lib):
    assert lib.edt2d_batched_workspace_size(1, 64, 64) == lib.edt2d_workspace_size(64, 64)
    assert lib.edt2d_batched_workspace_size(4, 64, 64) >= 4 * 64 * 64 * 2
    assert lib.edt2d_batched_workspace_size(0, 64, 64) == 0
    assert lib.edt2d_batched_workspace_size(70000, 8, 8) == 0
    assert lib.edt1d_workspace_size(5, 100) == lib.edt2d_batched_workspace_size(5, 100, 1)
    assert call2db(lib, mask=None) == INVALID
    assert call2db(lib, B=0) == INVALID
    assert call2db(lib, B=70000) == SHAPE
    assert call2db(lib, W=40000) == SHAPE
    assert call2db(lib, sampling=(2.0, 1.0)) == INVALID
    assert call2db(lib, ws_bytes=lib.edt2d_batched_workspace_size(3, 64, 64) - 1) == SMALL
    # the outputs of a batch span B images: an output starting inside the
    # third image's part of another output aliases it
    assert call2db(lib, dist=SQ + 2 * 64 * 64 * 4) == INVALID
    assert call2db(lib, sq=None, dist=None, idx=None) == INVALID
    assert call1d(lib, mask=None) == INVALID
    assert call1d(lib, N=0) == INVALID
    assert call1d(lib, N=70000) == SHAPE
    assert call1d(lib, sampling=(2.0,)) == INVALID           # sqdist needs unit spacing
    assert call1d(lib, sampling=(0.0,), sq=None) == INVALID
    assert call1d(lib, ws_bytes=lib.edt1d_workspace_size(3, 64) - 1) == SMALL


@fake_pointers
def test_unravel_argument_errors(lib):
    shp = (ctypes.c_int32 * 3)(4, 5, 6)
    assert lib.edt_unravel_indices(None, 1, 3, shp, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 1, 3, shp, None, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 1, 3, None, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 0, 3, shp, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 1, 4, shp, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 1, 0, shp, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX + 2, 1, 3, shp, DIST, None) == INVALID
    assert lib.edt_unravel_indices(IDX, 1, 3, shp, IDX + 16, None) == INVALID   # overlap
    bad = (ctypes.c_int32 * 3)(4, 0, 6)
    assert lib.edt_unravel_indices(IDX, 1, 3, bad, DIST, None) == INVALID
    big = (ctypes.c_int32 * 3)(65535, 65535, 2)
    assert lib.edt_unravel_indices(IDX, 1, 3, big, DIST, None) == SHAPE


@fake_pointers
def test_brute_argument_errors(lib):
    shp = (ctypes.c_int32 * 3)(8, 9, 10)
    need = lib.edt_brute_workspace_size(2, 3, shp)
    assert need >= 2 * 8 * 9 * 10 * 4
    assert lib.edt_brute_workspace_size(2, 4, shp) == 0
    assert lib.edt_brute_workspace_size(0, 3, shp) == 0

    def call(mask=MASK, B=2, ndim=3, shape=shp, sampling=None, sq=SQ, dist=DIST, idx=IDX, ws=WS,
             ws_bytes=BIG):
        samp = None if sampling is None else (ctypes.c_float * ndim)(*sampling)
        return lib.edt_brute_u8(mask, B, ndim, shape, samp, sq, dist, idx, ws, ws_bytes, None)

    assert call(mask=None) == INVALID
    assert call(B=0) == INVALID
    assert call(ndim=0) == INVALID
    assert call(ndim=4) == INVALID
    assert call(shape=None) == INVALID
    assert call(shape=(ctypes.c_int32 * 3)(8, 0, 10)) == INVALID
    assert call(shape=(ctypes.c_int32 * 3)(8, 70000, 10)) == SHAPE
    assert call(B=70000) == SHAPE
    assert call(sampling=(2.0, 1.0, 1.0)) == INVALID          # sqdist needs unit spacing
    assert call(sampling=(2.0, -1.0, 1.0), sq=None) == INVALID
    assert call(ws_bytes=need - 1) == SMALL
    assert call(sq=None, dist=None, idx=None) == INVALID
    assert call(idx=SQ + 4) == INVALID


@fake_pointers
def test_brute_metric_argument_errors(lib):
    shp = (ctypes.c_int32 * 2)(40, 50)
    need = lib.edt_brute_workspace_size(3, 2, shp)
    assert need >= 3 * 40 * 50 * 4

    def call(mask=MASK, B=3, ndim=2, shape=shp, metric=1, dist=SQ, idx=IDX, ws=WS, ws_bytes=BIG):
        return lib.edt_brute_metric_u8(mask, B, ndim, shape, metric, dist, idx, ws, ws_bytes, None)

    assert call(mask=None) == INVALID
    assert call(metric=0) == INVALID
    assert call(metric=3) == INVALID
    assert call(ndim=4) == INVALID
    assert call(shape=(ctypes.c_int32 * 2)(40, 0)) == INVALID
    assert call(shape=(ctypes.c_int32 * 2)(40, 70000)) == SHAPE
    assert call(ws_bytes=need - 1) == SMALL
    assert call(dist=None, idx=None) == INVALID
    assert call(dist=SQ + 2) == INVALID
    assert call(ws=WS + 8) == INVALID


@fake_pointers
def test_idx64_argument_errors(lib):
    def call(idx=IDX, **kw):
        a = dict(mask=MASK, B=2, D=8, H=8, W=8, samp=None, sq=SQ, dist=DIST, ws=WS, ws_bytes=BIG)
        a.update(kw)
        return lib.edt3d_u8_batched_idx64(a["mask"], a["B"], a["D"], a["H"], a["W"], a["samp"],
                                          a["sq"], a["dist"], idx, a["ws"], a["ws_bytes"], None)
    assert call(mask=None) == INVALID
    assert call(idx=IDX + 4) == INVALID                  # int64 indices need 8-byte alignment
    assert call(idx=SQ + 8) == INVALID                   # overlaps sqdist
    assert call(sq=IDX + 4096) == INVALID                # sqdist inside the int64 indices (2*8*8*8*8 B)
    assert call(ws_bytes=lib.edt3d_workspace_size(2, 8, 8, 8) - 1) == SMALL
    assert call(H=40000) == SHAPE


@fake_pointers
@pytest.mark.parametrize("metric", ["taxicab", "chessboard"])
def test_chamfer_argument_errors(lib, metric):
    f2 = getattr(lib, f"edt2d_{metric}_u8_batched")
    f3 = getattr(lib, f"edt3d_{metric}_u8_batched")

    def c2(mask=MASK, B=2, H=8, W=8, dist=DIST, idx=IDX, ws=WS, ws_bytes=BIG):
        return f2(mask, B, H, W, dist, idx, ws, ws_bytes, None)

    def c3(mask=MASK, B=2, D=8, H=8, W=8, dist=DIST, idx=IDX, ws=WS, ws_bytes=BIG):
        return f3(mask, B, D, H, W, dist, idx, ws, ws_bytes, None)

    assert c2(mask=None) == INVALID
    assert c2(B=0) == INVALID
    assert c2(W=40000) == SHAPE
    assert c2(dist=None, idx=None) == INVALID
    assert c2(dist=DIST + 2) == INVALID
    assert c2(idx=DIST) == INVALID
    assert c2(ws_bytes=lib.edt2d_batched_workspace_size(2, 8, 8) - 1) == SMALL
    assert c3(mask=None) == INVALID
    assert c3(D=0) == INVALID
    assert c3(W=20000) == SHAPE
    assert c3(B=1, D=2100, H=1024, W=1000) == SHAPE      # int32 indices of > 2^31 elements
    assert c3(ws_bytes=lib.edt3d_workspace_size(2, 8, 8, 8) - 1) == SMALL


def _i64(vals):
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def callnd(lib, shape=(4, 5, 6, 7), nbatch=0, strides=None, sampling=None, sq=SQ, dist=DIST,
           idx=IDX, ib=4, ws=WS, ws_bytes=BIG, mask=MASK):
    ndim = len(shape) - nbatch
    samp = None if sampling is None else (ctypes.c_float * len(sampling))(*sampling)
    strd = None if strides is None else _i64(strides)
    return lib.edt_nd_u8(mask, nbatch, ndim, _i64(shape), strd, samp, sq, dist, idx, ib, ws, ws_bytes,
                         None)


def test_nd_workspace_sizes(lib):
    ws = lambda shape, nb=0, strides=None, ib=4: lib.edt_nd_workspace_size(   # noqa: E731
        nb, len(shape) - nb, _i64(shape), None if strides is None else _i64(strides), ib)
    # C-contiguous 2-D / 3-D shapes within the LDS limits take those kernels' workspace
    assert ws((512, 512)) == lib.edt2d_workspace_size(512, 512)
    assert ws((16, 128, 128, 128), nb=1) == lib.edt3d_workspace_size(16, 128, 128, 128)
    assert ws((3, 5, 7, 9), nb=2) == lib.edt2d_batched_workspace_size(15, 7, 9)
    # rank 4 and extents over 65535 take the workspace path: 40 bytes per element
    for shape, kw in (((4, 5, 6, 7), {}), ((70000, 3), {})):
        n = int(np.prod(shape))
        assert ws(shape, **kw) >= 40 * n, (shape, kw)
    # strided masks, int64 2-D indices and rows past the LDS kernels take a
    # reordered run: the gathered mask, the permuted int32 index, sqdist and
    # dist (13 bytes per element, each part rounded to 256 bytes), then the
    # LDS kernels' workspace for the shape in the order they take it
    rup = lambda x: (x + 255) // 256 * 256   # noqa: E731
    for shape, kw, inner in (((64, 64), {"strides": (128, 1)}, lib.edt2d_workspace_size(64, 64)),
                             ((64, 64), {"ib": 8}, lib.edt2d_workspace_size(64, 64)),
                             ((40, 40000), {}, lib.edt2d_workspace_size(40000, 40)),
                             ((2, 3, 20000), {}, lib.edt3d_workspace_size(1, 2, 20000, 3))):
        n = int(np.prod(shape))
        assert ws(shape, **kw) == rup(n) + 3 * rup(4 * n) + inner, (shape, kw)
    assert ws((4, 5), nb=-1) == 0
    assert ws((4,) * 9) == 0
    assert ws((4, 5), ib=3) == lib.edt_nd_workspace_size(0, 2, _i64((4, 5)), None, 4)
    assert ws((4, -5)) == 0


@fake_pointers
def test_nd_argument_errors(lib):
    assert callnd(lib, mask=None) == INVALID
    assert callnd(lib, shape=(4,) * 9) == INVALID                 # spatial rank 9
    assert callnd(lib, shape=(2, 3), nbatch=2) == INVALID         # no spatial axis
    assert callnd(lib, shape=(2,) * 10, nbatch=9) == INVALID      # nine batch axes
    assert callnd(lib, shape=(4, -1, 6)) == INVALID
    assert callnd(lib, strides=(1, -1, 1, 1)) == INVALID
    assert callnd(lib, ib=3) == INVALID
    assert callnd(lib, sq=None, dist=None, idx=None) == INVALID
    assert callnd(lib, sampling=(2.0, 1.0, 1.0, 1.0)) == INVALID  # sqdist needs unit spacing
    assert callnd(lib, sampling=(1.0, 0.0, 1.0, 1.0), sq=None) == INVALID
    assert callnd(lib, ws=None) == INVALID
    assert callnd(lib, ws=WS + 8) == INVALID
    need = lib.edt_nd_workspace_size(0, 4, _i64((4, 5, 6, 7)), None, 4)
    assert callnd(lib, ws_bytes=need - 1) == SMALL
    assert callnd(lib, sq=SQ + 2) == INVALID
    assert callnd(lib, idx=IDX + 4, ib=8) == INVALID               # int64 indices 8-byte aligned
    assert callnd(lib, dist=MASK + 100) == INVALID                 # inside the mask's span
    assert callnd(lib, dist=WS + 256) == INVALID
    assert callnd(lib, shape=(50000, 50000), dist=None, idx=None) == SHAPE   # sqdist range
    assert callnd(lib, shape=(3, 1 << 31), sq=None, dist=None) == SHAPE      # int32 indices
    # an empty shape is done before any HIP call
    assert callnd(lib, shape=(4, 0, 6, 7)) == OK


@fake_pointers
def test_unravel_nd_argument_errors(lib):
    shp = _i64((3, 4, 5, 6, 7))
    assert lib.edt_unravel_indices_nd(None, 4, 2, 5, shp, IDX, None) == INVALID
    assert lib.edt_unravel_indices_nd(SQ, 3, 2, 5, shp, IDX, None) == INVALID
    assert lib.edt_unravel_indices_nd(SQ, 4, 2, 9, shp, IDX, None) == INVALID
    assert lib.edt_unravel_indices_nd(SQ, 8, 2, 5, shp, IDX + 4, None) == INVALID
    assert lib.edt_unravel_indices_nd(SQ, 4, 2, 5, shp, SQ + 8, None) == INVALID      # overlap
    assert lib.edt_unravel_indices_nd(SQ, 4, 2, 2, _i64((1 << 20, 1 << 20)), IDX, None) == SHAPE
    assert lib.edt_unravel_indices_nd(SQ, 4, 2, 2, _i64((0, 3)), IDX, None) == INVALID
