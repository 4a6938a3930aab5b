"""Thin Python binding of the C ABI: argument marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
transform runs in the library's kernels.  The keywords follow TorchMorph's
SciPy-compatible distance-transform interface (``sampling``,
``return_distances`` / ``return_indices``, preallocated outputs).
"""

from __future__ import annotations

import contextlib
import ctypes
import functools
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import EDTError


@dataclass
class EDTResult:
    sqdist: Optional[torch.Tensor]   # int32, exact squared distances
    dist: Optional[torch.Tensor]     # float32 distances
    indices: Optional[torch.Tensor]  # flat index of the nearest background (per image), int32 or int64


def _on_stream(fn):
    """Run ``fn`` with its ``stream`` argument (when given) as the current
    stream, so that every tensor it allocates (workspace and outputs) belongs
    to the stream the kernels are enqueued on: the caching allocator then
    hands a freed workspace out again only after that stream's work."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        s = kwargs.get("stream")
        ctx = torch.cuda.stream(s) if s is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, **kwargs)
    return wrapper


def workspace_size_2d(H: int, W: int) -> int:
    return int(_lib.load().edt2d_workspace_size(H, W))


def workspace_size_3d(B: int, D: int, H: int, W: int) -> int:
    return int(_lib.load().edt3d_workspace_size(B, D, H, W))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer; torch allocations are at least 256-byte aligned."""
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_mask(mask: torch.Tensor, ndim: Sequence[int]):
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a torch.Tensor")
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8 (0 = background)")
    if not mask.is_cuda:
        raise ValueError("mask must be a device (HIP) tensor")
    if mask.dim() not in ndim:
        raise ValueError(f"mask must have {ndim} dimensions, got {mask.dim()}")
    if not mask.is_contiguous():
        raise ValueError("mask must be C-contiguous")


def _out(t, shape, dtype, device, want):
    if t is not None:
        if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
            raise ValueError(f"preallocated output must be contiguous {dtype} of shape {tuple(shape)}")
        return t
    if want:
        return torch.empty(shape, dtype=dtype, device=device)
    return None


def _sampling(sampling, n):
    if sampling is None:
        return None
    vals = [float(s) for s in sampling]
    if len(vals) != n:
        raise ValueError(f"sampling needs {n} values")
    return (ctypes.c_float * n)(*vals)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size_2d_batched(B: int, H: int, W: int) -> int:
    return int(_lib.load().edt2d_batched_workspace_size(B, H, W))


def _timed_call(fn, name, args):
    ms = (ctypes.c_float * 8)()
    names = (ctypes.c_char_p * 8)()
    cnt = ctypes.c_int32(0)
    st = fn(*args, ms, names, 8, ctypes.byref(cnt))
    if st != 0:
        raise EDTError(st, name)
    return [(names[i].decode(), ms[i]) for i in range(cnt.value)]


@_on_stream
def edt2d(mask: torch.Tensor, sampling=None, *, return_distances: bool = True,
          return_sqdist: bool = False, return_indices: bool = False,
          dist=None, sqdist=None, indices=None, workspace=None, stream=None,
          timed: bool = False, method: str = "separable"):
    """Exact EDT of one (H, W) uint8 mask, or of a batch (B, H, W) or
    (B, C, H, W) of independent images (indices flat within each image).
    ``method="proximate"`` runs PR-EDT's row-recursive proximate-point row
    pass instead of the separable envelope (same result; W <= 16384).
    Returns :class:`EDTResult` (and the per-kernel times in ms when ``timed``)."""
    if method not in ("separable", "proximate"):
        raise ValueError("method must be 'separable' or 'proximate'")
    _check_mask(mask, (2, 3, 4))
    m3 = mask if mask.dim() == 3 else (mask.unsqueeze(0) if mask.dim() == 2 else mask.flatten(0, 1))
    B, H, W = m3.shape
    shape = tuple(mask.shape)
    dev = mask.device
    sq = _out(sqdist, shape, torch.int32, dev, return_sqdist)
    ds = _out(dist, shape, torch.float32, dev, return_distances)
    ix = _out(indices, shape, torch.int32, dev, return_indices)
    lib = _lib.load()
    if method == "proximate":
        need = int(lib.edt2d_proximate_workspace_size(B, H, W))
        if need == 0:
            raise EDTError(2, "edt2d_proximate_workspace_size")
    else:
        need = int(lib.edt2d_batched_workspace_size(B, H, W))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    samp = _sampling(sampling, 2)
    wsb = workspace.numel() * workspace.element_size()
    if method == "proximate":
        if B > 65535:
            raise ValueError("at most 65535 images per call")
        args = [_ptr(mask), B, H, W, samp, _ptr(sq), _ptr(ds), _ptr(ix), _ptr(workspace), wsb,
                _stream(stream)]
        fn, tfn, name = (lib.edt2d_proximate_u8_batched, lib.edt2d_proximate_u8_batched_timed,
                         "edt2d_proximate_u8_batched")
    elif mask.dim() == 2:
        args = [_ptr(mask), H, W, samp, _ptr(sq), _ptr(ds), _ptr(ix), _ptr(workspace), wsb,
                _stream(stream)]
        fn, tfn, name = lib.edt2d_u8, lib.edt2d_u8_timed, "edt2d_u8"
    else:
        if B > 65535:
            raise ValueError("at most 65535 images per call")
        args = [_ptr(mask), B, H, W, samp, _ptr(sq), _ptr(ds), _ptr(ix), _ptr(workspace), wsb,
                _stream(stream)]
        fn, tfn, name = lib.edt2d_u8_batched, lib.edt2d_u8_batched_timed, "edt2d_u8_batched"
    if not timed:
        st = fn(*args)
        if st != 0:
            raise EDTError(st, name)
        return EDTResult(sq, ds, ix)
    return EDTResult(sq, ds, ix), _timed_call(tfn, name + "_timed", args)


@_on_stream
def edt1d(mask: torch.Tensor, sampling=None, *, return_distances: bool = True,
          return_sqdist: bool = False, return_indices: bool = False,
          dist=None, sqdist=None, indices=None, workspace=None, stream=None):
    """Exact distance transform of one (N,) uint8 line or a batch (B, N) of
    independent lines; indices are positions within each line (-1: the
    virtual element of a line without background)."""
    _check_mask(mask, (1, 2))
    m2 = mask if mask.dim() == 2 else mask.unsqueeze(0)
    B, N = m2.shape
    shape = tuple(mask.shape)
    dev = mask.device
    sq = _out(sqdist, shape, torch.int32, dev, return_sqdist)
    ds = _out(dist, shape, torch.float32, dev, return_distances)
    ix = _out(indices, shape, torch.int32, dev, return_indices)
    lib = _lib.load()
    need = int(lib.edt1d_workspace_size(B, N))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    samp = _sampling(sampling, 1)
    st = lib.edt1d_u8_batched(_ptr(m2), B, N, samp, _ptr(sq), _ptr(ds), _ptr(ix), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise EDTError(st, "edt1d_u8_batched")
    return EDTResult(sq, ds, ix)


@_on_stream
def unravel_indices(indices: torch.Tensor, image_shape: Sequence[int], *, out=None, stream=None):
    """Per-axis coordinates of flat indices returned by the transforms:
    (*batch, *image_shape) int32 or int64 -> (*batch, ndim, *image_shape) of the
    same type, the layout of SciPy's feature transform (virtual index ->
    (-1, 0, ...)); images of 1 to 8 axes."""
    if not isinstance(indices, torch.Tensor) or indices.dtype not in (torch.int32, torch.int64):
        raise TypeError("indices must be an int32 or int64 torch.Tensor")
    if not indices.is_cuda or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous device tensor")
    img = tuple(int(s) for s in image_shape)
    nd = len(img)
    if tuple(indices.shape[indices.dim() - nd:]) != img:
        raise ValueError(f"indices must end with the image shape {img}")
    batch = tuple(indices.shape[:indices.dim() - nd])
    images = 1
    for b in batch:
        images *= int(b)
    shape = batch + (nd,) + img
    coords = _out(out, shape, indices.dtype, indices.device, True)
    if indices.dtype == torch.int32 and nd <= 3:
        shp = (ctypes.c_int32 * nd)(*img)
        st = _lib.load().edt_unravel_indices(_ptr(indices), images, nd, shp, _ptr(coords),
                                             _stream(stream))
        if st != 0:
            raise EDTError(st, "edt_unravel_indices")
        return coords
    ib = 8 if indices.dtype == torch.int64 else 4
    st = _lib.load().edt_unravel_indices_nd(_ptr(indices), ib, images, nd, _i64(img), _ptr(coords),
                                            _stream(stream))
    if st != 0:
        raise EDTError(st, "edt_unravel_indices_nd")
    return coords


@_on_stream
def edt_brute(mask: torch.Tensor, sampling=None, *, batched: bool = False,
              return_distances: bool = True, return_sqdist: bool = False,
              return_indices: bool = False, dist=None, sqdist=None, indices=None,
              workspace=None, stream=None, metric: str = "euclidean"):
    """The transform by its definition on the device (every element against
    every background element): an exactness check.  mask is one image of 1-3
    axes, or a batch of them (leading axis) when ``batched``.  ``metric``
    "taxicab" or "chessboard" gives those transforms instead (int32
    distances in ``dist``, no spacing, no sqdist)."""
    _check_mask(mask, (1, 2, 3, 4))
    img = tuple(mask.shape[1:]) if batched else tuple(mask.shape)
    B = int(mask.shape[0]) if batched else 1
    if not 1 <= len(img) <= 3:
        raise ValueError("images must have 1 to 3 axes")
    if metric not in ("euclidean", "taxicab", "chessboard"):
        raise ValueError("metric must be 'euclidean', 'taxicab' or 'chessboard'")
    shape = tuple(mask.shape)
    dev = mask.device
    lib = _lib.load()
    shp = (ctypes.c_int32 * len(img))(*img)
    need = int(lib.edt_brute_workspace_size(B, len(img), shp))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    wsb = workspace.numel() * workspace.element_size()
    if metric != "euclidean":
        if sampling is not None or return_sqdist or sqdist is not None:
            raise ValueError("the chamfer metrics take no spacing and give no sqdist")
        ds = _out(dist, shape, torch.int32, dev, return_distances)
        ix = _out(indices, shape, torch.int32, dev, return_indices)
        code = 1 if metric == "taxicab" else 2
        st = lib.edt_brute_metric_u8(_ptr(mask), B, len(img), shp, code, _ptr(ds), _ptr(ix),
                                     _ptr(workspace), wsb, _stream(stream))
        if st != 0:
            raise EDTError(st, "edt_brute_metric_u8")
        return EDTResult(None, ds, ix)
    sq = _out(sqdist, shape, torch.int32, dev, return_sqdist)
    ds = _out(dist, shape, torch.float32, dev, return_distances)
    ix = _out(indices, shape, torch.int32, dev, return_indices)
    samp = _sampling(sampling, len(img))
    st = lib.edt_brute_u8(_ptr(mask), B, len(img), shp, samp, _ptr(sq), _ptr(ds), _ptr(ix),
                          _ptr(workspace), wsb, _stream(stream))
    if st != 0:
        raise EDTError(st, "edt_brute_u8")
    return EDTResult(sq, ds, ix)


def _chamfer(metric: str, mask: torch.Tensor, return_indices: bool, dist, indices, workspace, stream):
    _check_mask(mask, (2, 3, 4))
    shape = tuple(mask.shape)
    dev = mask.device
    ds = _out(dist, shape, torch.int32, dev, True)
    ix = _out(indices, shape, torch.int32, dev, return_indices)
    lib = _lib.load()
    if mask.dim() == 4:
        B, D, H, W = shape
        need = int(lib.edt3d_workspace_size(B, D, H, W))
    else:
        B, H, W = (1,) + shape if mask.dim() == 2 else shape
        need = int(lib.edt2d_batched_workspace_size(B, H, W))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    wsb = workspace.numel() * workspace.element_size()
    if mask.dim() == 4:
        fn = getattr(lib, f"edt3d_{metric}_u8_batched")
        st = fn(_ptr(mask), B, D, H, W, _ptr(ds), _ptr(ix), _ptr(workspace), wsb, _stream(stream))
    else:
        fn = getattr(lib, f"edt2d_{metric}_u8_batched")
        st = fn(_ptr(mask), B, H, W, _ptr(ds), _ptr(ix), _ptr(workspace), wsb, _stream(stream))
    if st != 0:
        raise EDTError(st, metric)
    return EDTResult(None, ds, ix)


@_on_stream
def taxicab(mask: torch.Tensor, *, return_indices: bool = False, dist=None, indices=None,
            workspace=None, stream=None):
    """City-block (L1) distance transform: int32 distances (and flat indices)
    of one (H, W) image, a batch (B, H, W), or a batch of volumes
    (B, D, H, W)."""
    return _chamfer("taxicab", mask, return_indices, dist, indices, workspace, stream)


@_on_stream
def chessboard(mask: torch.Tensor, *, return_indices: bool = False, dist=None, indices=None,
               workspace=None, stream=None):
    """Chessboard (L-infinity) distance transform: int32 distances (and flat
    indices) of one (H, W) image, a batch (B, H, W), or a batch of volumes
    (B, D, H, W)."""
    return _chamfer("chessboard", mask, return_indices, dist, indices, workspace, stream)


@_on_stream
def edt3d(mask: torch.Tensor, sampling=None, *, return_distances: bool = True,
          return_sqdist: bool = False, return_indices: bool = False,
          dist=None, sqdist=None, indices=None, workspace=None, stream=None,
          timed: bool = False, index_dtype=torch.int32):
    """Exact EDT of a batch of volumes, mask (B, D, H, W), (B, C, D, H, W) or
    (D, H, W) uint8.  Indices are flat within each volume;
    ``index_dtype=torch.int64`` returns them as int64 (volumes over 2^31 - 1
    elements)."""
    if index_dtype not in (torch.int32, torch.int64):
        raise ValueError("index_dtype must be torch.int32 or torch.int64")
    _check_mask(mask, (3, 4, 5))
    m4 = mask if mask.dim() == 4 else (mask.unsqueeze(0) if mask.dim() == 3 else mask.flatten(0, 1))
    B, D, H, W = m4.shape
    shape = tuple(mask.shape)
    dev = mask.device
    sq = _out(sqdist, shape, torch.int32, dev, return_sqdist)
    ds = _out(dist, shape, torch.float32, dev, return_distances)
    ix = _out(indices, shape, index_dtype, dev, return_indices)
    lib = _lib.load()
    need = int(lib.edt3d_workspace_size(B, D, H, W))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    samp = _sampling(sampling, 3)
    args = [_ptr(m4), B, D, H, W, samp, _ptr(sq), _ptr(ds), _ptr(ix), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if index_dtype == torch.int64:
        if timed:
            raise ValueError("timed calls return int32 indices")
        st = lib.edt3d_u8_batched_idx64(*args)
        if st != 0:
            raise EDTError(st, "edt3d_u8_batched_idx64")
        return EDTResult(sq, ds, ix)
    if not timed:
        st = lib.edt3d_u8_batched(*args)
        if st != 0:
            raise EDTError(st, "edt3d_u8_batched")
        return EDTResult(sq, ds, ix)
    return EDTResult(sq, ds, ix), _timed_call(lib.edt3d_u8_batched_timed, "edt3d_u8_batched_timed",
                                              args)


def _i64(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


@_on_stream
def edt(mask: torch.Tensor, sampling=None, *, batch_dims: int = 0, return_distances: bool = True,
        return_sqdist: bool = False, return_indices: bool = False, index_dtype=torch.int32,
        dist=None, sqdist=None, indices=None, workspace=None, stream=None):
    """Exact EDT of a uint8 mask of any spatial rank (1..8) after
    ``batch_dims`` leading batch axes, e.g. (B, C, D, H, W, T) with
    ``batch_dims=2``.  The mask may be a strided view (slices, transposes);
    outputs are contiguous with the mask's shape.  Indices are flat within each
    image, int32 or int64 (``index_dtype``).  Shapes the LDS kernels take run
    there; the rest (rank 4+, strided masks, long rows, extents over 65535)
    run the workspace path of the same method."""
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a torch.Tensor")
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8 (0 = background)")
    if not mask.is_cuda:
        raise ValueError("mask must be a device (HIP) tensor")
    if index_dtype not in (torch.int32, torch.int64):
        raise ValueError("index_dtype must be torch.int32 or torch.int64")
    ndim = mask.dim() - int(batch_dims)
    if batch_dims < 0 or not 1 <= ndim <= 8:
        raise ValueError("need 1 to 8 spatial axes after the batch axes")
    shape = tuple(mask.shape)
    dev = mask.device
    sq = _out(sqdist, shape, torch.int32, dev, return_sqdist)
    ds = _out(dist, shape, torch.float32, dev, return_distances)
    ix = _out(indices, shape, index_dtype, dev, return_indices)
    ib = 8 if index_dtype == torch.int64 else 4
    lib = _lib.load()
    shp = _i64(shape)
    strd = _i64(mask.stride())
    need = int(lib.edt_nd_workspace_size(int(batch_dims), ndim, shp, strd, ib))
    if need == 0:
        raise EDTError(1, "edt_nd_workspace_size")
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    samp = _sampling(sampling, ndim)
    st = lib.edt_nd_u8(_ptr(mask), int(batch_dims), ndim, shp, strd, samp, _ptr(sq), _ptr(ds), _ptr(ix),
                       ib, _ptr(workspace), workspace.numel() * workspace.element_size(),
                       _stream(stream))
    if st != 0:
        raise EDTError(st, "edt_nd_u8")
    return EDTResult(sq, ds, ix)
