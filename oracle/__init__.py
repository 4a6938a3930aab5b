"""CPU oracle for the exact Euclidean distance transform -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``exact_euclidean_distance_amd``) and never imports it.

* :func:`edt` -- the separable serial scheme in ``oracle_edt.c`` (float64).
* :func:`edt_brute` -- the definition, every element against every background
  element, in the same C file (``oracle_edt_brute``).
* :func:`brute_numpy` -- an independent NumPy transcription of the definition.
* :func:`taxicab_brute` / :func:`taxicab_to` -- the city-block (L1) distance
  transform by its definition, and the L1 distance to a given flat index (for
  the chamfer transforms TorchMorph ships beside its EDT; the pages name them
  without defining them -- read as the L1 metric, as SciPy's ``taxicab``).

Pinning (see ``tests/test_oracle.py``): hand-derived fixtures under
``tests/golden/``, closed forms (one background element, full background
row/plane, two background elements, all background, no background), the 1-D
case against ``numpy.searchsorted``, SciPy's ``distance_transform_edt`` on
distances, exact equality with both brute forces on every small random mask,
and planted-mistake runs showing each of those pins catches a wrong oracle.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_edt.c")
_LIB = os.path.join(_HERE, "liboracle_edt.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the C oracle with gcc (plain -O2, single thread)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", out, src, "-lm", *extra]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building if absent) the oracle library; returns the ctypes handle."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        path = _LIB
    lib = ctypes.CDLL(path)
    for name in ("oracle_edt_separable", "oracle_edt_brute"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_void_p, ctypes.c_void_p]
    if path == _LIB:
        _lib = lib
    return lib


def _run(fname, mask, sampling, want_feature, lib=None):
    lib = lib or load()
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    ndim = mask.ndim
    shape = np.asarray(mask.shape, dtype=np.int64)
    samp = None
    if sampling is not None:
        samp = np.asarray(sampling, dtype=np.float64)
        if samp.shape != (ndim,):
            raise ValueError("sampling must have one entry per axis")
    sq = np.empty(mask.shape, np.float64)
    feat = np.empty(mask.shape + (ndim,), np.int32) if want_feature else None
    rc = getattr(lib, fname)(
        mask.ctypes.data, ndim, shape.ctypes.data,
        samp.ctypes.data if samp is not None else None,
        sq.ctypes.data, feat.ctypes.data if feat is not None else None)
    if rc != 0:
        raise RuntimeError(f"{fname} failed with {rc}")
    return sq, feat


def edt(mask, sampling=None, features=True, lib=None):
    """Separable oracle for one image: ``(sqdist float64, feature int32 [..., ndim])``."""
    return _run("oracle_edt_separable", mask, sampling, features, lib)


def edt_brute(mask, sampling=None, features=True, lib=None):
    """Brute force (the definition) in C for one image."""
    return _run("oracle_edt_brute", mask, sampling, features, lib)


def edt_batch(masks, sampling=None, features=True, lib=None):
    """Apply :func:`edt` to each image of a batch (leading axis)."""
    sqs, feats = [], []
    for m in masks:
        s, f = edt(m, sampling, features, lib)
        sqs.append(s)
        feats.append(f)
    return np.stack(sqs), (np.stack(feats) if features else None)


def brute_numpy(mask, sampling=None):
    """Independent NumPy transcription of the definition: for every element the
    minimum over all background elements of sum_k s_k^2 (p_k - b_k)^2.  Returns
    float64 squared distances (virtual background (-1, 0, ...) if none)."""
    mask = np.asarray(mask)
    shape = mask.shape
    s2 = np.ones(mask.ndim) if sampling is None else np.asarray(sampling, np.float64) ** 2
    coords = np.indices(shape).reshape(mask.ndim, -1).T.astype(np.float64)
    bg = coords[mask.reshape(-1) == 0]
    if len(bg) == 0:
        bg = np.zeros((1, mask.ndim))
        bg[0, 0] = -1.0
    out = np.empty(len(coords))
    step = max(1, (1 << 22) // len(bg))
    for i in range(0, len(coords), step):
        diff = coords[i:i + step, None, :] - bg[None, :, :]
        out[i:i + step] = (diff * diff * s2).sum(-1).min(1)
    return out.reshape(shape)


def flat_index(feature, shape):
    """Row-major flat index of feature coordinates within their image (int64);
    the virtual background (-1, 0, ...) maps to -(shape[1]*...*shape[-1])."""
    feature = np.asarray(feature, np.int64)
    strides = np.ones(len(shape), np.int64)
    for k in range(len(shape) - 2, -1, -1):
        strides[k] = strides[k + 1] * shape[k + 1]
    return (feature * strides).sum(-1)


def sqdist_to(feature_flat, shape, sampling=None):
    """Squared distance from every element to the element at the given flat index
    (same image), float64 -- used to check that a returned index attains the
    minimum.  Negative indices are decoded as the virtual background."""
    shape = tuple(shape)
    ndim = len(shape)
    s2 = np.ones(ndim) if sampling is None else np.asarray(sampling, np.float64) ** 2
    idx_all = np.asarray(feature_flat, np.int64).reshape(shape)
    inner = int(np.prod(shape[1:])) if ndim > 1 else 1
    out = np.empty(shape, np.float64)
    rows = max(1, (1 << 22) // inner)
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        idx = idx_all[r0:r1]
        # decode: axis 0 may be -1 for the virtual background
        a0 = np.floor_divide(idx, inner)
        rest = idx - a0 * inner
        comps = [a0]
        for k in range(1, ndim):
            st = int(np.prod(shape[k + 1:])) if k + 1 < ndim else 1
            comps.append(rest // st)
            rest = rest % st
        sub = (r1 - r0,) + shape[1:]
        grid = np.indices(sub)
        grid[0] += r0
        d = np.zeros(sub, np.float64)
        for k in range(ndim):
            t = (grid[k] - comps[k]).astype(np.float64)
            d += s2[k] * t * t
        out[r0:r1] = d
    return out


def taxicab_brute(mask):
    """City-block (L1) distance transform by its definition: for every element
    the minimum over all background elements of sum_k |p_k - b_k| (int64);
    without background, the virtual element at (-1, 0, ...).  Also returns the
    flat index of the first (smallest-index) minimiser."""
    mask = np.asarray(mask)
    shape = mask.shape
    coords = np.indices(shape).reshape(mask.ndim, -1).T.astype(np.int64)
    bgi = np.flatnonzero(mask.reshape(-1) == 0)
    if len(bgi) == 0:
        bg = np.zeros((1, mask.ndim), np.int64)
        bg[0, 0] = -1
        bgi = np.array([-(int(np.prod(shape[1:])) if mask.ndim > 1 else 1)])
    else:
        bg = coords[bgi]
    out = np.empty(len(coords), np.int64)
    who = np.empty(len(coords), np.int64)
    step = max(1, (1 << 22) // len(bg))
    for i in range(0, len(coords), step):
        d = np.abs(coords[i:i + step, None, :] - bg[None, :, :]).sum(-1)
        k = d.argmin(1)
        out[i:i + step] = d[np.arange(len(k)), k]
        who[i:i + step] = bgi[k]
    return out.reshape(shape), who.reshape(shape)


def chessboard_brute(mask):
    """Chessboard (L-infinity) distance transform by its definition: for every
    element the minimum over all background elements of max_k |p_k - b_k|
    (int64); without background, the virtual element at (-1, 0, ...).  Also
    returns the flat index of the first (smallest-index) minimiser."""
    mask = np.asarray(mask)
    shape = mask.shape
    coords = np.indices(shape).reshape(mask.ndim, -1).T.astype(np.int64)
    bgi = np.flatnonzero(mask.reshape(-1) == 0)
    if len(bgi) == 0:
        bg = np.zeros((1, mask.ndim), np.int64)
        bg[0, 0] = -1
        bgi = np.array([-(int(np.prod(shape[1:])) if mask.ndim > 1 else 1)])
    else:
        bg = coords[bgi]
    out = np.empty(len(coords), np.int64)
    who = np.empty(len(coords), np.int64)
    step = max(1, (1 << 22) // len(bg))
    for i in range(0, len(coords), step):
        d = np.abs(coords[i:i + step, None, :] - bg[None, :, :]).max(-1)
        k = d.argmin(1)
        out[i:i + step] = d[np.arange(len(k)), k]
        who[i:i + step] = bgi[k]
    return out.reshape(shape), who.reshape(shape)


def chessboard_at(mask, points):
    """Chessboard (L-infinity) distance by its definition at the elements with
    the given flat indices, one by one (int64; virtual element without
    background).  For sampled checks of large images."""
    mask = np.asarray(mask)
    pts = np.stack(np.unravel_index(np.asarray(points, np.int64), mask.shape), 1).astype(np.int64)
    bg = np.argwhere(mask == 0).astype(np.int64)
    if len(bg) == 0:
        bg = np.zeros((1, mask.ndim), np.int64)
        bg[0, 0] = -1
    out = np.empty(len(pts), np.int64)
    for i, p in enumerate(pts):
        out[i] = np.abs(bg - p[None, :]).max(1).min()
    return out


def chessboard_to(feature_flat, shape):
    """L-infinity distance from every element to the element at the given flat
    index (same image); negative indices are decoded as the virtual background
    (floor division: -(n1 * ... ) becomes (-1, 0, ...))."""
    shape = tuple(shape)
    ndim = len(shape)
    idx = np.asarray(feature_flat, np.int64).reshape(shape)
    inner = int(np.prod(shape[1:])) if ndim > 1 else 1
    a0 = np.floor_divide(idx, inner)
    rest = idx - a0 * inner
    comps = [a0]
    for k in range(1, ndim):
        st = int(np.prod(shape[k + 1:])) if k + 1 < ndim else 1
        comps.append(rest // st)
        rest = rest % st
    grid = np.indices(shape)
    return np.max([np.abs(grid[k] - comps[k]) for k in range(ndim)], axis=0)


def taxicab_at(mask, points):
    """City-block (L1) distance by its definition at the elements with the given
    flat indices, one by one: the minimum over all background elements of
    sum_k |p_k - b_k| (int64); without background, the virtual element at
    (-1, 0, ...).  For sampled checks of images too large for taxicab_brute."""
    mask = np.asarray(mask)
    pts = np.stack(np.unravel_index(np.asarray(points, np.int64), mask.shape), 1).astype(np.int64)
    bg = np.argwhere(mask == 0).astype(np.int64)
    if len(bg) == 0:
        bg = np.zeros((1, mask.ndim), np.int64)
        bg[0, 0] = -1
    out = np.empty(len(pts), np.int64)
    for i, p in enumerate(pts):
        out[i] = np.abs(bg - p[None, :]).sum(1).min()
    return out


def taxicab_to(feature_flat, shape):
    """L1 distance from every element to the element at the given flat index
    (same image); negative indices are decoded as the virtual background."""
    shape = tuple(shape)
    ndim = len(shape)
    idx = np.asarray(feature_flat, np.int64).reshape(shape)
    inner = int(np.prod(shape[1:])) if ndim > 1 else 1
    a0 = np.floor_divide(idx, inner)
    rest = idx - a0 * inner
    comps = [a0]
    for k in range(1, ndim):
        st = int(np.prod(shape[k + 1:])) if k + 1 < ndim else 1
        comps.append(rest // st)
        rest = rest % st
    grid = np.indices(shape)
    return sum(np.abs(grid[k] - comps[k]) for k in range(ndim))
