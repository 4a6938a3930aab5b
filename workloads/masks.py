"""Seeded mask generators for the five workloads and the stress cases.

Every generator takes a ``numpy.random.Generator`` (see :func:`rng_for`) and
returns a C-contiguous ``uint8`` array with ``0`` = background and ``1`` =
foreground.  The random-image protocol (fixed seed 42, reproducible inputs)
follows "GPU-Based Parallel Euclidean Distance Transform Algorithm", §4.1
Experimental Setup; the shapes and structures are the five workloads this
library is measured on:

=====  ==========================  =============================================
name   shape                       structure
=====  ==========================  =============================================
c1     512 x 512                   background i.i.d. Bernoulli(0.01)
c2a    4096 x 4096                 foreground = union of 300 disks, r ~ U[8,400]
c2b    4096 x 4096                 one background pixel at a random location
c3     16384 x 16384               background i.i.d. Bernoulli(1e-4)
c4     16 x 128 x 128 x 128        per volume, foreground = union of 5..20
                                   axis-aligned ellipsoids, semi-axes U[5,50]
c5     512 x 512 x 512             background Bernoulli(1e-3) plus a 64-voxel
                                   background slab across axis 0;
                                   sampling (2.5, 1, 1)
=====  ==========================  =============================================

Every generator guarantees at least one background element per image (the
no-background convention is exercised by dedicated tests instead).
"""

from __future__ import annotations

import numpy as np

SEED = 42

# name -> (shape, sampling, outputs timed by the benchmark)
CONFIGS = {
    "c1": dict(shape=(512, 512), sampling=None, outputs=("sqdist", "dist", "indices")),
    "c2a": dict(shape=(4096, 4096), sampling=None, outputs=("sqdist", "dist", "indices")),
    "c2b": dict(shape=(4096, 4096), sampling=None, outputs=("sqdist", "dist", "indices")),
    "c3": dict(shape=(16384, 16384), sampling=None, outputs=("sqdist", "dist")),
    "c4": dict(shape=(16, 128, 128, 128), sampling=None, outputs=("dist",)),
    "c5": dict(shape=(1, 512, 512, 512), sampling=(2.5, 1.0, 1.0), outputs=("dist", "indices")),
    # batched 2-D (not one of the five headline workloads): 32 images shaped like c1
    "b2d": dict(shape=(32, 1024, 1024), sampling=None, outputs=("sqdist", "dist", "indices")),
    # a stack of 2048^2 slices (middle axis longer than 1024)
    "v2048": dict(shape=(1, 64, 2048, 2048), sampling=None, outputs=("dist",)),
    # shapes for the any-rank path: a 4-D array, and rows longer than the
    # LDS kernels take
    "nd4": dict(shape=(80, 80, 80, 80), sampling=(2.5, 1.0, 1.0, 1.0), outputs=("dist", "indices")),
    "w40k": dict(shape=(256, 40000), sampling=None, outputs=("sqdist", "dist", "indices")),
    # one 1-D signal of 2^22 samples (a single long line)
    "l4m": dict(shape=(1 << 22,), sampling=None, outputs=("dist", "indices")),
}
# PR-EDT's own workloads (its §4.1 and Table 1): random square images, seed 42,
# background ratio 1 % or 99 %; distances timed
for _n in (1024, 2048, 4096, 8192):
    for _pct in (1, 99):
        CONFIGS[f"p1_{_n}_{_pct}"] = dict(shape=(_n, _n), sampling=None, outputs=("dist",))

_CFG_ID = {"c1": 1, "c2a": 2, "c2b": 2, "c3": 3, "c4": 4, "c5": 5, "stress_row": 6, "b2d": 7,
           "v2048": 8, "nd4": 9, "w40k": 10, "l4m": 11}
_CFG_ID.update({f"p1_{n}_{pct}": 100 + 10 * i + pct % 10
                for i, n in enumerate((1024, 2048, 4096, 8192)) for pct in (1, 99)})
_SUB_ID = {"c2a": 0, "c2b": 1}


def rng_for(name: str, sub: int | None = None) -> np.random.Generator:
    """Generator seeded with ``[42, config id, sub id]``."""
    cfg = _CFG_ID.get(name, 99)
    if sub is None:
        sub = _SUB_ID.get(name, 0)
    return np.random.default_rng([SEED, cfg, sub])


def _ensure_background(mask: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    if not (mask == 0).any():
        flat = mask.reshape(-1)
        flat[int(rng.integers(0, flat.size))] = 0
    return mask


def bernoulli_2d(rng: np.random.Generator, H: int, W: int, p: float,
                 rows_per_chunk: int = 1024) -> np.ndarray:
    """Background i.i.d. with probability ``p``; drawn in row chunks to bound memory."""
    mask = np.empty((H, W), np.uint8)
    for r0 in range(0, H, rows_per_chunk):
        r1 = min(H, r0 + rows_per_chunk)
        u = rng.random((r1 - r0, W), dtype=np.float32)
        mask[r0:r1] = (u >= p).astype(np.uint8)
    return _ensure_background(mask, rng)


def bernoulli_3d(rng: np.random.Generator, D: int, H: int, W: int, p: float) -> np.ndarray:
    mask = np.empty((D, H, W), np.uint8)
    step = max(1, (1 << 24) // max(1, H * W))
    for d0 in range(0, D, step):
        d1 = min(D, d0 + step)
        u = rng.random((d1 - d0, H, W), dtype=np.float32)
        mask[d0:d1] = (u >= p).astype(np.uint8)
    return _ensure_background(mask, rng)


def disks_2d(rng: np.random.Generator, H: int = 4096, W: int = 4096, n: int = 300,
             rmin: float = 8.0, rmax: float = 400.0) -> np.ndarray:
    """All background, then ``n`` foreground disks; pixel (y, x) is inside a disk
    centred at (cy, cx) with radius r iff (y-cy)^2 + (x-cx)^2 <= r^2."""
    mask = np.zeros((H, W), np.uint8)
    cy = rng.uniform(0, H, n)
    cx = rng.uniform(0, W, n)
    r = rng.uniform(rmin, rmax, n)
    for k in range(n):
        y0 = max(0, int(np.floor(cy[k] - r[k])))
        y1 = min(H, int(np.ceil(cy[k] + r[k])) + 1)
        x0 = max(0, int(np.floor(cx[k] - r[k])))
        x1 = min(W, int(np.ceil(cx[k] + r[k])) + 1)
        if y0 >= y1 or x0 >= x1:
            continue
        yy = (np.arange(y0, y1, dtype=np.float64) - cy[k])[:, None]
        xx = (np.arange(x0, x1, dtype=np.float64) - cx[k])[None, :]
        inside = yy * yy + xx * xx <= r[k] * r[k]
        mask[y0:y1, x0:x1] |= inside.astype(np.uint8)
    return _ensure_background(mask, rng)


def single_pixel_2d(rng: np.random.Generator, H: int = 4096, W: int = 4096):
    """All foreground except one background pixel; returns (mask, (r0, c0))."""
    mask = np.ones((H, W), np.uint8)
    r0 = int(rng.integers(0, H))
    c0 = int(rng.integers(0, W))
    mask[r0, c0] = 0
    return mask, (r0, c0)


def full_row_2d(rng: np.random.Generator, H: int = 4096, W: int = 4096):
    """All foreground except one full background row: every candidate of every
    row pass lies on the lower envelope (the longest possible envelope)."""
    mask = np.ones((H, W), np.uint8)
    r0 = int(rng.integers(0, H))
    mask[r0, :] = 0
    return mask, r0


def ellipsoids_3d_batch(rng: np.random.Generator, B: int = 16, n: int = 128,
                        kmin: int = 5, kmax: int = 20,
                        amin: float = 5.0, amax: float = 50.0) -> np.ndarray:
    """Per volume: all background, then k ~ U{kmin..kmax} axis-aligned foreground
    ellipsoids, centre ~ U[0,n)^3, semi-axes ~ U[amin,amax] independently;
    voxel p is inside iff sum_k ((p_k - c_k) / a_k)^2 <= 1."""
    vols = np.zeros((B, n, n, n), np.uint8)
    for b in range(B):
        k = int(rng.integers(kmin, kmax + 1))
        c = rng.uniform(0, n, (k, 3))
        a = rng.uniform(amin, amax, (k, 3))
        for e in range(k):
            lo = [max(0, int(np.floor(c[e, i] - a[e, i]))) for i in range(3)]
            hi = [min(n, int(np.ceil(c[e, i] + a[e, i])) + 1) for i in range(3)]
            if any(lo[i] >= hi[i] for i in range(3)):
                continue
            z = ((np.arange(lo[0], hi[0]) - c[e, 0]) / a[e, 0])[:, None, None]
            y = ((np.arange(lo[1], hi[1]) - c[e, 1]) / a[e, 1])[None, :, None]
            x = ((np.arange(lo[2], hi[2]) - c[e, 2]) / a[e, 2])[None, None, :]
            inside = z * z + y * y + x * x <= 1.0
            vols[b, lo[0]:hi[0], lo[1]:hi[1], lo[2]:hi[2]] |= inside.astype(np.uint8)
        _ensure_background(vols[b], rng)
    return vols


def slab_volume(rng: np.random.Generator, n: int = 512, p: float = 1e-3,
                thickness: int = 64):
    """Background Bernoulli(p) plus a background slab z in [z0, z0+thickness)
    across axis 0; returns (mask, z0)."""
    mask = bernoulli_3d(rng, n, n, n, p)
    z0 = int(rng.integers(0, n - thickness + 1))
    mask[z0:z0 + thickness] = 0
    return mask, z0


def make_config(name: str, scale: int = 1):
    """Build the named workload.  Returns ``(mask, sampling, meta)``; 3D masks are
    returned with a leading batch axis ``(B, D, H, W)``.  ``scale`` > 1 divides
    every spatial extent (for quick runs of the same structure)."""
    if name == "c1":
        n = 512 // scale
        return bernoulli_2d(rng_for(name), n, n, 0.01), None, {}
    if name == "c2a":
        n = 4096 // scale
        return disks_2d(rng_for(name), n, n, 300, 8.0 / scale, 400.0 / scale), None, {}
    if name == "c2b":
        n = 4096 // scale
        m, rc = single_pixel_2d(rng_for(name), n, n)
        return m, None, {"bg": rc}
    if name == "c3":
        n = 16384 // scale
        return bernoulli_2d(rng_for(name), n, n, 1e-4), None, {}
    if name == "c4":
        n = 128 // scale
        return ellipsoids_3d_batch(rng_for(name), 16, n, 5, 20, 5.0 / scale, 50.0 / scale), None, {}
    if name == "c5":
        n = 512 // scale
        m, z0 = slab_volume(rng_for(name), n, 1e-3, max(1, 64 // scale))
        return m[None], (2.5, 1.0, 1.0), {"z0": z0}
    if name == "b2d":
        n = 1024 // scale
        rng = rng_for(name)
        return np.stack([bernoulli_2d(rng, n, n, 0.01) for _ in range(32)]), None, {}
    if name == "v2048":
        n = 2048 // scale
        return bernoulli_3d(rng_for(name), max(1, 64 // scale), n, n, 1e-3)[None], None, {}
    if name.startswith("p1_"):
        _, n, pct = name.split("_")
        n = int(n) // scale
        return bernoulli_2d(rng_for(name), n, n, int(pct) / 100.0), None, {}
    if name == "nd4":
        n = max(2, 80 // scale)
        rng = rng_for(name)
        m = np.empty((n, n, n, n), np.uint8)
        for i in range(n):   # one 3-D slab at a time
            m[i] = (rng.random((n, n, n), dtype=np.float32) >= 1e-3).astype(np.uint8)
        return _ensure_background(m, rng), (2.5, 1.0, 1.0, 1.0), {}
    if name == "w40k":
        return bernoulli_2d(rng_for(name), max(1, 256 // scale), max(1, 40000 // scale), 1e-3), None, {}
    if name == "l4m":
        rng = rng_for(name)
        return _ensure_background((rng.random(max(1, (1 << 22) // scale), dtype=np.float32) >= 1e-4)
                                  .astype(np.uint8), rng), None, {}
    if name == "stress_row":
        n = 4096 // scale
        m, r0 = full_row_2d(rng_for(name), n, n)
        return m, None, {"row": r0}
    raise KeyError(name)
