"""Shared comparison of a GPU result with the oracle (used by the GPU tests,
the smoke check and the benchmark's parity leg)."""

import numpy as np

import oracle

# float32 distances: 1e-6 relative (unit spacing) / 1e-5 relative (anisotropic)
TOL_ISO = 1e-6
TOL_ANISO = 1e-5


def compare(mask, sampling, ref_sq, sq=None, dist=None, idx=None, batch=False):
    """mask/ref_sq/outputs are NumPy arrays of one image, or of a batch
    (leading axis) when ``batch``.  Raises AssertionError on any mismatch."""
    if batch:
        for b in range(mask.shape[0]):
            compare(mask[b], sampling, ref_sq[b],
                    None if sq is None else sq[b],
                    None if dist is None else dist[b],
                    None if idx is None else idx[b])
        return
    iso = sampling is None or all(float(s) == 1.0 for s in sampling)
    if sq is not None:
        assert sq.dtype == np.int32
        bad = np.flatnonzero(sq.astype(np.float64).reshape(-1) != ref_sq.reshape(-1))
        assert bad.size == 0, (
            f"sqdist mismatch at {bad.size} elements; first {bad[:5]}: "
            f"gpu {sq.reshape(-1)[bad[:5]]} oracle {ref_sq.reshape(-1)[bad[:5]]}")
    if dist is not None:
        assert dist.dtype == np.float32
        ref = np.sqrt(ref_sq)
        tol = TOL_ISO if iso else TOL_ANISO
        err = np.abs(dist.astype(np.float64) - ref)
        zero = ref_sq == 0
        assert (dist[zero] == 0).all(), "nonzero distance on background"
        rel = err[~zero] / ref[~zero]
        assert rel.size == 0 or rel.max() <= tol, f"dist rel err {rel.max():.3g} > {tol}"
    if idx is not None:
        assert idx.dtype == np.int32
        d2 = oracle.sqdist_to(idx, mask.shape, sampling)
        bad = np.flatnonzero(d2.reshape(-1) != ref_sq.reshape(-1))
        assert bad.size == 0, (
            f"index does not attain the minimum at {bad.size} elements; first {bad[:5]}: "
            f"d2 {d2.reshape(-1)[bad[:5]]} oracle {ref_sq.reshape(-1)[bad[:5]]}")
        if (mask == 0).any():
            flat = idx.reshape(-1).astype(np.int64)
            assert (flat >= 0).all() and (flat < mask.size).all()
            assert (mask.reshape(-1)[flat] == 0).all(), "index is not a background element"
