"""Shared comparison of a GPU result with the oracle (used by the GPU tests,
the smoke check and the benchmark's parity leg)."""

import numpy as np

import oracle

# float32 distances: 1e-6 relative (unit spacing) / 1e-5 relative (anisotropic)
TOL_ISO = 1e-6
TOL_ANISO = 1e-5
# attaining indices under squared spacings that are not multiples of 2^-20:
# squared distances equal up to a relative 1e-12 (float64 rounding of the sums)
TOL_TIE = 1e-12


def _exact_sums(sampling):
    """True when every squared spacing is a multiple of 2^-20 (then every
    squared distance of the tested sizes is an exact float64 sum)."""
    if sampling is None:
        return True
    return all(float(s) * float(s) * 2.0 ** 20 == float(int(float(s) * float(s) * 2.0 ** 20))
               for s in sampling)


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
        if _exact_sums(sampling):
            bad = np.flatnonzero(d2.reshape(-1) != ref_sq.reshape(-1))
        else:
            # squared spacings with no finite binary form: two background
            # elements at one distance can differ in their float64 sums by a
            # rounding step, and either is a correct answer
            diff = np.abs(d2.reshape(-1) - ref_sq.reshape(-1))
            bad = np.flatnonzero(diff > TOL_TIE * np.maximum(ref_sq.reshape(-1), 1.0))
        assert bad.size == 0, (
            f"index does not attain the minimum at {bad.size} elements; first {bad[:5]}: "
            f"d2 {d2.reshape(-1)[bad[:5]]} oracle {ref_sq.reshape(-1)[bad[:5]]}")
        if (mask == 0).any():
            flat = idx.reshape(-1).astype(np.int64)
            assert (flat >= 0).all() and (flat < mask.size).all()
            assert (mask.reshape(-1)[flat] == 0).all(), "index is not a background element"
