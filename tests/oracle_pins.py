"""Pins for the CPU oracle: checks that tie it to the definition of the transform
and to results fixed by mathematics, independent of the oracle's own code.

Each ``pin_*`` takes a loaded oracle library handle (``oracle.load(path)``) so
that ``tests/test_oracle.py`` can run them both on the real oracle (all must
pass) and on copies with a planted mistake (at least one must fail).
"""

import numpy as np
from scipy import ndimage as ndi

import oracle
from golden_io import load as load_golden, names as golden_names

EXACT_SAMPLINGS_2D = [None, (1.0, 1.0), (2.0, 1.0), (1.0, 0.5), (2.5, 1.25)]
EXACT_SAMPLINGS_3D = [None, (2.5, 1.0, 1.0), (1.0, 2.0, 0.5), (0.75, 1.5, 3.0)]


def _check_features(mask, sq, feat, sampling):
    """Every returned feature is a background element (or the virtual one) and
    its squared distance equals the returned minimum exactly."""
    flat = oracle.flat_index(feat, mask.shape)
    d = oracle.sqdist_to(flat, mask.shape, sampling)
    np.testing.assert_array_equal(d, sq)
    if (mask == 0).any():
        assert (flat >= 0).all()
        assert (mask.reshape(-1)[flat.reshape(-1)] == 0).all()


def pin_golden(lib):
    """Hand-derived fixtures (tests/golden/)."""
    for name in golden_names():
        g = load_golden(name)
        for fn in (oracle.edt, oracle.edt_brute):
            sq, feat = fn(g["mask"], g["sampling"], True, lib)
            np.testing.assert_array_equal(sq, g["sqdist"], err_msg=f"{name} via {fn.__name__}")
            _check_features(g["mask"], sq, feat, g["sampling"])


def _random_cases(seed, count):
    rng = np.random.default_rng([42, 1000, seed])
    dens = [0.001, 0.01, 0.1, 0.5, 0.9, 0.999]
    for t in range(count):
        nd = (2, 2, 3, 1, 4)[t % 5]
        if nd == 1:
            shape = (int(rng.integers(1, 65)),)
            samp = [None, (1.5,)][t % 2]
        elif nd == 2:
            shape = tuple(int(x) for x in rng.integers(1, 65, 2))
            samp = EXACT_SAMPLINGS_2D[t % len(EXACT_SAMPLINGS_2D)]
        elif nd == 3:
            shape = tuple(int(x) for x in rng.integers(1, 17, 3))
            samp = EXACT_SAMPLINGS_3D[t % len(EXACT_SAMPLINGS_3D)]
        else:
            shape = tuple(int(x) for x in rng.integers(1, 7, 4))
            samp = [None, (1.0, 2.0, 1.0, 0.5)][t % 2]
        p = dens[t % len(dens)]
        mask = (rng.random(shape) >= p).astype(np.uint8)
        yield shape, samp, mask


def pin_brute_random(lib, count=120, seed=0):
    """Separable oracle == C brute force == NumPy brute force, exactly, on random
    masks of every density (spacings chosen so float64 is exact)."""
    for shape, samp, mask in _random_cases(seed, count):
        sq, feat = oracle.edt(mask, samp, True, lib)
        sqb, _ = oracle.edt_brute(mask, samp, True, lib)
        sqn = oracle.brute_numpy(mask, samp)
        np.testing.assert_array_equal(sqn, sqb, err_msg=f"brute C vs numpy {shape} {samp}")
        np.testing.assert_array_equal(sq, sqn, err_msg=f"separable vs brute {shape} {samp}")
        _check_features(mask, sq, feat, samp)


def pin_closed_forms(lib):
    """Closed forms: one background element, all background, a full background
    row/plane, two background elements."""
    rng = np.random.default_rng([42, 1001])
    for t in range(12):
        nd = 2 + t % 2
        shape = tuple(int(x) for x in rng.integers(1, 40 if nd == 2 else 12, nd))
        samp = tuple(float(x) for x in rng.choice([0.5, 1.0, 2.0, 2.5], nd))
        s2 = np.asarray(samp) ** 2
        b = tuple(int(rng.integers(0, n)) for n in shape)
        mask = np.ones(shape, np.uint8)
        mask[b] = 0
        sq, feat = oracle.edt(mask, samp, True, lib)
        grid = np.indices(shape)
        expect = sum(s2[k] * (grid[k] - b[k]).astype(np.float64) ** 2 for k in range(nd))
        np.testing.assert_array_equal(sq, expect)
        np.testing.assert_array_equal(feat.reshape(-1, nd), np.tile(np.asarray(b, np.int32), (mask.size, 1)))

        # all background: zero everywhere and each element is its own feature
        sq, feat = oracle.edt(np.zeros(shape, np.uint8), samp, True, lib)
        assert (sq == 0).all()
        np.testing.assert_array_equal(np.moveaxis(feat, -1, 0), np.indices(shape))

        # full background hyperplane across axis 0 at index r
        r = int(rng.integers(0, shape[0]))
        mask = np.ones(shape, np.uint8)
        mask[r] = 0
        sq, _ = oracle.edt(mask, samp, True, lib)
        np.testing.assert_array_equal(sq, s2[0] * (grid[0] - r).astype(np.float64) ** 2)

        # two background elements: the smaller of two radial distances
        c = tuple(int(rng.integers(0, n)) for n in shape)
        mask = np.ones(shape, np.uint8)
        mask[b] = 0
        mask[c] = 0
        sq, _ = oracle.edt(mask, samp, True, lib)
        e2 = sum(s2[k] * (grid[k] - c[k]).astype(np.float64) ** 2 for k in range(nd))
        np.testing.assert_array_equal(sq, np.minimum(expect, e2))


def pin_1d(lib):
    """A single line: the textbook nearest background on a line, found with
    numpy.searchsorted over the sorted background positions."""
    rng = np.random.default_rng([42, 1002])
    for t in range(50):
        n = int(rng.integers(1, 200))
        mask = (rng.random(n) >= [0.02, 0.3, 0.9][t % 3]).astype(np.uint8)
        bg = np.flatnonzero(mask == 0)
        if len(bg) == 0:
            continue
        q = np.arange(n)
        k = np.searchsorted(bg, q)
        left = bg[np.clip(k - 1, 0, len(bg) - 1)]
        right = bg[np.clip(k, 0, len(bg) - 1)]
        d = np.minimum(np.abs(q - left), np.abs(q - right)).astype(np.float64)
        for shape in [(n,), (1, n), (n, 1)]:
            sq, _ = oracle.edt(mask.reshape(shape), None, True, lib)
            np.testing.assert_array_equal(sq.reshape(-1), d * d)


def pin_scipy(lib):
    """SciPy's distance_transform_edt gives the same distances (a library
    special case; checked on distances, which are unique)."""
    rng = np.random.default_rng([42, 1003])
    for t in range(20):
        nd = 2 + t % 2
        shape = tuple(int(x) for x in rng.integers(2, 80 if nd == 2 else 20, nd))
        samp = [None, tuple(float(x) for x in rng.uniform(0.3, 3.0, nd))][t % 2]
        mask = (rng.random(shape) >= [0.01, 0.2, 0.7][t % 3]).astype(np.uint8)
        if not (mask == 0).any():
            mask.reshape(-1)[0] = 0
        sq, _ = oracle.edt(mask, samp, False, lib)
        ref = ndi.distance_transform_edt(mask, sampling=samp)
        np.testing.assert_allclose(np.sqrt(sq), ref, rtol=1e-12, atol=0)


PINS = [pin_golden, pin_brute_random, pin_closed_forms, pin_1d, pin_scipy]
