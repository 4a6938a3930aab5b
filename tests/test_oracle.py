"""CPU tests of the oracle against its pins (no GPU needed)."""

import os
import shutil

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_invariants(lib):
    """Background is 0; flipping or transposing the input permutes the output;
    adding background never increases a value; the distance is 1-Lipschitz per
    axis step (|d(p) - d(q)| <= s_k for axis neighbours)."""
    rng = np.random.default_rng([42, 1010])
    for t in range(10):
        shape = tuple(int(x) for x in rng.integers(5, 60, 2))
        samp = (1.0, 1.0) if t % 2 == 0 else (2.0, 0.5)
        mask = (rng.random(shape) >= 0.05).astype(np.uint8)
        mask[0, 0] = 0
        sq, _ = oracle.edt(mask, samp, False, lib)
        assert (sq[mask == 0] == 0).all()
        sqf, _ = oracle.edt(mask[::-1, ::-1].copy(), samp, False, lib)
        np.testing.assert_array_equal(sqf, sq[::-1, ::-1])
        sqt, _ = oracle.edt(mask.T.copy(), samp[::-1], False, lib)
        np.testing.assert_array_equal(sqt, sq.T)
        more = mask.copy()
        more[rng.integers(0, shape[0]), rng.integers(0, shape[1])] = 0
        sqm, _ = oracle.edt(more, samp, False, lib)
        assert (sqm <= sq).all()
        d = np.sqrt(sq)
        assert (np.abs(np.diff(d, axis=0)) <= samp[0] + 1e-12).all()
        assert (np.abs(np.diff(d, axis=1)) <= samp[1] + 1e-12).all()


def test_batch_equals_single(lib):
    from workloads import ellipsoids_3d_batch, rng_for
    vols = ellipsoids_3d_batch(rng_for("c4", 7), 3, 16, 2, 4, 2.0, 6.0)
    vols[1] = 1  # one volume without background
    sq, feat = oracle.edt_batch(vols, None, True, lib)
    for b in range(3):
        s, f = oracle.edt(vols[b], None, True, lib)
        np.testing.assert_array_equal(sq[b], s)
        np.testing.assert_array_equal(feat[b], f)
    assert (feat[1][..., 0] == -1).all()


# Planted mistakes: each replaces one piece of oracle_edt.c in a temporary copy.
# A useful set of pins must fail for every one of them.
MUTANTS = {
    "transposed_operands_in_dominance":
        ("return (Y[b] - Y[a]) * (double)(c - b) >= (Y[c] - Y[b]) * (double)(b - a);",
         "return (Y[b] - Y[a]) * (double)(b - a) >= (Y[c] - Y[b]) * (double)(c - b);"),
    "reversed_dominance":
        ("return (Y[b] - Y[a]) * (double)(c - b) >= (Y[c] - Y[b]) * (double)(b - a);",
         "return (Y[b] - Y[a]) * (double)(c - b) <= (Y[c] - Y[b]) * (double)(b - a);"),
    "dropped_square_in_lifting":
        ("Y[j] = f[j] + s2 * (double)j * (double)j;", "Y[j] = f[j] + s2 * (double)j;"),
    "dropped_spacing_in_query":
        ("2.0 * s2 * (double)q * (double)(stack[m + 1] - stack[m]) >",
         "2.0 * (double)q * (double)(stack[m + 1] - stack[m]) >"),
    "dropped_column_term_in_query":
        ("out[q] = s2 * (double)(q - j) * (double)(q - j) + f[j];",
         "out[q] = s2 * (double)(q - j) * (double)(q - j);"),
    "wrong_choice_between_up_and_down":
        ("if (up >= 0 && (next < 0 || i - up <= next - i)) g = up;",
         "if (up >= 0 && (next < 0 || i - up >= next - i)) g = up;"),
    "virtual_background_wrong_side":
        ("double d = s2[0] * (double)(coord[0] + 1) * (double)(coord[0] + 1);",
         "double d = s2[0] * (double)(coord[0] - 1) * (double)(coord[0] - 1);"),
    "spacing_of_wrong_axis":
        ("envelope_1d((int)nk, s2[ax], fl, Y, stack, owner, outl);",
         "envelope_1d((int)nk, s2[0], fl, Y, stack, owner, outl);"),
    "query_stops_one_early":
        ("while (m + 1 < k &&", "while (m + 2 < k &&"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mdir = tmp_path / "mutant"
    mdir.mkdir()
    shutil.copy(os.path.join(os.path.dirname(oracle._SRC), "oracle_edt.h"), mdir)
    (mdir / "oracle_edt.c").write_text(src.replace(old, new))
    so = str(mdir / "libmutant.so")
    oracle.build(str(mdir / "oracle_edt.c"), so)
    mlib = oracle.load(so)
    failed = []
    for pin in pins.PINS:
        try:
            if pin is pins.pin_brute_random:
                pin(mlib, count=60)
            else:
                pin(mlib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


def test_taxicab_oracle_pins():
    """The L1 oracle against closed forms: one background element, two, all
    background, none (virtual element), the 1-D nearest-background case, and
    the index it returns attains its minimum."""
    rng = np.random.default_rng([42, 7001])
    for shape in ((1,), (9,), (7, 11), (5, 6, 7)):
        m = np.ones(shape, np.uint8)
        b = tuple(int(rng.integers(n)) for n in shape)
        m[b] = 0
        d, who = oracle.taxicab_brute(m)
        grid = np.indices(shape)
        assert (d == sum(np.abs(grid[k] - b[k]) for k in range(len(shape)))).all()
        assert (who == np.ravel_multi_index(b, shape)).all()
    m = np.ones((6, 9), np.uint8)
    m[1, 2] = 0
    m[4, 7] = 0
    d, _ = oracle.taxicab_brute(m)
    g = np.indices(m.shape)
    assert (d == np.minimum(abs(g[0] - 1) + abs(g[1] - 2), abs(g[0] - 4) + abs(g[1] - 7))).all()
    assert (oracle.taxicab_brute(np.zeros((4, 5), np.uint8))[0] == 0).all()
    d, who = oracle.taxicab_brute(np.ones((3, 4), np.uint8))
    assert (d == (g[0][:3, :4] + 1) + g[1][:3, :4]).all() and (who == -4).all()
    line = (rng.random(200) >= 0.05).astype(np.uint8)
    line[17] = 0
    d, _ = oracle.taxicab_brute(line)
    bgp = np.flatnonzero(line == 0)
    k = np.searchsorted(bgp, np.arange(200))
    lo = bgp[np.clip(k - 1, 0, len(bgp) - 1)]
    hi = bgp[np.clip(k, 0, len(bgp) - 1)]
    assert (d == np.minimum(np.abs(np.arange(200) - lo), np.abs(hi - np.arange(200)))).all()
    m = (rng.random((13, 17, 5)) >= 0.1).astype(np.uint8)
    m[0, 0, 0] = 0
    d, who = oracle.taxicab_brute(m)
    assert (oracle.taxicab_to(who, m.shape) == d).all()
    assert (m.reshape(-1)[who.reshape(-1)] == 0).all()


def test_taxicab_at_pins():
    """The one-by-one L1 oracle: the closed form for one background element and
    for none (virtual element at (-1, 0, ...)), and the pinned brute-force
    transform at every element of random 2-D and 3-D masks."""
    rng = np.random.default_rng([42, 7002])
    m = np.ones((8, 9, 10), np.uint8)
    m[3, 7, 2] = 0
    pts = rng.integers(0, m.size, 50)
    z, y, x = np.unravel_index(pts, m.shape)
    assert (oracle.taxicab_at(m, pts) == abs(z - 3) + abs(y - 7) + abs(x - 2)).all()
    e = np.ones((6, 7), np.uint8)
    r, c = np.unravel_index(np.arange(e.size), e.shape)
    assert (oracle.taxicab_at(e, np.arange(e.size)) == (r + 1) + c).all()
    for shape, p in (((23, 31), 0.05), ((7, 9, 11), 0.02)):
        m = (rng.random(shape) >= p).astype(np.uint8)
        m.reshape(-1)[5] = 0
        d, _ = oracle.taxicab_brute(m)
        assert (oracle.taxicab_at(m, np.arange(m.size)) == d.reshape(-1)).all()


def test_chessboard_oracle_pins():
    """The L-infinity oracle against what the mathematics fixes: one background
    element (closed form), none (virtual element), 1-D (equal to the L1
    transform there), the 2-D identity max(|a|, |b|) = (|a + b| + |a - b|) / 2
    (half the L1 transform of the same points on the 45-degree rotated grid),
    the bounds L-inf <= L1 <= n L-inf and L-inf^2 <= EDT^2 <= n L-inf^2, the
    returned index attaining the minimum, and the one-by-one form."""
    rng = np.random.default_rng([42, 7003])
    for shape in ((1,), (9,), (7, 11), (5, 6, 7)):
        m = np.ones(shape, np.uint8)
        b = tuple(int(rng.integers(n)) for n in shape)
        m[b] = 0
        d, who = oracle.chessboard_brute(m)
        grid = np.indices(shape)
        assert (d == np.max([np.abs(grid[k] - b[k]) for k in range(len(shape))], axis=0)).all()
        assert (who == np.ravel_multi_index(b, shape)).all()
    g = np.indices((3, 4))
    d, who = oracle.chessboard_brute(np.ones((3, 4), np.uint8))
    assert (d == np.maximum(g[0] + 1, g[1])).all() and (who == -4).all()
    line = (rng.random(300) >= 0.05).astype(np.uint8)
    line[40] = 0
    assert (oracle.chessboard_brute(line)[0] == oracle.taxicab_brute(line)[0]).all()
    # 2-D: (x, y) -> (x + y, x - y + W - 1) on an (H + W - 1)^2 grid
    H, W = 13, 17
    m = (rng.random((H, W)) >= 0.08).astype(np.uint8)
    m[3, 5] = 0
    R = np.ones((H + W - 1, H + W - 1), np.uint8)
    xs, ys = np.nonzero(m == 0)
    R[xs + ys, xs - ys + W - 1] = 0
    l1r, _ = oracle.taxicab_brute(R)
    gx, gy = np.indices((H, W))
    d, who = oracle.chessboard_brute(m)
    assert (2 * d == l1r[gx + gy, gx - gy + W - 1]).all()
    assert (oracle.chessboard_to(who, m.shape) == d).all()
    assert (m.reshape(-1)[who.reshape(-1)] == 0).all()
    for shape, p in (((19, 23), 0.03), ((6, 9, 11), 0.02)):
        m = (rng.random(shape) >= p).astype(np.uint8)
        m.reshape(-1)[7] = 0
        d, who = oracle.chessboard_brute(m)
        l1, _ = oracle.taxicab_brute(m)
        e2, _ = oracle.edt(m, None, features=False)
        n = len(shape)
        assert (d <= l1).all() and (l1 <= n * d).all()
        assert (d * d <= e2).all() and (e2 <= n * d * d).all()
        assert (oracle.chessboard_to(who, shape) == d).all()
        assert (oracle.chessboard_at(m, np.arange(m.size)) == d.reshape(-1)).all()
