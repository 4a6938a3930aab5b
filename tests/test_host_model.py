"""CPU checks of the envelope algorithm the kernels run.

tests/host_model/host_model.cpp compiles the device helpers of
exact_euclidean_distance_amd/csrc/envelope.h as host C++ and drives them in the
kernels' phase order (candidate filter -> chunk envelopes -> per-chunk owners,
or whole-line rounds -> interval marks -> scan).  Here that model is checked against the definition of a 1-D pass
(brute force over all candidates) and, composed into full transforms, against
the oracle.  No GPU is needed.
"""

import ctypes
import itertools
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_model", "host_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_model") / "host_model.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", out, SRC], check=True)
    lib = ctypes.CDLL(out)
    lib.model_envelope_lines.restype = ctypes.c_int
    lib.model_envelope_lines.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]

    def run(fb, s2l, K, G, reach=8):
        fb = np.ascontiguousarray(fb, np.float64)
        nl, L = fb.shape
        own = np.empty((nl, L), np.int32)
        rc = lib.model_envelope_lines(fb.ctypes.data, nl, L, s2l, K, G, reach, own.ctypes.data)
        assert rc == 0
        return own

    return run


def _brute_lines(fb, s2l):
    L = fb.shape[1]
    q = np.arange(L, dtype=np.float64)
    vals = s2l * (q[:, None] - q[None, :]) ** 2 + fb[:, None, :]   # [line][q][j]
    return vals.min(-1)


def _value_at(fb, own, s2l):
    q = np.arange(fb.shape[1])
    sel = np.take_along_axis(fb, np.maximum(own, 0), 1)
    v = s2l * (q[None, :] - own).astype(np.float64) ** 2 + sel
    return np.where(own < 0, np.inf, v)


def _layouts(L):
    out = []
    for K in (8, 16, 32, 64):
        g0 = -(-L // K)
        p2 = 1 << max(0, (g0 - 1).bit_length())
        out += [(K, g0), (K, p2), (K, g0 + 3)]
    return out


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 64, 100, 257, 1000, 4096])
def test_lines_match_definition(model, L):
    rng = np.random.default_rng([42, 2000, L])
    nl = 24
    fb = np.empty((nl, L))
    for i in range(nl):
        kind = i % 6
        if kind == 0:      # squared column distances, some columns without background
            g = rng.integers(0, 3 * L + 1, L).astype(np.float64)
            fb[i] = g * g
            fb[i][rng.random(L) < 0.3] = np.inf
        elif kind == 1:    # all equal: every candidate on the envelope
            fb[i] = float(rng.integers(0, 50)) ** 2
        elif kind == 2:    # a single candidate
            fb[i] = np.inf
            fb[i][rng.integers(0, L)] = float(rng.integers(0, 100))
        elif kind == 3:    # no candidate
            fb[i] = np.inf
        elif kind == 4:    # deep dip at the end: long removal cascades at junctions
            fb[i] = float(L) ** 2
            fb[i][-1] = 0.0
        else:              # random small integers (many ties)
            fb[i] = rng.integers(0, 4, L).astype(np.float64)
    for s2l in (1.0, 6.25):
        ref = _brute_lines(fb, s2l)
        for (K, G), reach in itertools.product(_layouts(L), (8, 1, 0)):
            own = model(fb, s2l, K, G, reach)
            got = _value_at(fb, own, s2l)
            np.testing.assert_array_equal(got, ref, err_msg=f"L={L} K={K} G={G} s2={s2l} reach={reach}")
            has = np.isfinite(fb)
            ok = own >= 0
            assert (ok == has.any(1)[:, None]).all()
            assert np.isfinite(np.take_along_axis(fb, np.maximum(own, 0), 1)[ok]).all()


def _axis0_nearest(mask):
    """Nearest background along axis 0 (the smaller coordinate on ties); -1 if none."""
    n0 = mask.shape[0]
    i = np.arange(n0).reshape((n0,) + (1,) * (mask.ndim - 1))
    big = 1 << 30
    up = np.maximum.accumulate(np.where(mask == 0, i, -1), axis=0)
    dn = np.flip(np.minimum.accumulate(np.flip(np.where(mask == 0, i, big), 0), axis=0), 0)
    use_up = (up >= 0) & ((dn >= big) | (i - up <= dn - i))
    g = np.where(use_up, up, np.where(dn < big, dn, -1))
    return g


def _model_edt(model, mask, sampling, K, reach=8):
    """Full transform composed from the model: axis-0 nearest, then one
    envelope pass per further axis (values are squared distances so far)."""
    s2 = np.ones(mask.ndim) if sampling is None else np.asarray(sampling, np.float64) ** 2
    g = _axis0_nearest(mask)
    i = np.arange(mask.shape[0]).reshape((mask.shape[0],) + (1,) * (mask.ndim - 1))
    F = np.where(g >= 0, s2[0] * (i - g).astype(np.float64) ** 2, np.inf)
    for ax in range(1, mask.ndim):
        Fm = np.moveaxis(F, ax, -1)
        shp = Fm.shape
        fb = Fm.reshape(-1, shp[-1])
        L = shp[-1]
        G = -(-L // K)
        own = model(fb, s2[ax], K, G, reach)
        F = np.moveaxis(_value_at(fb, own, s2[ax]).reshape(shp), -1, ax)
    return F


@pytest.mark.parametrize("K", [8, 16, 32, 64])
@pytest.mark.parametrize("reach", [8, 0])
def test_model_transform_matches_oracle(model, K, reach):
    rng = np.random.default_rng([42, 2001, K])
    cases = []
    for t in range(16):
        shape = tuple(int(x) for x in rng.integers(1, 200, 2))
        mask = (rng.random(shape) >= [1e-3, 0.01, 0.2, 0.9][t % 4]).astype(np.uint8)
        cases.append((mask, [None, (2.5, 1.0)][t % 2]))
    full_row = np.ones((150, 300), np.uint8)
    full_row[77] = 0
    cases.append((full_row, None))
    single = np.ones((130, 170), np.uint8)
    single[3, 160] = 0
    cases.append((single, None))
    for t in range(6):
        shape = tuple(int(x) for x in rng.integers(1, 40, 3))
        mask = (rng.random(shape) >= [0.001, 0.05, 0.5][t % 3]).astype(np.uint8)
        cases.append((mask, [None, (2.5, 1.0, 1.0)][t % 2]))
    for mask, samp in cases:
        if not (mask == 0).any():
            mask.reshape(-1)[0] = 0
        ref, _ = oracle.edt(mask, samp, False)
        got = _model_edt(model, mask, samp, K, reach)
        np.testing.assert_array_equal(got, ref, err_msg=f"shape {mask.shape} sampling {samp}")


@pytest.fixture(scope="module")
def int_model(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_model_int") / "host_model.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", out, SRC], check=True)
    lib = ctypes.CDLL(out)
    lib.model_envelope_lines_int.restype = ctypes.c_int
    lib.model_envelope_lines_int.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]

    def run(fb, s2l, K, G, reach=8):
        fb = np.ascontiguousarray(fb, np.int32)
        nl, L = fb.shape
        own = np.empty((nl, L), np.int32)
        assert lib.model_envelope_lines_int(fb.ctypes.data, nl, L, s2l, K, G, reach, own.ctypes.data) == 0
        return own

    return run


@pytest.mark.parametrize("L", [1, 33, 257, 1000, 4096])
def test_int_lines_match_definition(int_model, L):
    """The squared Euclidean step in exact scaled integers (L2IntMetric, the
    kernels' integer values): owners attain the definition's minimum, with
    values S F up to the 2^29 bound the host allows."""
    rng = np.random.default_rng([42, 2004, L])
    for s2l in (1, 4, 25):
        top = (2 ** 29 - 1) // 2 - s2l * L * L   # heights below 2^29
        nl = 12
        fb = np.empty((nl, L), np.int64)
        for i in range(nl):
            kind = i % 4
            if kind == 0:
                fb[i] = rng.integers(0, max(1, min(top, 4 * L * L)), L)
                fb[i][rng.random(L) < 0.3] = -1
            elif kind == 1:
                fb[i] = rng.integers(0, max(1, top), L)
            elif kind == 2:
                fb[i] = -1
                fb[i][rng.integers(0, L)] = rng.integers(0, max(1, top))
            else:
                fb[i] = rng.integers(0, 4, L)
        ref_in = np.where(fb >= 0, fb.astype(np.float64), np.inf)
        ref = _brute_lines(ref_in, float(s2l))
        for (K, G), reach in itertools.product(_layouts(L), (8, 0)):
            own = int_model(fb, s2l, K, G, reach)
            got = _value_at(ref_in, own, float(s2l))
            np.testing.assert_array_equal(got, ref, err_msg=f"L={L} K={K} G={G} s2={s2l} reach={reach}")


# ---------------------------------------------------------------------------
# The same machinery under the chessboard metric, f_j(q) = max(g_j, |q - j|)
# (TorchMorph's chamfer transforms, read as the L-infinity metric): the line
# step against its definition, and composed transforms against the oracle's
# brute force.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def linf_model(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host_model_linf") / "host_model.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", out, SRC], check=True)
    lib = ctypes.CDLL(out)
    lib.model_linf_envelope_lines.restype = ctypes.c_int
    lib.model_linf_envelope_lines.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]

    def run(gb, K, G, reach=8):
        gb = np.ascontiguousarray(gb, np.int32)
        nl, L = gb.shape
        own = np.empty((nl, L), np.int32)
        val = np.empty((nl, L), np.int32)
        rc = lib.model_linf_envelope_lines(gb.ctypes.data, nl, L, K, G, reach, own.ctypes.data,
                                           val.ctypes.data)
        assert rc == 0
        # the value the metric forms for the owner (the kernels' output step)
        np.testing.assert_array_equal(val, _linf_value_at(gb, own))
        return own

    run.path = out
    return run


def test_linf_crossings_match_definition(linf_model):
    """LinfMetric's closed-form crossings against the definition, position by
    position: for j < k the positions where max(g_k, |q - k|) is below (at
    most) max(g_j, |q - j|) form a right half-line starting at first_below
    (first_at_most)."""
    lib = ctypes.CDLL(linf_model.path)
    lib.model_linf_crossings.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    rng = np.random.default_rng([42, 2005])
    q = np.arange(-300, 400)
    out = np.empty(2, np.int32)
    for _ in range(3000):
        j = int(rng.integers(0, 80))
        k = int(rng.integers(j + 1, 100))
        gj, gk = (int(x) for x in rng.integers(0, 60, 2))
        fj = np.maximum(gj, np.abs(q - j))
        fk = np.maximum(gk, np.abs(q - k))
        lib.model_linf_crossings(j, gj, k, gk, out.ctypes.data)
        for lt, x in ((fk < fj, out[0]), (fk <= fj, out[1])):
            first = q[np.argmax(lt)]
            assert lt[-1] and (lt[q >= first]).all() and not lt[q < first].any(), (j, gj, k, gk)
            assert x == first, (j, gj, k, gk, x, first)


def _linf_brute_lines(gb):
    """min_j max(g_j, |q - j|) over the sources (g >= 0) of every line (-1: none)."""
    L = gb.shape[1]
    q = np.arange(L)
    d = np.abs(q[:, None] - q[None, :])                       # [q][j]
    v = np.maximum(gb[:, None, :].astype(np.int64), d[None])  # [line][q][j]
    v = np.where(gb[:, None, :] >= 0, v, np.iinfo(np.int64).max)
    out = v.min(-1)
    return np.where(out == np.iinfo(np.int64).max, -1, out)


def _linf_value_at(gb, own):
    q = np.arange(gb.shape[1])
    sel = np.take_along_axis(gb, np.maximum(own, 0), 1).astype(np.int64)
    v = np.maximum(sel, np.abs(q[None, :] - own))
    return np.where(own < 0, -1, v)


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 64, 100, 257, 1000, 2048])
def test_linf_lines_match_definition(linf_model, L):
    rng = np.random.default_rng([42, 2002, L])
    nl = 24
    gb = np.empty((nl, L), np.int64)
    for i in range(nl):
        kind = i % 7
        if kind == 0:      # column distances, some columns without background
            gb[i] = rng.integers(0, 2 * L + 1, L)
            gb[i][rng.random(L) < 0.3] = -1
        elif kind == 1:    # all equal: flat bottoms everywhere, every tie
            gb[i] = rng.integers(0, 50)
        elif kind == 2:    # a single source
            gb[i] = -1
            gb[i][rng.integers(0, L)] = rng.integers(0, 100)
        elif kind == 3:    # no source
            gb[i] = -1
        elif kind == 4:    # deep dip at the end: long removal cascades at junctions
            gb[i] = L
            gb[i][-1] = 0
        elif kind == 5:    # random small values (many ties)
            gb[i] = rng.integers(0, 4, L)
        else:              # large values near the uint16 limit, sparse
            gb[i] = np.where(rng.random(L) < 0.05, rng.integers(60000, 65535, L), -1)
    ref = _linf_brute_lines(gb)
    for (K, G), reach in itertools.product(_layouts(L), (8, 1, 0)):
        own = linf_model(gb, K, G, reach)
        got = _linf_value_at(gb, own)
        np.testing.assert_array_equal(got, ref, err_msg=f"L={L} K={K} G={G} reach={reach}")
        ok = own >= 0
        assert (ok == (gb >= 0).any(1)[:, None]).all()
        assert (np.take_along_axis(gb, np.maximum(own, 0), 1)[ok] >= 0).all()


def _model_chessboard(linf_model, mask, K, reach=8):
    """Chessboard transform composed from the model: axis-0 nearest, then one
    envelope pass per further axis (values are L-infinity distances so far)."""
    g = _axis0_nearest(mask)
    i = np.arange(mask.shape[0]).reshape((mask.shape[0],) + (1,) * (mask.ndim - 1))
    D = np.where(g >= 0, np.abs(i - g), -1)
    for ax in range(1, mask.ndim):
        Dm = np.moveaxis(D, ax, -1)
        shp = Dm.shape
        gb = Dm.reshape(-1, shp[-1])
        own = linf_model(gb, K, -(-shp[-1] // K), reach)
        D = np.moveaxis(_linf_value_at(gb, own).reshape(shp), -1, ax)
    return D


@pytest.mark.parametrize("K", [8, 16, 32, 64])
@pytest.mark.parametrize("reach", [8, 0])
def test_linf_model_transform_matches_oracle(linf_model, K, reach):
    rng = np.random.default_rng([42, 2003, K])
    cases = []
    for t in range(12):
        shape = tuple(int(x) for x in rng.integers(1, 120, 2))
        cases.append((rng.random(shape) >= [1e-3, 0.01, 0.2, 0.9][t % 4]).astype(np.uint8))
    single = np.ones((90, 170), np.uint8)
    single[3, 160] = 0
    cases.append(single)
    for t in range(6):
        shape = tuple(int(x) for x in rng.integers(1, 30, 3))
        cases.append((rng.random(shape) >= [0.001, 0.05, 0.5][t % 3]).astype(np.uint8))
    for mask in cases:
        if not (mask == 0).any():
            mask.reshape(-1)[0] = 0
        ref, _ = oracle.chessboard_brute(mask)
        got = _model_chessboard(linf_model, mask, K, reach)
        np.testing.assert_array_equal(got, ref, err_msg=f"shape {mask.shape}")
