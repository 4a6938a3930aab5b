"""CPU checks of the chessboard line step the kernels run
(exact_euclidean_distance_amd/csrc/linf_rmq.h, compiled as host C++ by
tests/host_model/linf_model.cpp): for random lines of sources, h(q) equals
the definition min_j max(g(j), |q - j|) and the returned source attains it.
No GPU is needed."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_model", "linf_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("linf_model") / "linf_model.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-o", out, SRC], check=True)
    lib = ctypes.CDLL(out)
    lib.model_linf_line.restype = ctypes.c_int
    lib.model_linf_line.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def run(g):
        g = np.ascontiguousarray(g, np.int32)
        h = np.empty(len(g), np.int32)
        j = np.empty(len(g), np.int32)
        assert lib.model_linf_line(g.ctypes.data, len(g), h.ctypes.data, j.ctypes.data) == 0
        return h, j

    return run


def _definition(g):
    L = len(g)
    q = np.arange(L)
    src = np.flatnonzero(g >= 0)
    v = np.maximum(g[src][None, :], np.abs(q[:, None] - src[None, :]))
    return v.min(1)


def _check(model, g):
    h, j = model(g)
    ref = _definition(g)
    np.testing.assert_array_equal(h, ref)
    assert (g[j] >= 0).all(), "the returned position holds no source"
    att = np.maximum(g[j], np.abs(np.arange(len(g)) - j))
    np.testing.assert_array_equal(att, ref)


def test_random_lines(model):
    rng = np.random.default_rng([42, 7100])
    for L in (1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 300, 512, 1000, 4096):
        for p in (0.002, 0.05, 0.3, 1.0):
            for gmax in (0, 3, 50, 1000, 65534):
                g = np.where(rng.random(L) < p, rng.integers(0, gmax + 1, L), -1)
                if (g < 0).all():
                    g[rng.integers(L)] = rng.integers(0, gmax + 1)
                _check(model, g)


def test_special_lines(model):
    L = 777
    g = np.full(L, -1)
    g[0] = 0                                  # one source at the start
    _check(model, g)
    g = np.full(L, -1)
    g[L - 1] = 65534                          # one far, very high source
    _check(model, g)
    _check(model, np.zeros(L, np.int64))      # every position a source of g = 0
    _check(model, np.arange(L) % 37)          # sawtooth
    _check(model, np.abs(np.arange(L) - L // 2))   # a V: every source ties
    g = np.full(L, 400)
    g[::100] = 3                              # sparse low sources among high ones
    _check(model, g)


@pytest.mark.parametrize("L", [8, 24, 40, 1024])
def test_exhaustive_small_values(model, L):
    """Many lines with small g, where ties between sources are the rule."""
    rng = np.random.default_rng([42, 7101, L])
    for _ in range(200):
        g = rng.integers(-1, 4, L)
        if (g < 0).all():
            g[0] = 0
        _check(model, g)
