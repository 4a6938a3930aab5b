"""GPU parity of PR-EDT's row-recursive proximate-point row pass
(edt2d_proximate_u8_batched; Python edt2d(..., method="proximate")) against
the oracle: int32 squared distances bit-exact, float32 distances within
tolerance, every index a nearest background element -- on random shapes
(sub-blocks cut short, single rows and columns, spacings), edge cases, and
every 2-D workload at full size, PR-EDT's own (random squares, 1 % and 99 %
background) included.  Outputs are poisoned before each call."""

import sys

import numpy as np
import pytest

import oracle
from gpu_check import compare

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from exact_euclidean_distance_amd import _lib
    _lib.load()
    return torch, torch.device("cuda:0")


def run(env, mask, sampling=None, want=("sqdist", "dist", "indices"), method="proximate"):
    torch, dev = env
    from exact_euclidean_distance_amd import edt2d
    shape = mask.shape
    sq = torch.full(shape, -7, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.full(shape, float("nan"), dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.full(shape, -7, dtype=torch.int32, device=dev) if "indices" in want else None
    edt2d(torch.from_numpy(np.ascontiguousarray(mask)).to(dev), sampling, sqdist=sq, dist=ds, indices=ix,
          return_distances=ds is not None, method=method)
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in (("sqdist", sq), ("dist", ds), ("indices", ix)) if t is not None}


def check(env, mask, sampling=None):
    iso = sampling is None or all(float(s) == 1.0 for s in sampling)
    want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
    out = run(env, mask, sampling, want)
    if mask.ndim == 2:
        ref, _ = oracle.edt(mask, sampling, features=False)
    else:
        ref, _ = oracle.edt_batch(mask, sampling, features=False)
    compare(mask, sampling, ref, out.get("sqdist"), out.get("dist"), out.get("indices"), batch=mask.ndim == 3)
    return out


SHAPES = [(1, 1), (1, 37), (37, 1), (64, 64), (65, 130), (200, 333), (129, 1031), (3, 4100), (700, 7),
          (130, 257), (63, 2000), (191, 17)]


@pytest.mark.parametrize("shape", SHAPES)
def test_random(env, shape):
    rng = np.random.default_rng([42, 9200, shape[0], shape[1]])
    for p in (0.002, 0.02, 0.3, 0.9):
        m = (rng.random(shape) >= p).astype(np.uint8)
        m.reshape(-1)[rng.integers(0, m.size)] = 0
        for samp in (None, (2.5, 1.0), (1.0, 0.5)):
            _say(f"proximate {shape} p={p} sampling={samp}")
            check(env, m, samp)


def test_edge_cases(env):
    rng = np.random.default_rng([42, 9201])
    h, w = 150, 300
    cases = {
        "all background": np.zeros((h, w), np.uint8),
        "one pixel": np.ones((h, w), np.uint8),
        "full row": np.ones((h, w), np.uint8),
        "full column": np.ones((h, w), np.uint8),
        "two far pixels": np.ones((h, w), np.uint8),
        "checkerboard": (np.indices((h, w)).sum(0) % 2).astype(np.uint8),
    }
    cases["one pixel"][77, 123] = 0
    cases["full row"][70, :] = 0
    cases["full column"][:, 200] = 0
    cases["two far pixels"][0, 0] = 0
    cases["two far pixels"][h - 1, w - 1] = 0
    for name, m in cases.items():
        _say(f"proximate edge case: {name}")
        check(env, m)
    # a batch with an image without background and one of background only
    b = (rng.random((4, 90, 110)) >= 0.01).astype(np.uint8)
    b[1] = 1
    b[2] = 0
    _say("proximate batch with empty images")
    out = check(env, b)
    assert (out["indices"][1] == -110).all()


def test_matches_separable(env):
    rng = np.random.default_rng([42, 9202])
    m = (rng.random((3, 500, 700)) >= 0.005).astype(np.uint8)
    a = run(env, m, method="proximate")
    b = run(env, m, method="separable")
    assert (a["sqdist"] == b["sqdist"]).all()
    # (the separable epilogue takes the float32 square root within one ulp,
    # this path rounds a float64 one: equal within the distance tolerance)
    d = np.abs(a["dist"].astype(np.float64) - b["dist"])
    assert (d <= 1e-6 * b["dist"]).all()


def test_width_limit(env):
    torch, dev = env
    from exact_euclidean_distance_amd import EDTError, edt2d
    m = torch.ones((2, 16385), dtype=torch.uint8, device=dev)
    with pytest.raises(EDTError):
        edt2d(m, method="proximate")


@pytest.mark.parametrize("name", ["c1", "c2a", "c2b", "c3", "p1_1024_1", "p1_1024_99", "p1_2048_1",
                                  "p1_2048_99", "p1_4096_1", "p1_4096_99", "p1_8192_1", "p1_8192_99"])
def test_full_size(env, name):
    from workloads import make_config
    mask, sampling, _ = make_config(name)
    _say(f"proximate full size {name} {mask.shape}")
    want = ("sqdist", "dist", "indices")
    out = run(env, mask, sampling, want)
    ref, _ = oracle.edt(mask, sampling, features=False)
    compare(mask, sampling, ref, out["sqdist"], out["dist"], out["indices"])
