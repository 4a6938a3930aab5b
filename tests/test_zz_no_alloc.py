"""GPU test of edt2d_u8_batched_noalloc, the entry point that allocates
nothing (its workspace is the library's own device array).  Called through
the C ABI and checked against edt2d_u8_batched on the same inputs: int32
squared distances and float32 distances equal, every index a nearest
background element.  Two calls in a row, the second on a smaller input, so a
stale array from the first call would show; the third is refused on the host
because its workspace would not fit the array."""

import ctypes
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

OK, SMALL = 0, 3


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from exact_euclidean_distance_amd import _lib
    return torch, torch.device("cuda:0"), _lib.load()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(env, fn_name, mask_np, sampling, want, ws=None):
    torch, dev, lib = env
    B, H, W = mask_np.shape
    mask = torch.from_numpy(mask_np).to(dev)
    sq = torch.full(mask_np.shape, -7, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.full(mask_np.shape, float("nan"), dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.full(mask_np.shape, -7, dtype=torch.int32, device=dev) if "indices" in want else None
    samp = None if sampling is None else (ctypes.c_float * 2)(*sampling)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn_name == "noalloc":
        st = lib.edt2d_u8_batched_noalloc(_p(mask), B, H, W, samp, _p(sq), _p(ds), _p(ix), stream)
    else:
        need = int(lib.edt2d_batched_workspace_size(B, H, W))
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)   # poisoned workspace
        st = lib.edt2d_u8_batched(_p(mask), B, H, W, samp, _p(sq), _p(ds), _p(ix), _p(ws), need,
                                  stream)
    assert st == OK, f"{fn_name}: status {st}"
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in (("sqdist", sq), ("dist", ds), ("indices", ix))
            if t is not None}


def _check_pair(env, mask_np, sampling, want):
    a = _run(env, "noalloc", mask_np, sampling, want)
    b = _run(env, "batched", mask_np, sampling, want)
    if "sqdist" in want:
        assert (a["sqdist"] == b["sqdist"]).all()
    assert (a["dist"] == b["dist"]).all()
    ref = np.stack([oracle.edt(m, sampling, features=False)[0] for m in mask_np])
    for i in range(mask_np.shape[0]):
        d2 = oracle.sqdist_to(a["indices"][i], mask_np.shape[1:], sampling)
        assert (d2 == ref[i]).all(), "noalloc index is not a nearest background element"
        assert (mask_np[i].reshape(-1)[a["indices"][i].reshape(-1)] == 0).all()
    if "sqdist" in want:
        assert (a["sqdist"] == ref).all()


def test_noalloc_matches_batched_twice(env):
    torch, dev, lib = env
    assert lib.edt2d_noalloc_max_workspace() == 64 << 20
    rng = np.random.default_rng([42, 7100])
    first = (rng.random((3, 700, 900)) >= 0.01).astype(np.uint8)
    first[:, 0, 0] = 0
    _say("noalloc call 1: 3 x 700 x 900, unit spacing, sqdist + dist + indices")
    _check_pair(env, first, None, ("sqdist", "dist", "indices"))
    second = (rng.random((2, 300, 517)) >= 0.02).astype(np.uint8)
    second[1] = 1   # an image without background inside the batch
    second[0, 5, 7] = 0
    _say("noalloc call 2: 2 x 300 x 517, spacing (1.5, 1), dist + indices")
    a = _run(env, "noalloc", second, (1.5, 1.0), ("dist", "indices"))
    b = _run(env, "batched", second, (1.5, 1.0), ("dist", "indices"))
    assert (a["dist"] == b["dist"]).all()
    assert (a["indices"] == b["indices"])[1].all()   # the virtual element, the same everywhere
    ref0 = oracle.edt(second[0], (1.5, 1.0), features=False)[0]
    assert (oracle.sqdist_to(a["indices"][0], second.shape[1:], (1.5, 1.0)) == ref0).all()
    ref1 = oracle.edt(second[1], (1.5, 1.0), features=False)[0]
    d = a["dist"][1].astype(np.float64)
    assert np.allclose(d, np.sqrt(ref1), rtol=1e-5, atol=0)


def test_noalloc_refuses_beyond_its_array(env):
    torch, dev, lib = env
    B, H, W = 4, 4096, 4096   # workspace about 150 MB > 64 MiB
    assert lib.edt2d_batched_workspace_size(B, H, W) > lib.edt2d_noalloc_max_workspace()
    # full-size buffers, so that nothing is out of bounds even if the check failed
    mask = torch.ones((B, H, W), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, W), dtype=torch.float32, device=dev)
    st = lib.edt2d_u8_batched_noalloc(_p(mask), B, H, W, None, None, _p(out), None,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == SMALL
