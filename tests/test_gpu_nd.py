"""GPU parity of edt_nd_u8 (Python: ``edt``), the transform of any spatial
rank, strided masks, long rows and extents over 65535, against the oracle
(which is N-dimensional): int32 squared distances bit-exact (unit spacing),
float32 distances within 1e-6 / 1e-5 relative, every index a background
element at exactly the oracle's minimum.  Outputs are poisoned first."""

import sys

import numpy as np
import pytest

import oracle
from gpu_check import TOL_ANISO, TOL_ISO

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


def run_nd(env, mask_t, sampling=None, batch_dims=0, index_dtype=None, want=("sqdist", "dist", "indices")):
    torch, dev = env
    from exact_euclidean_distance_amd import edt
    index_dtype = index_dtype or torch.int32
    shape = tuple(mask_t.shape)
    sq = torch.full(shape, -7, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.full(shape, float("nan"), dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.full(shape, -7, dtype=index_dtype, device=dev) if "indices" in want else None
    edt(mask_t, sampling, batch_dims=batch_dims, sqdist=sq, dist=ds, indices=ix,
        return_distances=ds is not None, index_dtype=index_dtype)
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in (("sqdist", sq), ("dist", ds), ("indices", ix)) if t is not None}


def check_images(mask_np, out, sampling, batch_dims):
    """Compare every image (the spatial part after batch_dims) with the oracle."""
    img = mask_np.shape[batch_dims:]
    flat = mask_np.reshape((-1,) + img)
    iso = sampling is None or all(float(s) == 1.0 for s in sampling)
    for b in range(flat.shape[0]):
        m = flat[b]
        ref, _ = oracle.edt(m, sampling, features=False)
        if "sqdist" in out:
            sq = out["sqdist"].reshape((-1,) + img)[b]
            assert (sq == ref).all(), f"sqdist mismatch in image {b}"
        if "dist" in out:
            d = out["dist"].reshape((-1,) + img)[b].astype(np.float64)
            r = np.sqrt(ref)
            zero = ref == 0
            assert (d[zero] == 0).all()
            rel = np.abs(d[~zero] - r[~zero]) / r[~zero]
            assert rel.size == 0 or rel.max() <= (TOL_ISO if iso else TOL_ANISO), rel.max()
        if "indices" in out:
            ix = out["indices"].reshape((-1,) + img)[b].astype(np.int64)
            d2 = oracle.sqdist_to(ix, img, sampling)
            assert (d2 == ref).all(), f"an index does not attain the minimum in image {b}"
            if (m == 0).any():
                assert (m.reshape(-1)[ix.reshape(-1)] == 0).all()


@pytest.mark.parametrize("shape,p", [((5, 6, 7, 8), 0.05), ((3, 4, 5, 6, 7), 0.02),
                                     ((2, 3, 3, 4, 5, 3), 0.1), ((6, 1, 9, 1), 0.2),
                                     ((4, 4, 4, 4, 4, 4, 4), 0.01), ((2, 2, 2, 2, 2, 2, 2, 3), 0.3)])
def test_rank_4_to_8(env, shape, p):
    torch, dev = env
    rng = np.random.default_rng([42, 9100, len(shape)])
    m = (rng.random(shape) >= p).astype(np.uint8)
    m.reshape(-1)[rng.integers(0, m.size)] = 0
    mt = torch.from_numpy(m).to(dev)
    for samp in (None, tuple([2.5, 1.0, 0.5, 1.5, 1.0, 2.0, 1.0, 0.5][:len(shape)])):
        _say(f"rank {len(shape)} {shape} p={p} sampling={samp}")
        want = ("sqdist", "dist", "indices") if samp is None else ("dist", "indices")
        out = run_nd(env, mt, samp, want=want)
        check_images(m, out, samp, 0)
        out64 = run_nd(env, mt, samp, index_dtype=torch.int64, want=("indices",))
        check_images(m, out64, samp, 0)


def test_batch_axes_and_empty_images(env):
    torch, dev = env
    rng = np.random.default_rng([42, 9101])
    m = (rng.random((2, 3, 4, 5, 6, 7)) >= 0.03).astype(np.uint8)
    m[1, 2] = 1            # an image without background: the virtual element
    m[0, 0] = 0            # an image of background only
    _say("batch axes (2, 3) + rank 4 images")
    out = run_nd(env, torch.from_numpy(m).to(dev), None, batch_dims=2)
    check_images(m, out, None, 2)
    assert (out["indices"][1, 2] == -(5 * 6 * 7)).all()


def test_strided_views(env):
    """Slices, steps and transposes: the mask is read through its strides."""
    torch, dev = env
    rng = np.random.default_rng([42, 9102])
    base = torch.from_numpy((rng.random((130, 70, 90)) >= 0.01).astype(np.uint8)).to(dev)
    views = {
        "transpose 2-D": base[5].t(),
        "step 2 slice 3-D": base[::2, 3:60:3, ::2],
        "permuted 3-D": base.permute(2, 0, 1),
        "sliced rows 2-D": base[0, :, 1:80],
        "step 1-D": base[:, 0, 0][::3],
        "channels-last 4-D": base.reshape(130, 70, 9, 10).permute(0, 3, 1, 2),
    }
    for name, v in views.items():
        assert not v.is_contiguous()
        vn = np.ascontiguousarray(v.cpu().numpy())
        if not (vn == 0).any():
            continue
        _say(f"strided view: {name} {tuple(v.shape)} strides {v.stride()}")
        out = run_nd(env, v, None)
        check_images(vn, out, None, 0)


def test_long_rows_and_big_extents(env):
    """Rows beyond the LDS envelope (2-D W > 32768, 3-D W > 16384, 3-D H >
    32768) take reordered runs of the LDS kernels; extents over 65535 the
    workspace path (its longest axis first when that axis has few lines)."""
    torch, dev = env
    rng = np.random.default_rng([42, 9103])
    cases = [((40, 40000), 0.0005, None), ((3, 4, 20000), 0.001, (2.5, 1.0, 1.0)),
             ((2, 40000, 3), 0.0005, None), ((70000, 3), 0.0002, None), ((100000,), 0.0001, None),
             ((3, 70000), 0.0003, (1.0, 0.5)), ((4, 5, 70000), 0.0005, (1.0, 2.0, 0.5)),
             ((2, 90000, 3), 0.0005, None)]
    for shape, p, samp in cases:
        m = (rng.random(shape) >= p).astype(np.uint8)
        m.reshape(-1)[-1] = 0
        _say(f"long/big {shape} sampling={samp}")
        # int32 squared distances only where every possible one fits (the
        # call refuses sqdist otherwise)
        fits = sum(n * n for n in shape) <= 2**31 - 1
        want = ("sqdist", "dist", "indices") if samp is None and fits else ("dist", "indices")
        out = run_nd(env, torch.from_numpy(m).to(dev), samp, want=want)
        check_images(m, out, samp, 0)
        if not fits:
            from exact_euclidean_distance_amd import EDTError, edt
            with pytest.raises(EDTError):
                edt(torch.from_numpy(m).to(dev), return_sqdist=True)


def test_routes_agree(env):
    """A C-contiguous 2-D batch runs the LDS kernels, the same values read
    through a strided view the workspace path: both equal the oracle and each
    other on distances."""
    torch, dev = env
    rng = np.random.default_rng([42, 9104])
    m = (rng.random((3, 300, 257)) >= 0.01).astype(np.uint8)
    wide = torch.ones((3, 300, 260), dtype=torch.uint8, device=dev)
    wide[:, :, :257] = torch.from_numpy(m).to(dev)
    view = wide[:, :, :257]
    assert not view.is_contiguous()
    fast = run_nd(env, torch.from_numpy(m).to(dev), None, batch_dims=1)
    slow = run_nd(env, view, None, batch_dims=1)
    check_images(m, fast, None, 1)
    check_images(m, slow, None, 1)
    assert (fast["sqdist"] == slow["sqdist"]).all()


def test_unravel_nd(env):
    torch, dev = env
    from exact_euclidean_distance_amd import unravel_indices
    rng = np.random.default_rng([42, 9105])
    img = (3, 4, 5, 6, 7)
    n = int(np.prod(img))
    for dt, npdt in ((torch.int32, np.int32), (torch.int64, np.int64)):
        flat = rng.integers(0, n, (2,) + img).astype(npdt)
        flat[0, 0, 0, 0, 0, :] = -(n // img[0])     # virtual elements
        c = unravel_indices(torch.from_numpy(flat).to(dev), img).cpu().numpy()
        assert c.dtype == npdt and c.shape == (2, 5) + img
        f = flat.astype(np.int64)
        for k in range(len(img) - 1, 0, -1):
            ref = np.mod(f, img[k])
            f = np.floor_divide(f, img[k])
            assert (c[:, k] == ref).all()
        assert (c[:, 0] == f).all()
        assert (c[0, :, 0, 0, 0, 0, 0] == np.array([-1, 0, 0, 0, 0])).all()


def test_reordered_runs(env):
    """Shapes whose axes are reordered for the LDS kernels (rows past their
    limits, strided masks, int64 indices of 2-D images), with images without
    background among them: the virtual element stays (-1, 0, ...) of the
    original axis 0."""
    torch, dev = env
    rng = np.random.default_rng([42, 9106])
    cases = [((3, 60, 40000), 1, None), ((2, 3, 5, 20000), 1, (2.5, 1.0, 0.5)),
             ((2, 20000, 5, 3), 1, None), ((4, 70, 33000), 1, (1.0, 2.5))]
    for shape, nb, samp in cases:
        m = (rng.random(shape) >= 0.002).astype(np.uint8)
        m[1] = 1                                   # an image without background
        m.reshape(shape[0], -1)[0, -1] = 0
        _say(f"reordered run {shape} batch_dims={nb} sampling={samp}")
        want = ("sqdist", "dist", "indices") if samp is None else ("dist", "indices")
        mt = torch.from_numpy(m).to(dev)
        out = run_nd(env, mt, samp, batch_dims=nb, want=want)
        check_images(m, out, samp, nb)
        img = shape[nb:]
        assert (out["indices"][1] == -int(np.prod(img[1:]))).all()
        out64 = run_nd(env, mt, samp, batch_dims=nb, index_dtype=torch.int64, want=("indices",))
        check_images(m, out64, samp, nb)
    # a strided 2-D view with int64 indices, and a transposed 3-D view
    base = torch.from_numpy((rng.random((2, 300, 500)) >= 0.003).astype(np.uint8)).to(dev)
    base[1] = 1
    for v in (base[:, ::2, 1:400], base.permute(0, 2, 1)):
        vn = np.ascontiguousarray(v.cpu().numpy())
        _say(f"reordered strided view {tuple(v.shape)} strides {v.stride()}")
        out = run_nd(env, v, None, batch_dims=1, index_dtype=torch.int64)
        check_images(vn, out, None, 1)
    v3 = base.reshape(2, 300, 20, 25).permute(0, 3, 1, 2)
    vn = np.ascontiguousarray(v3.cpu().numpy())
    _say(f"reordered strided view {tuple(v3.shape)}")
    check_images(vn, run_nd(env, v3, (1.5, 1.0, 2.0), batch_dims=1, want=("dist", "indices")), (1.5, 1.0, 2.0), 1)


def test_long_lines_in_segments(env):
    """Few long lines along axis 0 run in segments of 64 (per-segment
    summaries, carries across segments): a 1-D signal of 2^20 with sparse
    background, one whose only background is at the start (a carry across
    every segment), ties at segment edges, and a tall 2-D image."""
    torch, dev = env
    rng = np.random.default_rng([42, 9107])
    n = 1 << 20
    sig = (rng.random(n) >= 2e-4).astype(np.uint8)
    sig[-1] = 0
    edge = np.ones(4096, np.uint8)
    edge[[255, 769, 1024, 3000]] = 0          # midpoints fall on segment edges
    first = np.ones(300000, np.uint8)
    first[0] = 0
    tall = (rng.random((90000, 5)) >= 0.001).astype(np.uint8)
    tall[-1] = 0
    for name, m, samp in (("signal 2^20", sig, None), ("background at the start", first, (0.5,)),
                          ("ties at segment edges", edge, None), ("tall 90000 x 5", tall, (2.5, 1.0))):
        _say(f"segmented axis 0: {name} {m.shape}")
        fits = sum(k * k for k in m.shape) <= 2**31 - 1
        want = ("sqdist", "dist", "indices") if samp is None and fits else ("dist", "indices")
        out = run_nd(env, torch.from_numpy(m).to(dev), samp, want=want)
        check_images(m, out, samp, 0)
