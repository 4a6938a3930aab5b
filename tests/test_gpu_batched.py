"""GPU parity of the batched 2-D and 1-D entry points, of the per-axis index
layout and of PR-EDT's own workloads, through the C ABI, against the CPU
oracle run image by image.

Same bar as the single-image tests: int32 squared distances bit-exact (unit
spacing), float32 distances within 1e-6 / 1e-5 relative, every index attains
the oracle's minimum exactly.  Outputs are poisoned before each call.
"""

import numpy as np
import pytest

import oracle
from gpu_check import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from exact_euclidean_distance_amd import _lib
    _lib.load()
    return torch, torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _poisoned(torch, dev, shape, want):
    sq = torch.full(shape, -7, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.full(shape, float("nan"), dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.full(shape, -7, dtype=torch.int32, device=dev) if "indices" in want else None
    return sq, ds, ix


def _np(t):
    return None if t is None else t.cpu().numpy()


def run_batched_2d(torch_dev, masks, sampling=None):
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt2d
    iso = sampling is None or all(float(s) == 1.0 for s in sampling)
    want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
    sq, ds, ix = _poisoned(torch, dev, masks.shape, want)
    edt2d(torch.from_numpy(masks).to(dev), sampling, sqdist=sq, dist=ds, indices=ix)
    torch.cuda.synchronize()
    ref = np.stack([oracle.edt(m, sampling, features=False)[0] for m in masks])
    compare(masks, sampling, ref, _np(sq), _np(ds), _np(ix), batch=True)
    return ref, _np(ix)


def test_batched_2d_matches_per_image(torch_dev):
    rng = np.random.default_rng([42, 5001])
    # few short lines (one wave per line), many lines (chunk kernel), long rows
    for shape in ((5, 40, 70), (3, 1, 517), (70, 1000, 3), (2, 37, 1031), (4, 300, 260)):
        for p in (0.003, 0.2):
            masks = (rng.random(shape) >= p).astype(np.uint8)
            for b in range(shape[0]):
                masks[b].reshape(-1)[rng.integers(masks[b].size)] = 0
            _say(f"batched 2d {shape} p={p}")
            run_batched_2d(torch_dev, masks)
            run_batched_2d(torch_dev, masks, (2.5, 1.0))
            run_batched_2d(torch_dev, masks, (0.5, 1.25))


def test_batched_2d_image_without_background(torch_dev):
    """Each image of a batch takes the virtual element on its own."""
    rng = np.random.default_rng([42, 5002])
    masks = (rng.random((4, 33, 90)) >= 0.01).astype(np.uint8)
    masks[0] = 1
    masks[2] = 1
    masks[1, 0, 0] = 0
    masks[3, 32, 89] = 0
    _say("batched 2d with empty images")
    ref, ix = run_batched_2d(torch_dev, masks)
    H, W = masks.shape[1:]
    r, c = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    for b in (0, 2):
        assert (ref[b] == (r + 1) ** 2 + c ** 2).all()
        assert (ix[b] == -W).all()


def test_batched_2d_equals_single_calls(torch_dev):
    """The batched entry point gives bit-identical outputs to one call per image."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt2d
    rng = np.random.default_rng([42, 5003])
    masks = (rng.random((3, 129, 4100)) >= 0.001).astype(np.uint8)
    masks[:, 5, 7] = 0
    m = torch.from_numpy(masks).to(dev)
    rb = edt2d(m, return_sqdist=True, return_indices=True)
    for b in range(3):
        r1 = edt2d(m[b].contiguous(), return_sqdist=True, return_indices=True)
        torch.cuda.synchronize()
        assert torch.equal(rb.sqdist[b], r1.sqdist)
        assert torch.equal(rb.dist[b], r1.dist)
        assert torch.equal(rb.indices[b], r1.indices)


def test_1d_lines(torch_dev):
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt1d
    rng = np.random.default_rng([42, 5004])
    # 46000: the longest line whose squared distances (up to N^2) fit in int32
    for B, N in ((1, 1), (1, 7), (5, 1000), (300, 257), (2, 46000)):
        for p in (0.001, 0.05, 0.6):
            masks = (rng.random((B, N)) >= p).astype(np.uint8)
            masks[0] = 1                       # a line without background
            for s in (None, (2.5,)):
                iso = s is None
                want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
                sq, ds, ix = _poisoned(torch, dev, (B, N), want)
                edt1d(torch.from_numpy(masks).to(dev), s, sqdist=sq, dist=ds, indices=ix)
                torch.cuda.synchronize()
                ref = np.stack([oracle.edt(m, s, features=False)[0] for m in masks])
                _say(f"1d B={B} N={N} p={p} s={s}")
                compare(masks, s, ref, _np(sq), _np(ds), _np(ix), batch=True)
                pos = np.arange(N)
                s0 = 1.0 if s is None else s[0]
                assert (ref[0] == (s0 * (pos + 1.0)) ** 2).all()
                assert (_np(ix)[0] == -1).all()
    # longer lines: distances only (their squared distances would overflow int32)
    from exact_euclidean_distance_amd import EDTError
    masks = (rng.random((2, 65535)) >= 0.001).astype(np.uint8)
    masks[0] = 1
    with pytest.raises(EDTError):
        edt1d(torch.from_numpy(masks).to(dev), return_sqdist=True)
    sq, ds, ix = _poisoned(torch, dev, masks.shape, ("dist", "indices"))
    edt1d(torch.from_numpy(masks).to(dev), dist=ds, indices=ix)
    torch.cuda.synchronize()
    ref = np.stack([oracle.edt(m, None, features=False)[0] for m in masks])
    compare(masks, None, ref, None, _np(ds), _np(ix), batch=True)
    # a single (N,) line
    mask = np.ones(50, np.uint8)
    mask[[3, 40]] = 0
    r = edt1d(torch.from_numpy(mask).to(dev), return_sqdist=True, return_indices=True)
    torch.cuda.synchronize()
    ref, _ = oracle.edt(mask, None, features=False)
    compare(mask, None, ref, _np(r.sqdist), _np(r.dist), _np(r.indices))


def _unravel_ref(flat, shape):
    """Floor-division unravel of flat indices (NumPy), per image."""
    f = flat.astype(np.int64)
    out = []
    for n in reversed(shape[1:]):
        out.append(np.mod(f, n))
        f = np.floor_divide(f, n)
    out.append(f)
    return np.stack(out[::-1]).astype(np.int32)


def test_unravel_indices(torch_dev):
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt2d, edt3d, unravel_indices
    rng = np.random.default_rng([42, 5005])
    # 3-D batch with a volume without background: its coordinates are (-1, 0, 0)
    vols = (rng.random((3, 9, 17, 30)) >= 0.02).astype(np.uint8)
    vols[1] = 1
    vols[0, 0, 0, 0] = 0
    vols[2, 8, 16, 29] = 0
    r = edt3d(torch.from_numpy(vols).to(dev), return_indices=True)
    co = unravel_indices(r.indices, vols.shape[1:])
    torch.cuda.synchronize()
    assert tuple(co.shape) == (3, 3, 9, 17, 30)
    flat = r.indices.cpu().numpy()
    got = co.cpu().numpy()
    for b in range(3):
        assert (got[b] == _unravel_ref(flat[b], vols.shape[1:])).all()
    assert (got[1, 0] == -1).all() and (got[1, 1:] == 0).all()
    _, feat = oracle.edt(vols[1], None, features=True)
    assert (np.moveaxis(got[1], 0, -1) == feat).all()
    # single background element: the coordinates are that element everywhere
    vol = np.ones((1, 6, 7, 8), np.uint8)
    vol[0, 2, 3, 4] = 0
    r = edt3d(torch.from_numpy(vol).to(dev), return_indices=True)
    co = unravel_indices(r.indices, vol.shape[1:]).cpu().numpy()
    assert (co[0, 0] == 2).all() and (co[0, 1] == 3).all() and (co[0, 2] == 4).all()
    # 2-D batch and one image; 1-D
    imgs = (rng.random((2, 31, 45)) >= 0.05).astype(np.uint8)
    imgs[0] = 1
    imgs[1, 3, 3] = 0
    r = edt2d(torch.from_numpy(imgs).to(dev), return_indices=True)
    co = unravel_indices(r.indices, imgs.shape[1:]).cpu().numpy()
    flat = r.indices.cpu().numpy()
    for b in range(2):
        assert (co[b] == _unravel_ref(flat[b], imgs.shape[1:])).all()
    assert (co[0, 0] == -1).all() and (co[0, 1] == 0).all()
    co1 = unravel_indices(r.indices[1].contiguous(), imgs.shape[1:]).cpu().numpy()
    assert (co1 == co[1]).all()
    flat1 = torch.tensor([-1, 0, 3, 2], dtype=torch.int32, device=dev)   # one line of 4
    assert (unravel_indices(flat1, (4,)).cpu().numpy() == [[-1, 0, 3, 2]]).all()


def test_full_size_batched_workload(torch_dev):
    """The batched 2-D workload the benchmark times, at full size, with the
    outputs it times."""
    from workloads import make_config
    masks, sampling, _ = make_config("b2d")
    _say(f"b2d {masks.shape}: GPU + oracle")
    run_batched_2d(torch_dev, masks, sampling)


@pytest.mark.parametrize("name", ["p1_1024_1", "p1_1024_99", "p1_8192_1", "p1_8192_99"])
def test_pr_edt_workloads(torch_dev, name):
    """PR-EDT's own workloads (random squares, seed 42, 1 % / 99 % background),
    as benchmarked, with exact squared distances and indices checked too."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt2d
    from workloads import make_config
    mask, _, _ = make_config(name)
    _say(f"{name}: GPU + oracle")
    sq, ds, ix = _poisoned(torch, dev, mask.shape, ("sqdist", "dist", "indices"))
    edt2d(torch.from_numpy(mask).to(dev), sqdist=sq, dist=ds, indices=ix)
    torch.cuda.synchronize()
    ref, _ = oracle.edt(mask, None, features=False)
    compare(mask, None, ref, _np(sq), _np(ds), _np(ix))


def test_brute_force_transform(torch_dev):
    """The device brute force against the oracle's brute force (the definition;
    both return the smallest index among equally near background elements,
    so indices match exactly) and against the separable GPU path."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt1d, edt2d, edt3d, edt_brute
    rng = np.random.default_rng([42, 5006])
    cases = [((40,), None), ((300,), (2.5,)), ((23, 57), None), ((64, 64), (2.5, 1.0)),
             ((9, 13, 17), None), ((16, 16, 16), (2.5, 1.0, 1.0)), ((5, 31, 2), (0.5, 1.25, 2.0))]
    for shape, samp in cases:
        for p in (0.002, 0.05, 0.5):
            mask = (rng.random(shape) >= p).astype(np.uint8)
            mask.reshape(-1)[rng.integers(mask.size)] = 0
            iso = samp is None
            _say(f"brute {shape} p={p} s={samp}")
            r = edt_brute(torch.from_numpy(mask).to(dev), samp, return_sqdist=iso, return_indices=True)
            torch.cuda.synchronize()
            ref, feat = oracle.edt_brute(mask, samp, features=True)
            compare(mask, samp, ref, _np(r.sqdist), _np(r.dist), _np(r.indices))
            assert (_np(r.indices) == oracle.flat_index(feat, mask.shape)).all()
    # batched, with an image without background (virtual element)
    masks = (rng.random((3, 20, 30)) >= 0.02).astype(np.uint8)
    masks[1] = 1
    masks[0, 0, 0] = 0
    masks[2, 19, 29] = 0
    r = edt_brute(torch.from_numpy(masks).to(dev), batched=True, return_sqdist=True,
                  return_indices=True)
    torch.cuda.synchronize()
    ref = np.stack([oracle.edt_brute(m, None, features=False)[0] for m in masks])
    compare(masks, None, ref, _np(r.sqdist), _np(r.dist), _np(r.indices), batch=True)
    assert (_np(r.indices)[1] == -30).all()
    # the device check of the fast path on sizes beyond the quick CPU brute force
    m2 = (rng.random((2, 700, 900)) >= 0.003).astype(np.uint8)
    m2[:, 1, 1] = 0
    t2 = torch.from_numpy(m2).to(dev)
    a = edt_brute(t2, batched=True, return_sqdist=True)
    b = edt2d(t2, return_sqdist=True)
    m3 = (rng.random((2, 40, 50, 60)) >= 0.01).astype(np.uint8)
    m3[:, 0, 0, 0] = 0
    t3 = torch.from_numpy(m3).to(dev)
    c = edt_brute(t3, (2.5, 1.0, 1.0), batched=True)
    d = edt3d(t3, (2.5, 1.0, 1.0))
    m1 = (rng.random((4, 5000)) >= 0.01).astype(np.uint8)
    m1[:, 0] = 0
    t1 = torch.from_numpy(m1).to(dev)
    e = edt_brute(t1, batched=True, return_sqdist=True)
    f = edt1d(t1, return_sqdist=True)
    torch.cuda.synchronize()
    assert torch.equal(a.sqdist, b.sqdist) and torch.equal(a.dist, b.dist)
    assert torch.equal(c.dist, d.dist)
    assert torch.equal(e.sqdist, f.sqdist)


def test_brute_force_metrics(torch_dev):
    """The device brute force of the city-block and chessboard metrics (and
    the integer squared Euclidean one at unit spacing) against the oracle's
    brute forces: distances and the smallest-index minimiser equal, on 1-3
    axes, batches with an image without background, and ragged tile tails."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt_brute
    rng = np.random.default_rng([42, 5020])
    shapes = [(1,), (37,), (1, 1), (23, 57), (64, 65), (9, 13, 17), (5, 31, 2), (1, 300, 3)]
    for shape in shapes:
        for p in (0.003, 0.05, 0.5, 1.0):
            mask = (rng.random(shape) >= p).astype(np.uint8)
            mask.reshape(-1)[rng.integers(mask.size)] = 0
            t = torch.from_numpy(mask).to(dev)
            for metric, fn in (("taxicab", oracle.taxicab_brute), ("chessboard", oracle.chessboard_brute)):
                _say(f"brute {metric} {shape} p={p}")
                r = edt_brute(t, metric=metric, return_indices=True)
                torch.cuda.synchronize()
                ref, who = fn(mask)
                assert (_np(r.dist) == ref).all(), f"{metric} distance mismatch"
                assert (_np(r.indices) == who).all(), f"{metric} minimiser is not the smallest index"
            r = edt_brute(t, return_sqdist=True, return_indices=True)
            torch.cuda.synchronize()
            ref, feat = oracle.edt_brute(mask, None, features=True)
            assert (_np(r.sqdist) == ref).all()
            assert (_np(r.indices) == oracle.flat_index(feat, mask.shape)).all()
    masks = (rng.random((4, 30, 70)) >= 0.02).astype(np.uint8)
    masks[1] = 1
    masks[3] = 0
    t = torch.from_numpy(masks).to(dev)
    for metric, fn in (("taxicab", oracle.taxicab_brute), ("chessboard", oracle.chessboard_brute)):
        _say(f"brute {metric} batch with an image without background")
        r = edt_brute(t, batched=True, metric=metric, return_indices=True)
        torch.cuda.synchronize()
        for b in range(4):
            ref, who = fn(masks[b])
            assert (_np(r.dist)[b] == ref).all() and (_np(r.indices)[b] == who).all()
    with pytest.raises(ValueError):
        edt_brute(t, (2.0, 1.0), batched=True, metric="taxicab")


def test_randomized_sweep(torch_dev):
    """Seeded random cases across every entry point: shapes (ragged, tiny,
    lines of one), densities, dyadic spacings (exact in float64), images
    without background inside batches and full background lines.  Each case
    is checked against the oracle and, bit for bit, against the device brute
    force (both exact)."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt1d, edt2d, edt3d, edt_brute
    rng = np.random.default_rng([42, 5007])
    spacings = (0.5, 1.0, 1.25, 2.5)
    for case in range(200):
        kind = case % 4
        if kind == 0:
            shape = (int(rng.integers(1, 4)), int(rng.integers(1, 700)))
        elif kind == 1:
            shape = (int(rng.integers(1, 260)), int(rng.integers(1, 260)))
        elif kind == 2:
            shape = (int(rng.integers(1, 5)), int(rng.integers(1, 120)), int(rng.integers(1, 120)))
        else:
            shape = (int(rng.integers(1, 4)), int(rng.integers(1, 30)), int(rng.integers(1, 30)),
                     int(rng.integers(1, 40)))
        p = float(rng.choice([0.0005, 0.01, 0.1, 0.5, 0.95]))
        mask = (rng.random(shape) >= p).astype(np.uint8)
        batched = kind in (0, 2, 3)
        imgs = mask if batched else mask[None]
        for b in range(imgs.shape[0]):
            r = rng.random()
            if r < 0.15:
                imgs[b] = 1                                  # no background
            elif r < 0.3:
                ax = int(rng.integers(imgs[b].ndim))         # a full background line / plane
                sl = [slice(None)] * imgs[b].ndim
                sl[ax] = int(rng.integers(imgs[b].shape[ax]))
                imgs[b][tuple(sl)] = 0
        nd = imgs.ndim - 1
        samp = None if rng.random() < 0.5 else tuple(float(rng.choice(spacings)) for _ in range(nd))
        iso = samp is None or all(s == 1.0 for s in samp)
        want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
        t = torch.from_numpy(mask).to(dev)
        sq, ds, ix = _poisoned(torch, dev, mask.shape, want)
        fn = {0: edt1d, 1: edt2d, 2: edt2d, 3: edt3d}[kind]
        _say(f"sweep {case}: {fn.__name__} {shape} p={p} s={samp}")
        fn(t, samp, sqdist=sq, dist=ds, indices=ix)
        br = edt_brute(t, samp, batched=batched, return_sqdist=iso)
        torch.cuda.synchronize()
        ref = np.stack([oracle.edt(m, samp, features=False)[0] for m in imgs])
        compare(imgs, samp, ref, None if sq is None else _np(sq).reshape(imgs.shape), _np(ds).reshape(imgs.shape),
                _np(ix).reshape(imgs.shape), batch=True)
        assert torch.equal(br.dist, ds)
        if iso:
            assert torch.equal(br.sqdist, sq)


def _brute_points(pos, pts, s2):
    """Exact squared distance of each position (rows of pos) to the nearest of
    the background points pts (float64, chunked)."""
    out = np.full(len(pos), np.inf)
    for i in range(0, len(pos), 1 << 16):
        d = ((pos[i:i + (1 << 16), None, :] - pts[None, :, :]).astype(np.float64) ** 2 * s2).sum(-1)
        out[i:i + (1 << 16)] = d.min(1)
    return out


@pytest.mark.timeout(600)
def test_volume_over_2_31_elements(torch_dev):
    """A volume of 2100 x 1024 x 1000 (2.15e9 voxels, more than int32 can
    index; about 24 GB of HBM with its workspace): distances with 64-bit
    offsets everywhere.  Checked exactly on the whole last plane (offsets past
    2^31) and on a million random voxels against brute force over the
    background points; indices are refused.  Then three volumes with indices
    whose batch together passes 2^31 elements."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import EDTError, edt3d
    rng = np.random.default_rng([42, 5008])
    D, H, W = 2100, 1024, 1000
    n = D * H * W
    assert n > 2 ** 31
    flat = np.ones(n, np.uint8)
    bg = rng.choice(n, 400, replace=False)
    # and five in the last plane, whose flat indices pass 2^31
    bg = np.unique(np.concatenate([bg, (D - 1) * H * W + rng.choice(H * W, 5, replace=False)]))
    flat[bg] = 0
    pts = np.stack(np.unravel_index(bg, (D, H, W)), 1)
    _say("volume 2100x1024x1000: transfer")
    m = torch.from_numpy(flat).to(dev).view(1, D, H, W)
    del flat
    with pytest.raises(EDTError):
        edt3d(m, return_indices=True)
    for samp in (None, (2.5, 1.0, 1.0)):
        _say(f"volume 2100x1024x1000: transform, spacing {samp}")
        r = edt3d(m, samp, return_sqdist=samp is None)
        torch.cuda.synchronize()
        s2 = np.array([1.0, 1.0, 1.0] if samp is None else [s * s for s in samp])
        yy, xx = np.indices((H, W))
        last = np.stack([np.full(H * W, D - 1), yy.ravel(), xx.ravel()], 1)
        pick = np.sort(rng.choice(n, 1_000_000, replace=False))
        rand = np.stack(np.unravel_index(pick, (D, H, W)), 1)
        pos = np.concatenate([last, rand])
        lin = torch.from_numpy(np.ravel_multi_index(pos.T, (D, H, W))).to(dev)
        ref = _brute_points(pos, pts, s2)
        got = r.dist.view(-1)[lin].cpu().numpy().astype(np.float64)
        tol = 1e-6 if samp is None else 1e-5
        assert np.all(np.abs(got - np.sqrt(ref)) <= tol * np.sqrt(ref)), "dist mismatch"
        if samp is None:
            assert (r.sqdist.view(-1)[lin].cpu().numpy() == ref).all(), "sqdist mismatch"
        del r
    _say("volume 2100x1024x1000: int64 indices")
    r = edt3d(m, return_distances=False, return_indices=True, index_dtype=torch.int64)
    torch.cuda.synchronize()
    got = r.indices.view(-1)[lin].cpu().numpy()
    fz, fy, fx = np.unravel_index(got, (D, H, W))
    d2 = (fz - pos[:, 0]) ** 2 + (fy - pos[:, 1]) ** 2 + (fx - pos[:, 2]) ** 2
    ref = _brute_points(pos, pts, np.ones(3))
    assert (d2 == ref).all(), "int64 index does not attain the minimum"
    assert (got.reshape(-1)[:H * W] >= 2 ** 31).any()   # the last plane's owners lie past 2^31
    del r, m
    torch.cuda.empty_cache()
    # a batch over 2^31 elements in total, indices within each volume
    B, D, H, W = 3, 700, 1024, 1024
    flat = np.ones(B * D * H * W, np.uint8)
    per = D * H * W
    pts3 = []
    for b in range(B):
        bgb = rng.choice(per, 300, replace=False)
        flat[b * per + bgb] = 0
        pts3.append(np.stack(np.unravel_index(bgb, (D, H, W)), 1))
    _say("batch 3x700x1024x1024: transform with indices")
    m = torch.from_numpy(flat).to(dev).view(B, D, H, W)
    del flat
    r = edt3d(m, return_sqdist=True, return_indices=True)
    torch.cuda.synchronize()
    b = B - 1
    yy, xx = np.indices((H, W))
    pos = np.stack([np.full(H * W, D - 1), yy.ravel(), xx.ravel()], 1)
    ref = _brute_points(pos, pts3[b], np.ones(3))
    got_sq = r.sqdist[b, D - 1].cpu().numpy().ravel()
    got_ix = r.indices[b, D - 1].cpu().numpy().ravel().astype(np.int64)
    assert (got_sq == ref).all()
    fz, fy, fx = np.unravel_index(got_ix, (D, H, W))
    d2 = (fz - pos[:, 0]) ** 2 + (fy - pos[:, 1]) ** 2 + (fx - pos[:, 2]) ** 2
    assert (d2 == ref).all(), "index does not attain the minimum"


def test_int64_indices_small(torch_dev):
    """int64 indices (chunk row kernel for any shape) attain the minimum and
    come with the same distances as the int32 call."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt3d
    rng = np.random.default_rng([42, 5009])
    for shape, samp in (((2, 9, 17, 30), None), ((1, 40, 33, 70), (2.5, 1.0, 1.0)),
                        ((3, 5, 7, 513), None), ((2, 20, 30, 40), (0.5, 1.25, 1.0))):
        vols = (rng.random(shape) >= 0.02).astype(np.uint8)
        vols[0] = 1                                   # a volume without background
        vols[-1].reshape(-1)[0] = 0
        t = torch.from_numpy(vols).to(dev)
        iso = samp is None
        r64 = edt3d(t, samp, return_sqdist=iso, return_indices=True, index_dtype=torch.int64)
        r32 = edt3d(t, samp, return_sqdist=iso, return_indices=True)
        torch.cuda.synchronize()
        assert r64.indices.dtype == torch.int64
        assert torch.equal(r64.dist, r32.dist)
        if iso:
            assert torch.equal(r64.sqdist, r32.sqdist)
        ix = r64.indices.cpu().numpy()
        assert (np.abs(ix) < 2 ** 31).all()
        ref = np.stack([oracle.edt(v, samp, features=False)[0] for v in vols])
        _say(f"int64 indices {shape} s={samp}")
        compare(vols, samp, ref, None, None, ix.astype(np.int32), batch=True)


def test_channel_axes(torch_dev):
    """(B, C, H, W) and (B, C, D, H, W) inputs: every (batch, channel) image
    or volume is transformed on its own."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt2d, edt3d
    rng = np.random.default_rng([42, 5010])
    m = (rng.random((2, 3, 40, 70)) >= 0.02).astype(np.uint8)
    m[1, 2] = 1
    m[0, 0, 0, 0] = 0
    r = edt2d(torch.from_numpy(m).to(dev), return_sqdist=True, return_indices=True)
    torch.cuda.synchronize()
    assert tuple(r.sqdist.shape) == m.shape
    flat = m.reshape(-1, 40, 70)
    ref = np.stack([oracle.edt(x, None, features=False)[0] for x in flat])
    compare(flat, None, ref, _np(r.sqdist).reshape(flat.shape), _np(r.dist).reshape(flat.shape),
            _np(r.indices).reshape(flat.shape), batch=True)
    v = (rng.random((2, 2, 9, 20, 30)) >= 0.02).astype(np.uint8)
    v[0, 1] = 1
    v[1, 1, 0, 0, 0] = 0
    r = edt3d(torch.from_numpy(v).to(dev), (2.5, 1.0, 1.0), return_indices=True)
    torch.cuda.synchronize()
    flat = v.reshape(-1, 9, 20, 30)
    ref = np.stack([oracle.edt(x, (2.5, 1.0, 1.0), features=False)[0] for x in flat])
    compare(flat, (2.5, 1.0, 1.0), ref, None, _np(r.dist).reshape(flat.shape),
            _np(r.indices).reshape(flat.shape), batch=True)


def test_long_middle_axis(torch_dev):
    """Volumes whose middle axis is longer than 1024 (stacks of 2048^2 and
    larger slices): column tiles of 512 / Gp lines, down to one line per block
    at H = 32768; ragged lengths, spacing, and a full background plane."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import edt3d
    rng = np.random.default_rng([42, 5011])
    # (middle axes over 4096 with several lines per tile: each line keeps two
    # or more occupancy words, 4100 -> 4 lines per tile, 8200 -> 2)
    for shape, p in (((1, 3, 2048, 40), 0.002), ((2, 2, 4100, 17), 0.001), ((1, 3, 8200, 9), 0.001),
                     ((1, 2, 16384, 6), 0.0005), ((1, 1, 32768, 3), 0.0003)):
        vols = (rng.random(shape) >= p).astype(np.uint8)
        vols[:, 0, 0, 0] = 0
        for samp in (None, (2.5, 1.0, 1.0)):
            iso = samp is None
            want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
            sq, ds, ix = _poisoned(torch, dev, vols.shape, want)
            edt3d(torch.from_numpy(vols).to(dev), samp, sqdist=sq, dist=ds, indices=ix)
            torch.cuda.synchronize()
            ref = np.stack([oracle.edt(v, samp, features=False)[0] for v in vols])
            _say(f"long middle axis {shape} s={samp}")
            compare(vols, samp, ref, _np(sq), _np(ds), _np(ix), batch=True)
    vols = np.ones((1, 4, 3000, 20), np.uint8)
    vols[0, :, :, 7] = 0                          # full background plane across the last axis
    vols[0, 1, 1500, :] = 0
    ref = np.stack([oracle.edt(v, None, features=False)[0] for v in vols])
    sq, ds, ix = _poisoned(torch, dev, vols.shape, ("sqdist", "dist", "indices"))
    edt3d(torch.from_numpy(vols).to(dev), sqdist=sq, dist=ds, indices=ix)
    torch.cuda.synchronize()
    compare(vols, None, ref, _np(sq), _np(ds), _np(ix), batch=True)


def test_taxicab(torch_dev):
    """City-block transform against the L1 oracle (its definition): exact int32
    distances, indices attaining them; 2-D, batched 2-D (rows up to 20000 across
    several waves), batched 3-D, images without background, full background
    lines."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import taxicab
    rng = np.random.default_rng([42, 5012])
    # rows of 1, 2, 4 and 8 tiles of 256, of one wave and of several; middle
    # axes up to 32768
    cases = [(1, 1), (1, 70), (37, 1), (64, 64), (4, 300), (33, 517), (3, 1100), (5, 20000),
             (3, 40, 70), (2, 13, 17, 30), (3, 9, 40, 64), (2, 3, 5, 400), (1, 5, 1100, 33),
             (1, 2, 3, 2000), (2, 1, 4100, 3), (2, 1, 32768, 2)]
    for shape in cases:
        # (dense backgrounds only on small cases: the oracle is a brute force)
        for p in ((0.003, 0.1, 0.6) if np.prod(shape) <= 20000 else (0.002,)):
            m = (rng.random(shape) >= p).astype(np.uint8)
            if len(shape) > 2:
                m[0] = 1                                 # one image/volume without background
            m.reshape(-1)[-1] = 0
            if len(shape) == 2 and shape[0] > 2:
                m[shape[0] // 2, :] = 0                  # a full background row
            r = taxicab(torch.from_numpy(m).to(dev), return_indices=True)
            torch.cuda.synchronize()
            d = r.dist.cpu().numpy()
            ix = r.indices.cpu().numpy()
            batch = [m] if len(shape) == 2 else list(m)
            dd = [d] if len(shape) == 2 else list(d)
            ii = [ix] if len(shape) == 2 else list(ix)
            _say(f"taxicab {shape} p={p}")
            for mm, d1, i1 in zip(batch, dd, ii):
                ref, _ = oracle.taxicab_brute(mm)
                assert (d1 == ref).all(), "taxicab distance mismatch"
                assert (oracle.taxicab_to(i1, mm.shape) == ref).all(), "index does not attain it"
                if (mm == 0).any():
                    assert (mm.reshape(-1)[i1.reshape(-1)] == 0).all()


@pytest.mark.parametrize("name", ["b2d", "c5", "c3", "c2b"])
def test_taxicab_full_size(torch_dev, name):
    """City-block transform at the full sizes that bench.py --taxicab times, in
    the same launch shapes: over the whole output, every index names a
    background element of its image at exactly the returned L1 distance
    (checked on the device), and sampled elements plus the corners equal
    the definition's minimum (oracle, one by one)."""
    torch, dev = torch_dev
    from workloads import make_config
    from exact_euclidean_distance_amd import taxicab
    mask, _, _ = make_config(name)
    _say(f"taxicab full size {name} {mask.shape}")
    m = torch.from_numpy(mask).to(dev)
    r = taxicab(m, return_indices=True)
    torch.cuda.synchronize()
    img = mask.shape[1:] if mask.ndim >= 3 else mask.shape   # one image / volume
    nb = mask.shape[0] if mask.ndim >= 3 else 1
    per = int(np.prod(img))
    d = r.dist.reshape(nb, per).long()
    ix = r.indices.reshape(nb, per).long()
    assert (ix >= 0).all(), "every benchmark image has background"
    assert (torch.gather(m.reshape(nb, per), 1, ix) == 0).all()
    flat = torch.arange(per, device=dev)
    l1 = torch.zeros_like(d)
    div = per
    for n in img:                      # decode axis by axis, first axis first
        div //= n
        a = (flat // div) % n
        b = (ix // div) % n
        l1 += (a[None, :] - b).abs()
    assert (l1 == d).all(), "an index does not attain the returned distance"
    rng = np.random.default_rng([42, 5013])
    dh = d.cpu().numpy()
    # (fewer samples where the background is large: each is a pass over all of it)
    ns = 384 if (mask == 0).sum() < 10**6 else 24
    for k in range(nb if nb <= 2 else 2):
        pts = np.concatenate([rng.integers(0, per, ns // min(nb, 2)), [0, per - 1]])
        ref = oracle.taxicab_at(mask[k] if mask.ndim >= 3 else mask, pts)
        assert (dh[k][pts] == ref).all(), f"sampled distance mismatch in image {k}"
    _brute_cross_check(torch, m, name, r.dist, "taxicab")


def _brute_cross_check(torch, m, name, dist, metric):
    """Every distance of a full-size chamfer output against the device brute
    force (the definition, itself checked against the oracle's brute force on
    small inputs) where it finishes in seconds: the 2-D workloads, not the
    512^3 volume (1.3e8 elements x 1.7e7 background elements)."""
    if m.dim() > 3:
        return
    from exact_euclidean_distance_amd import edt_brute
    _say(f"{metric} full size {name}: device brute force over the whole output")
    rb = edt_brute(m, metric=metric, batched=m.dim() == 3)
    torch.cuda.synchronize()
    assert torch.equal(rb.dist, dist), f"{metric} distance differs from the definition"


def test_chessboard(torch_dev):
    """Chessboard (L-infinity) transform against its oracle (the definition):
    exact int32 distances, indices attaining them; the same shapes as the
    taxicab test (rows of every staging form, batched 2-D, 3-D, images without
    background, full background rows)."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import chessboard
    rng = np.random.default_rng([42, 5014])
    cases = [(1, 1), (1, 70), (37, 1), (64, 64), (4, 300), (33, 517), (3, 1100), (5, 20000),
             (3, 40, 70), (2, 13, 17, 30), (3, 9, 40, 64), (2, 3, 5, 400), (1, 5, 1100, 33),
             (1, 2, 3, 2000), (1, 3, 700, 9), (2, 1, 4100, 3), (1, 3, 4100, 13), (1, 2, 8200, 7),
             (2, 1, 32768, 2)]
    for shape in cases:
        for p in ((0.003, 0.1, 0.6) if np.prod(shape) <= 20000 else (0.002,)):
            m = (rng.random(shape) >= p).astype(np.uint8)
            if len(shape) > 2:
                m[0] = 1                                 # one image/volume without background
            m.reshape(-1)[-1] = 0
            if len(shape) == 2 and shape[0] > 2:
                m[shape[0] // 2, :] = 0                  # a full background row
            _say(f"chessboard {shape} p={p}")
            r = chessboard(torch.from_numpy(m).to(dev), return_indices=True)
            torch.cuda.synchronize()
            d = r.dist.cpu().numpy()
            ix = r.indices.cpu().numpy()
            batch = [m] if len(shape) == 2 else list(m)
            dd = [d] if len(shape) == 2 else list(d)
            ii = [ix] if len(shape) == 2 else list(ix)
            for mm, d1, i1 in zip(batch, dd, ii):
                ref, _ = oracle.chessboard_brute(mm)
                assert (d1 == ref).all(), "chessboard distance mismatch"
                assert (oracle.chessboard_to(i1, mm.shape) == ref).all(), "index does not attain it"
                if (mm == 0).any():
                    assert (mm.reshape(-1)[i1.reshape(-1)] == 0).all()


@pytest.mark.parametrize("name", ["b2d", "c5", "c3", "c2b", "c2a"])
def test_chessboard_full_size(torch_dev, name):
    """Chessboard transform at the full sizes that bench.py --chessboard times:
    over the whole output, every index names a background element of its
    image at exactly the returned L-infinity distance (on the device), and
    sampled elements plus the corners equal the definition's minimum (oracle,
    one by one)."""
    torch, dev = torch_dev
    from workloads import make_config
    from exact_euclidean_distance_amd import chessboard
    mask, _, _ = make_config(name)
    _say(f"chessboard full size {name} {mask.shape}")
    m = torch.from_numpy(mask).to(dev)
    r = chessboard(m, return_indices=True)
    torch.cuda.synchronize()
    img = mask.shape[1:] if mask.ndim >= 3 else mask.shape
    nb = mask.shape[0] if mask.ndim >= 3 else 1
    per = int(np.prod(img))
    d = r.dist.reshape(nb, per).long()
    ix = r.indices.reshape(nb, per).long()
    assert (ix >= 0).all(), "every benchmark image has background"
    assert (torch.gather(m.reshape(nb, per), 1, ix) == 0).all()
    flat = torch.arange(per, device=dev)
    linf = torch.zeros_like(d)
    div = per
    for n in img:
        div //= n
        linf = torch.maximum(linf, ((flat // div) % n)[None, :].sub((ix // div) % n).abs())
    assert (linf == d).all(), "an index does not attain the returned distance"
    rng = np.random.default_rng([42, 5015])
    dh = d.cpu().numpy()
    ns = 384 if (mask == 0).sum() < 10**6 else 24
    for k in range(nb if nb <= 2 else 2):
        pts = np.concatenate([rng.integers(0, per, ns // min(nb, 2)), [0, per - 1]])
        ref = oracle.chessboard_at(mask[k] if mask.ndim >= 3 else mask, pts)
        assert (dh[k][pts] == ref).all(), f"sampled distance mismatch in image {k}"
    _brute_cross_check(torch, m, name, r.dist, "chessboard")


def test_chessboard_large_values(torch_dev):
    """The chessboard envelope kernels with large axis-0 distances (g up to
    40000; integer crossings far from the line): a tall image with a few
    background pixels, and a volume whose middle axis carries them; full
    output against the device brute force, sampled points and the corners
    against the oracle."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import chessboard, edt_brute
    rng = np.random.default_rng([42, 5017])
    m = np.ones((40000, 120), np.uint8)
    m[rng.integers(0, 40000, 6), rng.integers(0, 120, 6)] = 0
    v = np.ones((2, 3000, 900, 3), np.uint8)
    v[0, 0, 0, 0] = 0
    v[1, rng.integers(0, 3000, 4), rng.integers(0, 900, 4), rng.integers(0, 3, 4)] = 0
    for name, arr, batched in (("40000 x 120", m, False), ("2 x 3000 x 900 x 3", v, True)):
        _say(f"chessboard large values {name}")
        t = torch.from_numpy(arr).to(dev)
        r = chessboard(t, return_indices=True)
        ref = edt_brute(t, metric="chessboard", batched=batched).dist
        torch.cuda.synchronize()
        assert torch.equal(r.dist, ref), "chessboard distance differs from the definition"
        d = r.dist.cpu().numpy()
        ix = r.indices.cpu().numpy()
        imgs = [(arr, d, ix)] if not batched else list(zip(arr, d, ix))
        for a, dd, ii in imgs:
            assert (oracle.chessboard_to(ii, a.shape) == dd).all()
            pts = np.concatenate([rng.integers(0, a.size, 60), [0, a.size - 1]])
            assert (dd.reshape(-1)[pts] == oracle.chessboard_at(a, pts)).all()


def test_chessboard_long_rows_and_large_objects(torch_dev):
    """The chessboard envelope kernels where whole-line rounds are long:
    rows over 4096 with many sources far along axis 0 (dense candidates with
    large g) and a few near ones; an image covered by large disks (interior
    candidates are dominated only by sources many chunks away: witnesses far
    along the line, cascade steps); the same in the rows and columns of a
    volume.  The whole output against the device brute force (itself checked
    against the oracle's), sampled positions against the oracle's
    definition."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import chessboard, edt_brute
    rng = np.random.default_rng([42, 5016])
    cases = []
    for W in (4160, 4397):   # (4397: a ragged last chunk)
        m = np.ones((200, W), np.uint8)
        m[0, rng.random(W) < 0.4] = 0                  # sources at g = r on every row
        pts = rng.integers(0, [200, W], size=(W // 160, 2))
        m[pts[:, 0], pts[:, 1]] = 0                    # a few near sources
        m[150, 520:540] = 0
        cases.append((f"long rows 200 x {W}", m, False))
    yy, xx = np.mgrid[0:900, 0:1700]
    disks = np.zeros((900, 1700), bool)
    for cy, cx, r in ((450, 600, 420), (300, 1350, 260), (700, 1250, 180), (120, 150, 90)):
        disks |= (yy - cy) ** 2 + (xx - cx) ** 2 <= r * r
    m = disks.astype(np.uint8)                         # foreground disks, background elsewhere
    m[rng.integers(0, 900, 40), rng.integers(0, 1700, 40)] = 0
    cases.append(("large disks 900 x 1700", m, False))
    zz, yv, xv = np.mgrid[0:3, 0:240, 0:1200]
    v = ((yv - 120) ** 2 + (xv - 600) ** 2 <= 110 ** 2 + (zz * 40) ** 2).astype(np.uint8)[None]
    v[0, 1, :, 0:300] = 1                              # a long run of columns without background
    cases.append(("volume 1 x 3 x 240 x 1200", v, True))
    for name, arr, batched in cases:
        _say(f"chessboard {name}")
        t = torch.from_numpy(arr).to(dev)
        r = chessboard(t, return_indices=True)
        ref = edt_brute(t, metric="chessboard", batched=batched).dist
        torch.cuda.synchronize()
        assert torch.equal(r.dist, ref), f"chessboard distance mismatch ({name})"
        d = r.dist.cpu().numpy()
        ix = r.indices.cpu().numpy()
        imgs = [(arr, d, ix)] if not batched else list(zip(arr, d, ix))
        for a, dd, ii in imgs:
            assert (oracle.chessboard_to(ii, a.shape) == dd).all()
            assert (a.reshape(-1)[ii.reshape(-1)] == 0).all()
            pts = np.concatenate([rng.integers(0, a.size, 200), [0, a.size - 1]])
            assert (dd.reshape(-1)[pts] == oracle.chessboard_at(a, pts)).all(), f"sampled oracle mismatch ({name})"
