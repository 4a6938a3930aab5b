"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer squared distances must match bit for bit (unit spacing); float32
distances within 1e-6 relative (unit spacing) / 1e-5 (anisotropic); every
returned index must attain the oracle's minimum exactly (ties are legal).
Outputs are poisoned before each call so unwritten elements are caught.
"""

import os
import sys

import numpy as np
import pytest

import oracle
from gpu_check import compare
from golden_io import load as load_golden, names as golden_names

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from exact_euclidean_distance_amd import _lib
    _lib.load()
    return torch, torch.device("cuda:0")


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def run_gpu(torch_dev, mask, sampling=None, want=("sqdist", "dist", "indices"), offset=0, poison=0xFF):
    """Run the transform on ``mask`` (2-D, or 4-D batch of volumes); returns
    numpy outputs.  ``offset`` > 0 places the mask at a misaligned address.
    The workspace is filled with ``poison`` first (its contents on entry must
    not matter)."""
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import _lib, edt2d, edt3d
    flat = torch.from_numpy(np.ascontiguousarray(mask).reshape(-1))
    if offset:
        buf = torch.empty(flat.numel() + offset, dtype=torch.uint8, device=dev)
        buf[offset:].copy_(flat)
        m = buf[offset:].view(mask.shape)
    else:
        m = flat.to(dev).view(mask.shape)
    shape = mask.shape
    sq = torch.full(shape, -7, dtype=torch.int32, device=dev) if "sqdist" in want else None
    ds = torch.full(shape, float("nan"), dtype=torch.float32, device=dev) if "dist" in want else None
    ix = torch.full(shape, -7, dtype=torch.int32, device=dev) if "indices" in want else None
    lib = _lib.load()
    need = (lib.edt2d_workspace_size(*shape) if mask.ndim == 2 else lib.edt3d_workspace_size(*shape))
    ws = torch.full((max(1, int(need)),), poison, dtype=torch.uint8, device=dev)
    fn = edt2d if mask.ndim == 2 else edt3d
    fn(m, sampling, sqdist=sq, dist=ds, indices=ix, return_distances=ds is not None, workspace=ws)
    torch.cuda.synchronize()
    out = {}
    for k, t in (("sqdist", sq), ("dist", ds), ("indices", ix)):
        if t is not None:
            out[k] = t.cpu().numpy()
    return out


def check(torch_dev, mask, sampling=None, want=None, offset=0, ref=None):
    iso = sampling is None or all(float(s) == 1.0 for s in sampling)
    if want is None:
        want = ("sqdist", "dist", "indices") if iso else ("dist", "indices")
    out = run_gpu(torch_dev, mask, sampling, want, offset)
    if ref is None:
        if mask.ndim == 2:
            ref, _ = oracle.edt(mask, sampling, features=False)
        else:
            ref, _ = oracle.edt_batch(mask, sampling, features=False)
    compare(mask, sampling, ref, out.get("sqdist"), out.get("dist"), out.get("indices"),
            batch=(mask.ndim == 4))
    return out


# ---------------------------------------------------------------- small cases

SHAPES_2D = [(1, 1), (1, 37), (37, 1), (2, 2), (63, 65), (64, 64), (65, 130), (200, 333),
             (129, 1031), (3, 4100), (700, 7), (130, 257)]


@pytest.mark.parametrize("shape", SHAPES_2D)
def test_random_2d(torch_dev, shape):
    rng = np.random.default_rng([42, 3000, shape[0], shape[1]])
    for p in (0.001, 0.05, 0.5, 0.97):
        mask = (rng.random(shape) >= p).astype(np.uint8)
        if not (mask == 0).any():
            mask.reshape(-1)[rng.integers(0, mask.size)] = 0
        _say(f"2d {shape} p={p}")
        check(torch_dev, mask)                  # (exact integer values)
        check(torch_dev, mask, (2.5, 1.0))      # (integers after scaling by 4)
        check(torch_dev, mask, (1.0, 0.75))     # (by 16)
        check(torch_dev, mask, (1.0, 0.7))      # (no power of two makes 0.49 whole: float64 values)


SHAPES_3D = [(1, 1, 1, 1), (2, 5, 7, 9), (1, 1, 33, 70), (1, 70, 1, 33), (1, 66, 40, 1),
             (3, 40, 33, 65), (1, 130, 65, 100), (2, 9, 520, 17), (1, 5, 17, 600)]


@pytest.mark.parametrize("shape", SHAPES_3D)
def test_random_3d(torch_dev, shape):
    rng = np.random.default_rng([42, 3001, *shape])
    for p in (0.002, 0.1, 0.9):
        mask = (rng.random(shape) >= p).astype(np.uint8)
        for b in range(shape[0]):
            if not (mask[b] == 0).any():
                mask[b].reshape(-1)[0] = 0
        _say(f"3d {shape} p={p}")
        check(torch_dev, mask)
        check(torch_dev, mask, (2.5, 1.0, 1.0))
        check(torch_dev, mask, (1.0, 2.0, 0.5))
        check(torch_dev, mask, (1.3, 1.0, 0.7))   # (float64 values)


@pytest.mark.parametrize("name", golden_names())
def test_golden_fixtures(torch_dev, name):
    g = load_golden(name)
    mask = g["mask"]
    if mask.ndim == 3:
        mask = mask[None]
        ref = g["sqdist"][None]
    elif mask.ndim == 2:
        ref = g["sqdist"]
    else:
        pytest.skip("1-D fixture")
    check(torch_dev, mask, g["sampling"], ref=ref)


# ---------------------------------------------------------------- edge cases

def test_edge_cases_2d(torch_dev):
    rng = np.random.default_rng([42, 3002])
    # all background / no background (virtual element at (-1, 0))
    check(torch_dev, np.zeros((70, 90), np.uint8))
    check(torch_dev, np.ones((70, 90), np.uint8))
    check(torch_dev, np.ones((3, 4), np.uint8), (2.0, 1.0))
    # a single background pixel: closed form
    mask = np.ones((300, 500), np.uint8)
    mask[299, 0] = 0
    out = check(torch_dev, mask)
    yy, xx = np.indices(mask.shape)
    np.testing.assert_array_equal(out["sqdist"], (yy - 299) ** 2 + xx ** 2)
    assert (out["indices"] == 299 * 500).all()
    # one full background row: every candidate on every envelope
    mask = np.ones((257, 1500), np.uint8)
    mask[100] = 0
    check(torch_dev, mask)
    # misaligned mask address and widths not a multiple of 4 / 16
    for shape in [(100, 64), (100, 36), (90, 33)]:
        mask = (rng.random(shape) >= 0.05).astype(np.uint8)
        mask[0, 0] = 0
        check(torch_dev, mask, offset=1)
        check(torch_dev, mask, offset=4)
    # longest supported row
    mask = (rng.random((5, 32768)) >= 0.001).astype(np.uint8)
    mask[2, 5] = 0
    check(torch_dev, mask)
    # background only in the last row / first column
    mask = np.ones((1000, 300), np.uint8)
    mask[-1, -1] = 0
    mask[0, 0] = 0
    check(torch_dev, mask)


def test_edge_cases_3d(torch_dev):
    rng = np.random.default_rng([42, 3003])
    mask = (rng.random((3, 20, 30, 40)) >= 0.01).astype(np.uint8)
    mask[1] = 1       # a volume without background inside a batch
    mask[0, 0, 0, 0] = 0
    mask[2, 19, 29, 39] = 0
    check(torch_dev, mask)
    check(torch_dev, mask, (2.5, 1.0, 1.0))
    # longest supported middle line (K=64 column layout) and last line
    mask = (rng.random((1, 3, 1024, 70)) >= 0.002).astype(np.uint8)
    mask[0, 1, 5, 5] = 0
    check(torch_dev, mask)
    mask = (rng.random((1, 2, 3, 16384)) >= 0.001).astype(np.uint8)
    mask[0, 1, 1, 1] = 0
    check(torch_dev, mask)
    # full background plane across axis 1 (all envelopes full)
    mask = np.ones((2, 30, 50, 70), np.uint8)
    mask[:, :, 17, :] = 0
    check(torch_dev, mask)


def test_long_equal_value_envelopes(torch_dev):
    """Lines whose envelope holds every candidate (all F equal) far from the
    background: a full background column or plane makes every axis-1 or
    axis-2 line an envelope of equal parabolas; also mixed with sparse noise,
    and the longest lines along axes 0 and 1 in one volume."""
    rng = np.random.default_rng([42, 3005])
    # full background column x = 0 in every plane: F = x^2 along every axis-1 line
    mask = np.ones((1, 6, 300, 200), np.uint8)
    mask[:, :, :, 0] = 0
    _say("3d column x=0 (1,6,300,200)")
    check(torch_dev, mask)
    # full background plane y = 0: F = y^2 along every axis-0 line
    mask = np.ones((2, 400, 90, 64), np.uint8)
    mask[:, :, 0, :] = 0
    _say("3d plane y=0 (2,400,90,64)")
    check(torch_dev, mask)
    check(torch_dev, mask, (2.5, 1.0, 1.0))
    # the same with sparse noise: some lanes of a wave overflow, others not
    mask = (rng.random((1, 300, 70, 130)) >= 0.0005).astype(np.uint8)
    mask[:, :, 0, :] = 0
    mask[:, :, :, 0] = 0
    _say("3d mixed (1,300,70,130)")
    check(torch_dev, mask)
    check(torch_dev, mask, (2.5, 1.0, 1.0))
    # long lines along axis 0 (2048) and the longest along axis 1 (1024)
    mask = (rng.random((1, 2048, 3, 64)) >= 0.001).astype(np.uint8)
    mask[0, 0, 0, 0] = 0
    _say("3d D=2048")
    check(torch_dev, mask)
    mask = (rng.random((1, 2, 1024, 64)) >= 0.001).astype(np.uint8)
    mask[0, 1, 7, 3] = 0
    _say("3d H=1024")
    check(torch_dev, mask)


def test_many_short_lines(torch_dev):
    """More than 65536 rows of at most 1024 positions in a volume batch: the
    chunk-per-lane row kernel (fewer lines take the one-wave-per-line kernel,
    which the small shapes above exercise), with partial last chunks.  (2-D
    images have at most 65535 rows; their rows over 1024 positions use the
    chunk kernel, see the 4100- and 1031-wide shapes.)"""
    rng = np.random.default_rng([42, 3004])
    for shape in ((1, 300, 230, 70), (2, 260, 130, 20)):
        for p in (0.002, 0.3):
            mask = (rng.random(shape) >= p).astype(np.uint8)
            for b in range(shape[0]):
                mask[b].reshape(-1)[b] = 0
            _say(f"3d {shape} p={p}")
            check(torch_dev, mask)
            check(torch_dev, mask, (2.5, 1.0, 1.0))


def test_background_runs(torch_dev):
    """Whole chunks of background next to foreground: such chunks own
    themselves, and the members they offer to the neighbouring chunks must be
    exactly their positions (a foreground pair just past a background run of
    16 or 32 positions, nearer to the run than to the background after it)."""
    for shape, run in (((1, 2, 3, 70), 64), ((1, 3, 40, 70), 64), ((1, 1, 33, 70), 64)):
        mask = np.zeros(shape, np.uint8)
        mask[..., run:run + 2] = 1
        for samp in (None, (1.0, 2.0, 0.5), (2.5, 1.0, 1.0)):
            check(torch_dev, mask, samp)
    for shape, run in (((3, 4100), 4096), ((5, 200), 192), ((2, 70), 64)):
        mask = np.zeros(shape, np.uint8)
        mask[:, run:run + 2] = 1
        for samp in (None, (1.0, 0.5)):
            check(torch_dev, mask, samp)
    # background columns (the column pass sees whole background chunks)
    mask = np.zeros((1, 2, 70, 40), np.uint8)
    mask[:, :, 64:66, :] = 1
    for samp in (None, (1.0, 0.5, 1.0)):
        check(torch_dev, mask, samp)


def test_value_kinds(torch_dev):
    """The Euclidean passes take exact integer values (every squared spacing a
    whole number after scaling by a power of two, and the largest height
    S * sum s2 * extent^2 below 2^29) or float64 values otherwise; both give
    the oracle's result.  A tall image at unit spacing (integers) and with
    doubled axis-0 spacing (4 x 16384^2 is over the bound: float64), long
    rows, spacings that need a scale of 2^6 or 2^8, one that would need more
    than 2^10 and ones no power of two makes whole (float64).  (16384^2 at
    unit spacing, just under the bound, is one of the full-size tests.)"""
    rng = np.random.default_rng([42, 3011])
    for shape, samp in (((16384, 64), None), ((16384, 64), (2.0, 1.0)), ((64, 16384), (1.0, 1.0)),
                        ((300, 700), (0.125, 1.0)), ((300, 700), (1.0, 1.0 / 1024)),
                        ((300, 700), (1.0, 0.1)), ((300, 700), (3.0, 7.0))):
        mask = (rng.random(shape) >= 0.01).astype(np.uint8)
        mask[0, 0] = 0
        _say(f"value kinds {shape} sampling {samp}")
        check(torch_dev, mask, samp)
    for shape, samp in (((1, 40, 300, 520), (2.5, 1.0, 1.0)), ((1, 40, 300, 520), (0.3, 1.0, 1.0)),
                        ((1, 600, 600, 70), (4.0, 4.0, 1.0)), ((1, 20, 70, 600), (1.0, 1.0, 0.0625))):
        mask = (rng.random(shape) >= 0.003).astype(np.uint8)
        mask[0, 0, 0, 0] = 0
        _say(f"value kinds {shape} sampling {samp}")
        check(torch_dev, mask, samp)


def test_large_objects(torch_dev):
    """Large foreground objects, where whole-line rounds are long: interior
    candidates are dominated only by members many chunks away (the filter's
    far witnesses, the rounds' cascade steps), with runs of columns without
    background.  A 2-D image of large disks, a volume holding a wide
    cylinder (rows of 1200: whole-line rounds; middle axis of 600: chunks of
    64, always whole-line rounds) and a volume whose rows are 128 long
    (whole-line rounds in the 3-D row pass)."""
    rng = np.random.default_rng([42, 3010])
    yy, xx = np.mgrid[0:900, 0:1700]
    disks = np.zeros((900, 1700), bool)
    for cy, cx, r in ((450, 600, 420), (300, 1350, 260), (700, 1250, 180), (120, 150, 90)):
        disks |= (yy - cy) ** 2 + (xx - cx) ** 2 <= r * r
    m = disks.astype(np.uint8)
    m[rng.integers(0, 900, 40), rng.integers(0, 1700, 40)] = 0
    for samp in (None, (2.5, 1.0), (1.0, 0.75), (0.9, 1.1)):
        _say(f"large disks 900 x 1700 sampling {samp}")
        check(torch_dev, m, samp)
    zz, yv, xv = np.mgrid[0:3, 0:600, 0:1200]
    v = ((yv - 300) ** 2 + (xv - 600) ** 2 <= 280 ** 2 - (zz * 60) ** 2).astype(np.uint8)[None]
    v[0, 1, :, 0:300] = 1                                # columns without background
    for samp in (None, (2.5, 1.0, 1.0), (1.3, 0.9, 1.1)):
        _say(f"cylinder 1 x 3 x 600 x 1200 sampling {samp}")
        check(torch_dev, v, samp)
    zz, yv, xv = np.mgrid[0:40, 0:64, 0:128]
    w = ((zz - 20) ** 2 + (yv - 32) ** 2 + (xv - 64) ** 2 <= 60 ** 2).astype(np.uint8)[None]
    w[0, 0, 0, 0] = 0
    for samp in (None, (1.0, 2.0, 0.5)):
        _say(f"ball 1 x 40 x 64 x 128 sampling {samp}")
        check(torch_dev, w, samp)


@pytest.mark.parametrize("name", ["c1", "c3", "c5"])
def test_repeat_is_bit_identical(torch_dev, name):
    """Two calls on the same input, the workspace poisoned differently each
    time, give the same bits (ties resolved the same way every time)."""
    from workloads import make_config
    mask, sampling, _ = make_config(name)
    want = ("sqdist", "dist", "indices") if sampling is None else ("dist", "indices")
    _say(f"repeat {name}")
    a = run_gpu(torch_dev, mask, sampling, want, poison=0xFF)
    b = run_gpu(torch_dev, mask, sampling, want, poison=0x00)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


# ---------------------------------------------------------------- full sizes

# outputs as timed by bench.py for each workload
BENCH_OUTPUTS = {
    "c1": ("sqdist", "dist", "indices"),
    "c2a": ("sqdist", "dist", "indices"),
    "c2b": ("sqdist", "dist", "indices"),
    "c3": ("sqdist", "dist"),
    "c4": ("dist",),
    "c5": ("dist", "indices"),
}


@pytest.mark.parametrize("name", ["c1", "c2a", "c2b", "c4", "c5", "c3"])
def test_full_size_config(torch_dev, name):
    from workloads import make_config
    _say(f"config {name}: generating")
    mask, sampling, meta = make_config(name)
    _say(f"config {name}: GPU + oracle {mask.shape}")
    out = check(torch_dev, mask, sampling, want=BENCH_OUTPUTS[name])
    if name == "c2b":
        r0, c0 = meta["bg"]
        yy, xx = np.indices(mask.shape)
        np.testing.assert_array_equal(out["sqdist"], (yy - r0) ** 2 + (xx - c0) ** 2)
        assert (out["indices"] == r0 * mask.shape[1] + c0).all()
    if name == "c4":
        # the timed call returns distances only; a second call checks sqdist exactly
        check(torch_dev, mask, sampling, want=("sqdist", "indices"))
