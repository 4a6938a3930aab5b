"""GPU test of the Python binding's `stream=` argument: a transform enqueued
on a side stream while the current stream allocates and overwrites memory.
The binding allocates its workspace and outputs on the stream the kernels run
on, so the caching allocator cannot hand that memory to the current stream's
work before the kernels are done; the results must equal an eager call's."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def test_side_stream_results_equal_eager():
    import torch
    from exact_euclidean_distance_amd import chessboard, edt2d, edt3d
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    rng = np.random.default_rng([42, 7200])
    m2 = torch.from_numpy((rng.random((6, 1500, 1700)) >= 0.001).astype(np.uint8)).to(dev)
    m3 = torch.from_numpy((rng.random((2, 96, 200, 160)) >= 0.002).astype(np.uint8)).to(dev)
    ref2 = edt2d(m2, return_sqdist=True, return_indices=True)
    ref3 = edt3d(m3, (2.5, 1.0, 1.0), return_indices=True)
    refc = chessboard(m2, return_indices=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        _say(f"side-stream transforms, round {rep}")
        side.wait_stream(torch.cuda.current_stream())
        r2 = edt2d(m2, return_sqdist=True, return_indices=True, stream=side)
        r3 = edt3d(m3, (2.5, 1.0, 1.0), return_indices=True, stream=side)
        rc = chessboard(m2, return_indices=True, stream=side)
        # meanwhile the current stream allocates and fills memory of the
        # same sizes (what a freed workspace would be handed out as)
        junk = [torch.full((int(m2.numel()) * 3,), 0x7F, dtype=torch.uint8, device=dev)
                for _ in range(4)]
        for j in junk:
            j.add_(1)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for a, b in ((r2.sqdist, ref2.sqdist), (r2.dist, ref2.dist), (r2.indices, ref2.indices),
                     (r3.dist, ref3.dist), (r3.indices, ref3.indices), (rc.dist, refc.dist),
                     (rc.indices, refc.indices)):
            assert torch.equal(a, b), "side-stream result differs from the eager one"
        del junk
