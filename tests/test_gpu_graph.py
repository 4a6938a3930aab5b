"""The transforms inside a HIP graph (GPU): EDT 2-D and 3-D, taxicab 3-D, chessboard 2-D.

With outputs and workspace passed in, a call only launches kernels on the
caller's stream (no allocation, no memset, no synchronisation), so a caller
can capture it once and replay it.  Each replay must equal the eager result
bit for bit, also after the input buffer's contents have changed, with eager
work and synchronisations between the replays.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

KINDS = ["edt2d", "edt3d", "taxicab3d", "chessboard2d"]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from exact_euclidean_distance_amd import _lib
    _lib.load()
    return torch, torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("kind", KINDS)
def test_graph_replay(torch_dev, kind):
    torch, dev = torch_dev
    from exact_euclidean_distance_amd import api, chessboard, edt2d, edt3d, taxicab
    rng = np.random.default_rng([42, 6001 + KINDS.index(kind)])
    if kind in ("edt2d", "chessboard2d"):
        shape, sampling = (3, 300, 517), None   # unit spacing: squared distances too
        ws_bytes = api.workspace_size_2d_batched(*shape)
    else:
        shape, sampling = (2, 40, 33, 70), (2.5, 1.0, 1.0)
        ws_bytes = api.workspace_size_3d(*shape)
    hosts = [(rng.random(shape) >= p).astype(np.uint8) for p in (0.01, 0.002, 0.05)]
    hosts[2][1] = 1                      # an image / volume without background
    m = torch.from_numpy(hosts[0]).to(dev)

    def call(**out):
        if kind == "edt2d":
            return edt2d(m, sampling, return_sqdist=True, return_indices=True, **out)
        if kind == "edt3d":
            return edt3d(m, sampling, return_indices=True, **out)
        if kind == "chessboard2d":
            return chessboard(m, return_indices=True, **out)
        return taxicab(m, return_indices=True, **out)

    def fields(r):
        return [t for t in (r.sqdist, r.dist, r.indices) if t is not None]

    # eager references, one per input
    refs = []
    for h in hosts:
        m.copy_(torch.from_numpy(h).to(dev))
        refs.append([t.clone() for t in fields(call())])
    torch.cuda.synchronize()

    r0 = call()
    outs = {"dist": r0.dist, "indices": r0.indices,
            "workspace": api.alloc_workspace(ws_bytes, dev)}
    if r0.sqdist is not None:
        outs["sqdist"] = r0.sqdist
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(**outs)                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    _say(f"graph {kind} {shape}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(**outs)
    torch.cuda.synchronize()

    got = fields(r0)
    for rep, k in enumerate((0, 1, 2, 0, 2)):
        m.copy_(torch.from_numpy(hosts[k]).to(dev))
        for t in got:
            t.fill_(-1)
        torch.cuda.synchronize()
        _say(f"graph {kind}: replay {rep} (input {k})")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, refs[k]):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
