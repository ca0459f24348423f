"""The plain entry point captured in a HIP graph (as the decode benchmark
launches it): every replay, with eager work and synchronizations in
between, must give exactly the eager result."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


@pytest.mark.parametrize("T,K,N", [(8, 8192, 1040), (300, 1024, 520), (300, 24576, 520),
                                   (16, 8192, 1040), (8, 49152, 264), (4, 12288, 520),
                                   (200, 1024, 520), (64, 2048, 264),
                                   (8, 8192, 28672), (96, 12288, 520),
                                   (48, 12288, 2048), (160, 8192, 520)])   # last three: K split
def test_graph_replays_match_eager(mm, T, K, N):
    print(f"[case] graph replay {T}x{K}x{N}", flush=True)
    X, W = synth.random_case(40_000 + T, T, K, N, n_dims=3)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    Wq, sw = mm.quantize_weight(Wd)
    ws = mm.new_workspace(T, K, N)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
    eager = mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0, workspace=ws, out=Y)
    for rep in range(4):
        Y.fill_(0)
        # eager work between replays, on the same workspace-free path
        other = mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager), f"replay {rep} differs"
        assert torch.equal(other, eager)


def test_concurrent_streams_match_eager(mm):
    """Calls on two streams at once, each with its own workspace and output
    (different shapes and routes: the single decode kernel, the K-slab
    decode, the streaming tile, the large-tile kernel with K split): the
    library keeps no state between calls, so every result must equal the
    eager single-stream one."""
    print("[case] concurrent streams", flush=True)
    cases = []
    for i, (T, K, N) in enumerate([(8, 8192, 1040), (8, 49152, 264), (64, 2048, 264),
                                   (300, 24576, 520), (4, 8192, 28680), (128, 12288, 1040)]):
        X, W = synth.random_case(41_000 + i, T, K, N, n_dims=3)
        Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
        Wq, sw = mm.quantize_weight(Wd)
        eager = mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0).clone()
        cases.append((Xd, Wq, sw, Wd, eager, mm.new_workspace(T, K, N),
                      torch.empty((T, N), dtype=torch.float16, device="cuda")))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for c in cases:
            c[6].fill_(0)
        torch.cuda.synchronize()
        for i, (Xd, Wq, sw, Wd, eager, ws, Y) in enumerate(cases):
            with torch.cuda.stream(streams[i % 2]):
                for _ in range(3):
                    mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0, workspace=ws, out=Y)
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            assert torch.equal(c[6], c[4]), f"case {i} differs on pass {rep}"

