"""int8_mixed_matmul_noalloc (the entry point for callers that cannot
allocate) through the C ABI, against int8_mixed_matmul with its own
workspace on the same inputs: the same kernels run, so Y must be
bit-identical.  Two calls in a row, the second on a smaller input (the
scratch keeps the first call's contents), for several routes: the single
decode kernel, the K-slab decode, the streaming tile, the large-tile kernel
and the memory-halved variant."""
import ctypes

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


def case(mm, seed, T, K, N, halved=False):
    X, W = synth.random_case(seed, T, K, N, n_dims=3)
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    Wq, sw = mm.quantize_weight(Wd)
    W16 = None if halved else Wd
    ref = mm.mixed_matmul(Xd, Wq, sw, W16, 6.0)
    return Xd, Wq, sw, W16, ref


def call_noalloc(mm, Xd, Wq, sw, W16, out):
    vp = ctypes.c_void_p
    T, K = Xd.shape
    N = sw.shape[0]
    st = mm.lib().int8_mixed_matmul_noalloc(
        vp(Xd.data_ptr()), T, K, vp(Wq.data_ptr()), vp(sw.data_ptr()),
        vp(W16.data_ptr()) if W16 is not None else None, N, ctypes.c_float(6.0),
        vp(out.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
    assert st == mm.OK, mm.status_string(st)


@pytest.mark.parametrize("big,small,halved", [
    ((8, 8192, 1040), (4, 4096, 264), False),        # single decode kernel
    ((8, 8192, 28672), (2, 4096, 36864), True),      # decode kernel at full width, memory-halved
    ((8, 49152, 264), (2, 24576, 136), False),       # decode K slabs
    ((64, 2048, 520), (40, 1024, 264), True),        # streaming tile, memory-halved
    ((128, 12288, 1040), (72, 49152, 264), False),   # streaming tile with K split in 2, then 8
    ((600, 12288, 776), (300, 2048, 520), False),    # large tile (K split), then streaming
    ((2048, 12288, 2048), (520, 4096, 1032), False), # headline T and K, then a ragged tile
])
def test_noalloc_matches_workspace_entry(mm, big, small, halved):
    for i, (T, K, N) in enumerate((big, small)):
        print(f"[case] noalloc call {i}: {T}x{K}x{N} halved={halved}", flush=True)
        Xd, Wq, sw, W16, ref = case(mm, 60_000 + 17 * T + K, T, K, N, halved)
        out = torch.full((T, N), float("nan"), dtype=torch.float16, device="cuda")
        call_noalloc(mm, Xd, Wq, sw, W16, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i} ({T}x{K}x{N}) differs from the workspace entry point"
        # the binding's wrapper, once more on the same scratch
        out2 = mm.mixed_matmul_noalloc(Xd, Wq, sw, W16, 6.0, out=torch.empty_like(out))
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_rejects_shape_beyond_scratch(mm):
    Xd = torch.zeros((4096, 12288), dtype=torch.float16, device="cuda")
    Wq = torch.zeros(12288 * 8, dtype=torch.int8, device="cuda")
    sw = torch.ones(8, dtype=torch.float32, device="cuda")
    out = torch.empty((4096, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(mm.Int8mmError) as e:
        mm.mixed_matmul_noalloc(Xd, Wq, sw, None, 6.0, out=out)
    assert e.value.status == mm.E_WORKSPACE
