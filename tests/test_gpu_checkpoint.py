"""Int8 conversion of fp32 and bf16 checkpoint weights on the GPU (through the
C ABI), against the oracle: Wq and s_w bit-exact, the fp16 copy against the
round-to-nearest-even conversion, and the matmul on the converted weight
(with the fp16 copy, and memory-halved without it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.layout import unblock_weight
from tests.test_gpu_parity import check_y, gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


def checkpoint(seed, K, N, wtype):
    """Seeded fp32 weights N(0, 0.02) with a few large entries; for bf16 the
    values are rounded to bf16 first (numpy holds them as uint16 bits)."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.integers(0, K, 8), rng.integers(0, N, 8)] = 0.5
    if wtype == "f32":
        return W, torch.from_numpy(W).cuda()
    bits = torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits, torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def widened(Wn, wtype):
    return Wn if wtype == "f32" else (Wn.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("wtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,K,N", [(37, 64, 48), (300, 1040, 520), (8, 4096, 264),
                                   (257, 2048, 1000)])
def test_checkpoint_conversion(mm, wtype, T, K, N):
    say(f"[case] {wtype} checkpoint T={T} K={K} N={N}")
    Wn, Wd = checkpoint(7000 + K + N, K, N, wtype)
    Wq, sw, W16 = mm.quantize_checkpoint(Wd, fp16_copy=True)
    torch.cuda.synchronize()
    Wq_o, sw_o = oracle.quantize_weight_typed(Wn, wtype)
    assert np.array_equal(unblock_weight(Wq.cpu().numpy(), K, N), Wq_o), "Wq differs"
    assert np.array_equal(sw.cpu().numpy(), sw_o), "s_w differs"
    w16_ref = widened(Wn, wtype).astype(np.float16)
    assert np.array_equal(W16.cpu().numpy().view(np.uint16), w16_ref.view(np.uint16)), \
        "fp16 copy differs"

    X, _ = synth.random_case(7100 + T + K, T, K, 8, n_dims=3)
    Xd = gpu(X)
    for halved in (False, True):
        w16 = None if halved else W16
        Y = mm.mixed_matmul(Xd, Wq, sw, w16, 6.0)
        torch.cuda.synchronize()
        ref = oracle.mixed_matmul(X, Wq_o, sw_o, None if halved else w16_ref, 6.0)
        rel = check_y(Y.cpu().numpy(), ref["Y"], f"{wtype} checkpoint matmul halved={halved}")
        say(f"[case] {wtype} T={T} K={K} N={N} halved={halved}: ok, o={ref['o']}, rel {rel:.2e}")


def test_fp16_checkpoint_copy(mm):
    """An fp16 checkpoint through the typed entry point: the same conversion
    as int8_quantize_weight, and the copy equals the input."""
    X, W = synth.random_case(7200, 16, 272, 136, n_dims=2)
    Wd = gpu(W)
    Wq, sw, W16 = mm.quantize_checkpoint(Wd, fp16_copy=True)
    Wq2, sw2 = mm.quantize_weight(Wd)
    torch.cuda.synchronize()
    assert torch.equal(Wq, Wq2) and torch.equal(sw, sw2)
    assert torch.equal(W16.view(torch.int16), Wd.view(torch.int16))
