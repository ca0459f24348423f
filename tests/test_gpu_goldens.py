"""The hand-derived goldens (tests/golden/*.json) on the GPU, through the C
ABI: the library must reproduce every hand-derived value exactly.

The goldens are small (K = 4, 7, 8 or 9 values, N = 2); the library needs
K % 16 == 0 and N % 8 == 0, so they are embedded in zero-padded shapes that
reach each kernel route.  Zero padding changes no hand-derived value: a
zero column of X is below any tau > 0 and leaves every row maximum as it is,
a zero row of X has scale 0 and all-zero codes, a zero row of W adds 0 to
every sum, and a zero column of W has scale 0 and all-zero codes.
"""
import json
import os

import numpy as np
import pytest
import torch

from tests.layout import unblock_weight
from tests.oracle_pins import tiny_scale_cases

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


def bf16_bits(a):
    """Round-to-nearest-even bf16 bit patterns of float32 values that are
    exact in bf16 (checked)."""
    u = np.asarray(a, np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any(), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def to_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


# shapes (T, K, N) that route the call through each kernel family
HAND_ROUTES = [
    (2, 16, 8),          # activation segments + register-staged matmul
    (2, 4096, 8),        # single decode kernel
    (8, 12288, 8),       # decode kernel, precomputed mode
    (4, 49152, 8),       # decode kernel in K slabs
    (40, 256, 8),        # owned-column detection + streaming 64x64 tile
    (300, 64, 264),      # clearing + atomic detection + large tile
    (300, 24576, 264),   # large tile with K split in two
]


@pytest.mark.parametrize("T,K,N", HAND_ROUTES)
def test_hand_example(mm, T, K, N):
    g = load("hand_2x4x2.json")
    print(f"[case] hand example in {T}x{K}x{N}", flush=True)
    X = np.zeros((T, K), np.float16)
    X[:2, :4] = np.array(g["X"], np.float16)
    W = np.zeros((K, N), np.float16)
    W[:4, :2] = np.array(g["W"], np.float16)
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    Wq, sw = mm.quantize_weight(Wd)
    r = mm.mixed_matmul_debug(Xd, Wq, sw, Wd, g["tau"])
    Yh = mm.mixed_matmul(Xd, Wq, sw, None, g["tau"])          # memory-halved variant
    torch.cuda.synchronize()
    wq = unblock_weight(Wq.cpu().numpy(), K, N)
    assert np.array_equal(wq[:2, :4], np.array(g["Wq_NK"], np.int8)) and not wq[2:].any() \
        and not wq[:, 4:].any(), "Wq"
    assert sw.cpu().tolist()[:2] == g["sw"] and not sw[2:].any(), "s_w"
    o = int(r["count"][0])
    assert o == 1 and r["idx"][:1].cpu().tolist() == g["idx"], "outlier set"
    assert r["sx"].cpu().tolist()[:2] == g["sx"] and not r["sx"][2:].any(), "s_x"
    xq = r["xq"].cpu().numpy()
    assert np.array_equal(xq[:2, :4], np.array(g["Xq"], np.int8)) and not xq[2:].any() \
        and not xq[:, 4:].any(), "Xq"
    acc = r["acc"].cpu().numpy()
    assert np.array_equal(acc[:2, :2], np.array(g["acc"], np.int32)) and not acc[2:].any() \
        and not acc[:, 2:].any(), "acc"
    Y = r["Y"].cpu().numpy().astype(np.float64)
    assert np.array_equal(Y[:2, :2], np.array(g["Y"])), f"Y {Y[:2, :2].tolist()}"
    assert not Y[2:].any() and not Y[:, 2:].any()
    Yh = Yh.cpu().numpy().astype(np.float64)
    assert np.array_equal(Yh[:2, :2], np.array(g["memory_halved"]["Y"])), "Y memory-halved"


@pytest.mark.parametrize("T,K,N", [(2, 16, 8), (2, 4096, 8), (300, 64, 264)])
def test_hand_example_bf16(mm, T, K, N):
    g = load("hand_2x4x2.json")
    print(f"[case] hand example bf16 in {T}x{K}x{N}", flush=True)
    X = np.zeros((T, K), np.float32)
    X[:2, :4] = np.array(g["X"], np.float32)
    W = np.zeros((K, N), np.float32)
    W[:4, :2] = np.array(g["W"], np.float32)
    Xd, Wd = to_bf16(bf16_bits(X)).cuda(), to_bf16(bf16_bits(W)).cuda()
    Wq, sw, _ = mm.quantize_checkpoint(Wd)
    r = mm.mixed_matmul_debug(Xd, Wq, sw, Wd, g["tau"])
    torch.cuda.synchronize()
    assert np.array_equal(r["acc"].cpu().numpy()[:2, :2], np.array(g["acc"], np.int32)), "acc"
    Y = r["Y"].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(Y[:2, :2], np.array(g["bf16"]["Y"])), f"bf16 Y {Y[:2, :2].tolist()}"


@pytest.mark.parametrize("T,K", [(4, 16), (4, 4096), (8, 12288), (40, 256), (300, 64)])
def test_quant_ties(mm, T, K):
    """Ties to even, a zero row and a row of fp16 subnormals, tau = +inf
    (no outlier: the rows are quantized whole)."""
    g = load("quant_ties.json")
    print(f"[case] quantization ties in {T}x{K}", flush=True)
    X = np.zeros((T, K), np.float16)
    for t, c in enumerate(g["cases"]):
        X[t, :len(c["row"])] = np.array(c["row"], np.float16)
    N = 8
    W = np.ones((K, N), np.float16)
    Xd, Wd = torch.from_numpy(X).cuda(), torch.from_numpy(W).cuda()
    Wq, sw = mm.quantize_weight(Wd)
    r = mm.mixed_matmul_debug(Xd, Wq, sw, Wd, float("inf"))
    torch.cuda.synchronize()
    assert int(r["count"][0]) == 0
    xq, sx = r["xq"].cpu().numpy(), r["sx"].cpu().numpy()
    for t, c in enumerate(g["cases"]):
        assert float(sx[t]) == c["s"], f"case {t}: s_x {sx[t]}"
        assert xq[t, :len(c["q"])].tolist() == c["q"], f"case {t}: {xq[t, :len(c['q'])].tolist()}"
    assert not xq[:, 8:].any() and not xq[len(g["cases"]):].any()


@pytest.mark.parametrize("T,K", [(1, 16), (1, 4096), (8, 12288), (40, 256), (300, 64), (20, 49168)])
def test_tiny_scale_bf16_row(mm, T, K):
    """A bf16 activation row whose scale (2^-130) makes the fp32 quotient
    127/s overflow: the codes follow the reciprocal read with an unbounded
    exponent (tests/golden/tiny_scale.json), on every route."""
    row_bits, s_row, q_row, _, _, _ = tiny_scale_cases()
    print(f"[case] tiny-scale bf16 row in {T}x{K}", flush=True)
    X = np.zeros((T, K), np.uint16)
    X[0, :len(row_bits)] = row_bits
    N = 8
    W = np.ones((K, N), np.float32)
    Xd, Wd = to_bf16(X).cuda(), to_bf16(bf16_bits(W)).cuda()
    Wq, sw, _ = mm.quantize_checkpoint(Wd)
    r = mm.mixed_matmul_debug(Xd, Wq, sw, Wd, 6.0)
    torch.cuda.synchronize()
    assert int(r["count"][0]) == 0
    assert float(r["sx"][0]) == s_row, f"s_x {float(r['sx'][0])}"
    xq = r["xq"].cpu().numpy()
    assert xq[0, :len(q_row)].tolist() == q_row, f"codes {xq[0, :len(q_row)].tolist()}"
    assert not xq[0, len(q_row):].any() and not xq[1:].any()
    # every weight is 1.0 (code 127)
    assert np.array_equal(r["acc"].cpu().numpy()[0], np.full(N, 127 * sum(q_row), np.int32))


def test_tiny_scale_checkpoint_columns(mm):
    """fp32 and bf16 checkpoint columns with scales whose fp32 quotient
    127/s overflows (tests/golden/tiny_scale.json)."""
    row_bits, s_row, q_row, col, s_col, q_col = tiny_scale_cases()
    K, N = 16, 8
    W = np.ones((K, N), np.float32)
    W[:, 0] = 0.0
    W[:len(col), 0] = col
    Wq, sw, _ = mm.quantize_checkpoint(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    wq = unblock_weight(Wq.cpu().numpy(), K, N)
    assert float(sw[0]) == s_col and wq[0, :len(q_col)].tolist() == q_col, \
        f"fp32 column {wq[0].tolist()}"
    assert not wq[0, len(q_col):].any() and (wq[1:] == 127).all()
    Wb = np.full((K, N), 0x3F80, np.uint16)          # bf16 1.0
    Wb[:, 0] = 0
    Wb[:len(row_bits), 0] = row_bits
    Wq, sw, _ = mm.quantize_checkpoint(to_bf16(Wb).cuda())
    torch.cuda.synchronize()
    wq = unblock_weight(Wq.cpu().numpy(), K, N)
    assert float(sw[0]) == s_row and wq[0, :len(q_row)].tolist() == q_row, \
        f"bf16 column {wq[0].tolist()}"
    assert (wq[1:] == 127).all()
