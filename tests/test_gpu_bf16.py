"""The bf16 variant of the path (X, W16 and Y bfloat16) on the GPU through the
C ABI, against the oracle's bf16 branch.

Bit-exact: the outlier set, Xq, s_x, Wq, s_w and the int32 accumulators.
Output tolerance, derived the same way as the fp16 path's: the GPU adds in
fp32 and rounds once to bf16, the oracle adds exactly and rounds once, so
the two differ by at most one bf16 step of the value, which is at most
2^-7 * max|Y| (bf16 keeps 8 significant bits); and since the two sums agree
to fp32 precision, the roundings agree for almost every element (a
truncating or wrongly rounding kernel would miss about half of them)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.layout import unblock_weight
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu

BF16_RTOL = 2.0 ** -7


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


def to_bf16_bits(a16):
    """fp16 array -> the nearest bf16 values as uint16 bit patterns (input
    generation only: the seeded fp16 data rounded to bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(a16)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_y_bf16(y_bits, ref_bits, what):
    yg, yr = bf16_values(y_bits), bf16_values(ref_bits)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite output"
    scale = np.abs(yr).max()
    err = np.abs(yg - yr).max()
    assert err <= BF16_RTOL * scale, f"{what}: max|dY| = {err:.3e} > 2^-7 * {scale:.3e}"
    same = np.mean(y_bits == ref_bits)
    assert same >= 0.99, f"{what}: only {same:.4f} of the outputs round like the oracle's"
    return err / max(scale, 1e-30), same


def run_bf16(mm, name, X16, W16, tau, halved=False, big=None, rows=None):
    """X16, W16: seeded fp16 data, rounded to bf16 here; `big` plants one
    activation value beyond the fp16 range (bf16 has fp32's exponent);
    `rows`: check acc and Y on these rows only (full-size workloads)."""
    Xb, Wb = to_bf16_bits(X16), to_bf16_bits(W16)
    if big is not None:
        Xb[big] = 0x47C3   # 99840.0, beyond fp16's 65504
    T, K = Xb.shape
    N = Wb.shape[1]
    say(f"[case] bf16 {name}: T={T} K={K} N={N} tau={tau} halved={halved}")
    Xd, Wd = bf16_dev(Xb), bf16_dev(Wb)
    Wq, sw, _ = mm.quantize_checkpoint(Wd)
    r = mm.mixed_matmul_debug(Xd, Wq, sw, None if halved else Wd, tau)
    Yp = mm.mixed_matmul(Xd, Wq, sw, None if halved else Wd, tau)
    torch.cuda.synchronize()
    Wq_o, sw_o = oracle.quantize_weight_typed(Wb, "bf16")
    assert np.array_equal(unblock_weight(Wq.cpu().numpy(), K, N), Wq_o), f"{name}: Wq"
    assert np.array_equal(sw.cpu().numpy(), sw_o), f"{name}: s_w"
    sel = np.arange(T) if rows is None else np.asarray(rows)
    ref = oracle.mixed_matmul(Xb, Wq_o, sw_o, None if halved else Wb, tau, htype="bf16",
                              rows=None if rows is None else sel)
    o = int(r["count"][0])
    assert o == ref["o"] and np.array_equal(r["idx"][:o].cpu().numpy(), ref["idx"]), \
        f"{name}: outlier set"
    sel_t = torch.from_numpy(sel).cuda()
    pick = lambda t: t.index_select(0, sel_t).cpu()
    assert np.array_equal(pick(r["xq"]).numpy(), ref["xq"]), f"{name}: Xq"
    assert np.array_equal(pick(r["sx"]).numpy(), ref["sx"]), f"{name}: s_x"
    assert np.array_equal(pick(r["acc"]).numpy(), ref["acc"]), f"{name}: acc"
    ybits = pick(r["Y"]).view(torch.int16).numpy().view(np.uint16)
    rel, same = check_y_bf16(ybits, ref["Y"], name)
    check_y_bf16(pick(Yp).view(torch.int16).numpy().view(np.uint16), ref["Y"], name + " (plain)")
    say(f"[case] bf16 {name}: ok, o={o}, rel {rel:.2e}, identical {same:.4f}")
    return r, ref


@pytest.mark.parametrize("T,K,N,nd,tau,halved", [
    (37, 80, 200, 2, 6.0, False), (300, 1040, 520, 3, 6.0, False),       # staged kernels
    (1400, 24576, 8, 5, 6.0, False),                                      # long rows past 128 rows
    (600, 40960, 8, 9, 6.0, False),                                       # persistent long rows
    (257, 2048, 1000, 70, 6.0, False), (513, 128, 264, 2, 6.0, True),    # large-tile kernel
    (1, 4096, 1000, 3, 6.0, False), (8, 8192, 264, 300, 6.0, False),     # decode kernel
    (16, 4096, 520, 5, 6.0, True), (8, 8192, 2056, 6, 6.0, True),
    (70, 1024, 136, 0, 0.0, False), (2, 4096, 136, 0, 0.0, False),       # tau = 0
    (65, 320, 96, 4, float("inf"), False),                               # tau = inf
    (300, 24576, 520, 3, 6.0, True), (300, 8192, 264, 5, 6.0, False),   # K split in two
    (6, 16384, 520, 5, 6.0, False), (8, 12288, 264, 30, 6.0, True),      # decode, precomputed
    (8, 49152, 264, 4, 6.0, True), (16, 32768, 136, 3, 6.0, False),      # decode, K slabs
    (16, 8192, 520, 5, 6.0, False), (50, 1152, 520, 3, 6.0, True),       # streaming matmul
    (80, 12288, 520, 5, 6.0, False), (128, 8192, 1032, 4, 6.0, True),    # streaming, K split
    (48, 8192, 1032, 5, 6.0, False), (24, 12288, 264, 3, 6.0, True),     # 64x64 split, finishing kernel
    (192, 8192, 1032, 4, 6.0, False),                                     # 256x128 split
    (100, 2048, 264, 70, 6.0, False), (200, 2048, 264, 40, 6.0, True),   # outlier W rows through LDS
])
def test_bf16_path(mm, T, K, N, nd, tau, halved):
    X, W = synth.random_case(60_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_bf16(mm, f"{T}x{K}x{N}", X, W, tau, halved=halved)


@pytest.mark.parametrize("T,K,N", [(40, 512, 136), (4, 4096, 264)])
def test_bf16_beyond_fp16_range(mm, T, K, N):
    """An activation of 99840 (not representable in fp16) is an outlier like
    any other and is carried through the 16-bit matmul."""
    X, W = synth.random_case(61_000 + T + K, T, K, N, n_dims=2)
    r, ref = run_bf16(mm, f"beyond fp16 {T}x{K}x{N}", X, W, 6.0, big=(T // 2, 33))
    assert 33 in ref["idx"].tolist()


@pytest.mark.parametrize("name,halved", [("dec", False), ("dec", True), ("up", False)])
def test_bf16_config(mm, name, halved):
    """The decode and prefill up-projection workloads at full size in bf16
    (acc and Y on sampled rows for the prefill one)."""
    from tests.test_gpu_parity import _sample_rows
    w = synth.WORKLOADS[name]
    X, W = synth.make_x(w), synth.make_w(w)
    rows = None if w.T <= 16 else _sample_rows(w.T, synth.planted(w)[2], n=6)
    r, ref = run_bf16(mm, f"{name} (full size)", X, W, w.tau, halved=halved, rows=rows)
    assert set(synth.planted(w)[0].tolist()) <= set(ref["idx"].tolist())
