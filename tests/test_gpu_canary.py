"""Out-of-bounds writes: every buffer the library writes (Y, the workspace,
the debug outputs, the converted weight and its scales) sits between two
4 KB guards filled with a canary byte, and after the call both guards must
still hold it.  Each kernel route is covered once or more: the single-kernel
decode path, its precomputed mode and its K slabs, the few-row activation
pass, the owned-column detection, the row quantizers (cached, register and
persistent forms), every matmul kernel including the K split (all tiles
split, and whole tiles plus split ones), the memory-halved variant with its
recovered-rows region and with more outliers than that region holds, the
bf16 variant, the two-step entry points and the allocation-free one.

The workspace is checked at the size the size query returns and at the
smallest size the library accepts (found by bisection over calls), where the
optional regions (recovered rows, K split, K slabs) are off.  At the queried
size Y must be the same bits as a call with unguarded buffers (same layout,
same kernels); at the smallest size, where a route may change, it must meet
the parity tests' bar against that call."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


class Guarded:
    """A tensor of `shape` and `dtype` inside a canary-filled byte buffer."""

    def __init__(self, shape, dtype):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), CANARY, dtype=torch.uint8,
                              device="cuda")
        self.t = self.buf[GUARD:GUARD + self.nbytes].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.buf[:GUARD].cpu().numpy()
        tail = self.buf[GUARD + self.nbytes:].cpu().numpy()
        for name, g in (("before", head), ("after", tail)):
            bad = np.flatnonzero(g != CANARY)
            assert bad.size == 0, (f"{what}: {bad.size} guard bytes overwritten {name} the buffer "
                                   f"({self.nbytes} bytes), first at guard offset {bad[0]}")


def say(msg):
    print(msg, flush=True)


def inputs(mm, T, K, N, n_dims, bf16=False, seed=0):
    X, W = synth.random_case(60_000 + seed, T, K, N, n_dims=n_dims)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    Wq, sw = mm.quantize_weight(Wd)
    if bf16:
        Xd, Wd = Xd.to(torch.bfloat16), Wd.to(torch.bfloat16)
    return Xd, Wd, Wq, sw


def min_workspace(mm, X, Wq, sw, W16, N, fn):
    """Smallest workspace size the entry point accepts (bisection; calls
    below it are refused on the host before any launch)."""
    T, K = X.shape
    hi = mm.workspace_size(T, K, N)
    ws = torch.empty(hi, dtype=torch.uint8, device="cuda")
    Y = torch.empty((T, N), dtype=X.dtype, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def ok(n):
        st = fn(ctypes.c_void_p(X.data_ptr()), T, K, ctypes.c_void_p(Wq.data_ptr()),
                ctypes.c_void_p(sw.data_ptr()),
                None if W16 is None else ctypes.c_void_p(W16.data_ptr()), N, 6.0,
                ctypes.c_void_p(Y.data_ptr()), ctypes.c_void_p(ws.data_ptr()), n, stream)
        assert st in (mm.OK, mm.E_WORKSPACE), mm.status_string(st)
        return st == mm.OK

    lo = 0
    assert ok(hi)
    while lo + 1 < hi:   # ok(hi) holds, ok(lo) does not (lo = 0 is refused)
        mid = (lo + hi) // 2
        if ok(mid):
            hi = mid
        else:
            lo = mid
    torch.cuda.synchronize()
    return hi


ROUTES = [
    # (label, T, K, N, outlier dims): one line per kernel route
    ("decode fused K=8192", 8, 8192, 1040, 3),
    ("decode fused T=1", 1, 4096, 520, 2),
    ("decode fused, half last block", 8, 8192, 28680, 3),
    ("decode precomputed", 4, 12288, 520, 3),
    ("decode K slabs", 8, 49152, 264, 3),
    ("few rows, seg pass", 16, 12288, 520, 3),
    ("few rows, ragged K", 12, 1008, 264, 2),
    ("owned detection, stream 64x64", 64, 2048, 264, 4),
    ("owned detection, stream 128x128", 100, 1024, 520, 4),
    ("owned detection, register-staged 64x128", 40, 1040, 264, 3),
    ("owned detection, cached quantizer 12", 40, 20000, 264, 3),
    ("owned detection, compacted quantizer", 24, 65536, 264, 3),
    ("256x128 stream tile", 200, 1024, 520, 4),
    ("stream 128x128, K split in 8", 72, 49152, 264, 3),
    ("stream 64x64, K split, finishing kernel", 40, 12288, 1032, 3),
    ("stream 256x128, K split", 200, 8192, 1032, 3),
    ("stream 128x128, K split in 2", 128, 12288, 1040, 4),
    ("big tile, register quantizer K<=4096", 300, 1024, 520, 5),
    ("big tile, all tiles split in K", 300, 8192, 520, 5),
    ("register quantizer K<=12288", 140, 12288, 264, 3),
    ("register quantizer K<=16384", 140, 16384, 264, 3),
    ("register quantizer K<=24576", 140, 24576, 264, 3),
    ("register quantizer K<=32768", 140, 32768, 264, 3),
    ("whole + split tiles", 512, 8192, 33024, 4),
    ("persistent row quantizer", 200, 36880, 264, 6),
    ("two-row register quantizer past 2048 rows", 2056, 32784, 264, 4),
    ("compacted quantizer, K > 49152", 140, 49168, 264, 3),
    ("register-staged 128x128x64", 140, 1040, 264, 3),
    ("many outliers", 300, 2048, 264, 600),
]

_cached = {}


def cached_inputs(mm, T, K, N, nd):
    """Inputs of the last route asked for (both variants of a route run
    back to back)."""
    key = (T, K, N, nd)
    if key not in _cached:
        _cached.clear()
        torch.cuda.empty_cache()
        _cached[key] = inputs(mm, T, K, N, nd, seed=T + K)
    return _cached[key]


def close(Y, ref, what):
    """Same output to the parity tests' bar (another kernel route may round
    its outlier sums in another order)."""
    yg, yr = Y.float().cpu().numpy(), ref.float().cpu().numpy()
    scale = max(float(np.abs(yr).max()), 1e-30)
    assert float(np.abs(yg - yr).max()) <= 1e-3 * scale, f"{what}: Y differs beyond 1e-3 max|Y|"
    same = float((Y.view(torch.int16) == ref.view(torch.int16)).float().mean())
    assert same >= 0.99, f"{what}: only {same:.4f} of outputs bit-identical"


@pytest.mark.parametrize("label,T,K,N,nd", ROUTES, ids=[r[0] for r in ROUTES])
@pytest.mark.parametrize("halved", [False, True], ids=["w16", "halved"])
def test_matmul_writes_stay_in_bounds(mm, label, T, K, N, nd, halved):
    say(f"[case] canary {label}: T={T} K={K} N={N} dims={nd} halved={halved}")
    X, W, Wq, sw = cached_inputs(mm, T, K, N, nd)
    W16 = None if halved else W
    ref = mm.mixed_matmul(X, Wq, sw, W16, 6.0).clone()
    sizes = {"query": mm.workspace_size(T, K, N),
             "minimum": min_workspace(mm, X, Wq, sw, W16, N, mm.lib().int8_mixed_matmul)}
    # only the single-kernel decode path reserves nothing beyond the fixed regions
    fused = T <= 16 and K in (4096, 8192) and T * K <= 65536
    assert (sizes["minimum"] == sizes["query"]) == fused, sizes
    for which, nbytes in sizes.items():
        ws = Guarded((nbytes,), torch.uint8)
        Y = Guarded((T, N), torch.float16)
        mm.mixed_matmul(X, Wq, sw, W16, 6.0, workspace=ws.t, out=Y.t)
        ws.check(f"{label} workspace ({which} size, {nbytes} bytes)")
        Y.check(f"{label} Y ({which} workspace)")
        if which == "query":   # the plain call's own layout: the same kernels
            assert torch.equal(Y.t.view(torch.int16), ref.view(torch.int16)), \
                f"{label}: Y differs from the plain call"
        else:
            close(Y.t, ref, f"{label} (minimum workspace)")
    say(f"[case] canary {label}: ok, workspace {sizes}")


@pytest.mark.parametrize("T,K,N,nd", [(8, 8192, 1040, 3), (4, 12288, 520, 2), (300, 1024, 520, 5),
                                      (64, 2048, 264, 4)])
def test_debug_outputs_stay_in_bounds(mm, T, K, N, nd):
    say(f"[case] canary debug {T}x{K}x{N}")
    X, W, Wq, sw = inputs(mm, T, K, N, nd, seed=7 * T)
    ref = mm.mixed_matmul_debug(X, Wq, sw, W, 6.0)
    g = {"Y": Guarded((T, N), torch.float16), "count": Guarded((4,), torch.int32),
         "idx": Guarded((K,), torch.int32), "xq": Guarded((T, K), torch.int8),
         "sx": Guarded((T,), torch.float32), "acc": Guarded((T, N), torch.int32)}
    g["count"].t.zero_()
    g["idx"].t.zero_()
    ws = Guarded((mm.workspace_size(T, K, N),), torch.uint8)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = mm.lib().int8_mixed_matmul_debug(
        p(X), T, K, p(Wq), p(sw), p(W), N, 6.0, p(g["Y"].t), p(ws.t), ws.nbytes,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), p(g["count"].t),
        p(g["idx"].t), p(g["xq"].t), p(g["sx"].t), p(g["acc"].t))
    assert st == mm.OK, mm.status_string(st)
    ws.check("debug workspace")
    for name, b in g.items():
        b.check(f"debug {name}")
    o = int(ref["count"][0])
    assert int(g["count"].t[0]) == o
    assert torch.equal(g["idx"].t[:o], ref["idx"][:o])
    for name in ("xq", "sx", "acc"):
        assert torch.equal(g[name].t, ref[name]), f"debug {name} differs"
    assert torch.equal(g["Y"].t.view(torch.int16), ref["Y"].view(torch.int16))


@pytest.mark.parametrize("T,K,N,nd", [(8, 8192, 1040, 3), (300, 8192, 520, 5), (16, 12288, 520, 3)])
def test_bf16_writes_stay_in_bounds(mm, T, K, N, nd):
    say(f"[case] canary bf16 {T}x{K}x{N}")
    X, W, Wq, sw = inputs(mm, T, K, N, nd, bf16=True, seed=3 * T)
    ref = mm.mixed_matmul(X, Wq, sw, W, 6.0).clone()
    ws = Guarded((mm.workspace_size(T, K, N),), torch.uint8)
    Y = Guarded((T, N), torch.bfloat16)
    mm.mixed_matmul(X, Wq, sw, W, 6.0, workspace=ws.t, out=Y.t)
    ws.check("bf16 workspace")
    Y.check("bf16 Y")
    assert torch.equal(Y.t.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T,K,N,nd", [(4, 12288, 520, 3), (300, 1024, 520, 4), (140, 1040, 264, 3)])
def test_two_step_writes_stay_in_bounds(mm, T, K, N, nd):
    say(f"[case] canary two-step {T}x{K}x{N}")
    X, W, Wq, sw = inputs(mm, T, K, N, nd, seed=11 * T)
    ref = mm.mixed_matmul(X, Wq, sw, W, 6.0).clone()
    ws = Guarded((mm.workspace_size(T, K, N),), torch.uint8)
    Y = Guarded((T, N), torch.float16)
    mm.quantize_activations(X, N, 6.0, ws.t)
    ws.check("workspace after the activation steps")
    mm.matmul_prepared(ws.t, T, K, Wq, sw, W, out=Y.t)
    ws.check("workspace after the matmul steps")
    Y.check("two-step Y")
    assert torch.equal(Y.t.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T,K,N,nd", [(8, 8192, 1040, 3), (300, 1024, 520, 4)])
def test_noalloc_output_stays_in_bounds(mm, T, K, N, nd):
    say(f"[case] canary allocation-free {T}x{K}x{N}")
    X, W, Wq, sw = inputs(mm, T, K, N, nd, seed=13 * T)
    ref = mm.mixed_matmul(X, Wq, sw, W, 6.0).clone()
    Y = Guarded((T, N), torch.float16)
    mm.mixed_matmul_noalloc(X, Wq, sw, W, 6.0, out=Y.t)
    Y.check("allocation-free Y")
    assert torch.equal(Y.t.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("K,N", [(1008, 264), (12288, 520), (4096, 1048)])
@pytest.mark.parametrize("wtype", [torch.float16, torch.bfloat16, torch.float32])
def test_weight_conversion_stays_in_bounds(mm, K, N, wtype):
    say(f"[case] canary weight conversion {K}x{N} {wtype}")
    _, W = synth.random_case(61_000 + K, 1, K, N)
    W = torch.from_numpy(W).cuda().to(wtype)
    Wq0, sw0, W160 = mm.quantize_checkpoint(W, fp16_copy=True)
    Wq = Guarded((mm.weight_bytes(K, N),), torch.int8)
    sw = Guarded((N,), torch.float32)
    W16 = Guarded((K, N), torch.float16)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    code = {torch.float16: mm.WEIGHT_F16, torch.bfloat16: mm.WEIGHT_BF16,
            torch.float32: mm.WEIGHT_F32}[wtype]
    st = mm.lib().int8_quantize_weight_typed(
        p(W), code, K, N, p(Wq.t), p(sw.t), p(W16.t),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mm.OK, mm.status_string(st)
    for name, b in (("Wq", Wq), ("sw", sw), ("W16", W16)):
        b.check(f"weight conversion {name}")
    assert torch.equal(Wq.t, Wq0) and torch.equal(sw.t, sw0)
    assert torch.equal(W16.t.view(torch.int16), W160.view(torch.int16))
