"""The C ABI on the CPU: the library loads, exports every function that
include/int8mm.h declares, and validates arguments on the host before any
HIP call (fake, never-dereferenced device addresses are enough for that)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8mm.h")


@pytest.fixture(scope="module")
def mm():
    import int8_mixed_precision_amd as mm
    return mm


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_lists_entry_points():
    names = header_functions()
    assert "int8_mixed_matmul" in names and "int8_quantize_weight" in names
    assert len(names) == 12, names


def test_exports_every_declared_symbol(mm):
    lib = mm.lib()
    for name in header_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert sorted(mm.EXPORTS) == header_functions()


def test_status_strings(mm):
    for s in range(8):
        assert mm.status_string(s)
    assert mm.status_string(99) == "unknown status"
    assert mm.status_string(0) == "ok"


def test_workspace_size(mm):
    small = mm.workspace_size(16, 64, 48)
    big = mm.workspace_size(2048, 12288, 49152)
    # Xq (T*K bytes), the worst-case gathered outlier columns (2*T*K) and
    # min(K, 512) recovered 16-bit outlier rows of N values (memory-halved
    # variant), plus alignment padding
    rec = 2 * 512 * 49152
    # the matmul's K split adds 2 x 256 KB of partial sums and a counter per
    # split 256 x 256 tile (without a device the size query assumes 256 CUs)
    split = 2 * 65536 * 4 + 4
    assert 3 * 2048 * 12288 + rec <= big < 3 * 2048 * 12288 + rec + (1 << 20)
    assert 0 < small < big
    assert mm.workspace_size(16, 64, 8) < small    # fewer recovered-row columns
    # 384 tiles: 256 whole tiles and 128 split ones (2 rounds become 1.5)
    down = mm.workspace_size(2048, 49152, 12288)
    base = 3 * 2048 * 49152 + 2 * 512 * 12288
    assert base + 128 * split <= down < base + 128 * split + (1 << 20)
    # past 256 rows from K = 8192: T=512, N=36864 gives 288 tiles, 32 split
    t512 = mm.workspace_size(512, 12288, 36864)
    base = 3 * 512 * 12288 + 2 * 512 * 36864
    assert base + 32 * split <= t512 < base + 32 * split + (1 << 20)
    assert mm.workspace_size(256, 12288, 36864) < 3 * 256 * 12288 + 2 * 512 * 36864 + (1 << 20)
    t4096 = mm.workspace_size(4096, 49152, 12288)                         # 3 full rounds
    assert t4096 < 3 * 4096 * 49152 + 2 * 512 * 12288 + (1 << 20)
    # fewer than two whole rounds: no split (T=512, N=32768: 256 tiles)
    assert mm.workspace_size(512, 12288, 32768) < 3 * 512 * 12288 + 2 * 512 * 32768 + (1 << 20)
    # up to 256 rows, streaming tiles that fill at most half of the 256 CUs
    # (a quarter of the 512 slots for 64 x 64) split K into
    # S = min(slots / tiles, K / 2048, 8) slabs, each tile holding S blocks
    # of int32 partial sums of its size
    for T, K, N, tiles, bm, bn, s in ((256, 12288, 12288, 96, 256, 128, 2),
                                      (160, 12288, 4096, 32, 256, 128, 6),
                                      (128, 12288, 12288, 96, 128, 128, 2),
                                      (64, 49152, 4096, 64, 64, 64, 8)):
        base = 3 * T * K + 2 * 512 * N
        part = tiles * s * bm * bn * 4
        assert base + part <= mm.workspace_size(T, K, N) < base + part + (1 << 20), (T, K, N)
    # more than half of the CUs (T=256, N=36864 above; T=128, N=36864 here): no split
    assert mm.workspace_size(128, 12288, 36864) < 3 * 128 * 12288 + 2 * 512 * 36864 + (1 << 20)
    # decode shapes run as one kernel and need only the fixed regions
    assert mm.workspace_size(8, 8192, 28672) < 3 * 8 * 8192 + (1 << 16)
    # few rows with a long K: S = ceil(48 / 16) + 3 = 6 slabs of int32
    # partial sums [S][T][N] in place of the recovered rows
    fixed = 3 * 8 * 49152 + 4 * 49152 + 49152 // 4    # + idx, flags and prefixes
    dec_down = mm.workspace_size(8, 49152, 12288)
    assert fixed + 6 * 8 * 12288 * 4 <= dec_down < fixed + 6 * 8 * 12288 * 4 + (1 << 16)
    # T = 16 (8 chunks per slab) takes the slabs from K = 32768 on: S = 4 + 3;
    # below that the matmul kernels run and the recovered rows are reserved
    fixed16 = 3 * 16 * 32768 + 4 * 32768 + 32768 // 4
    ws16 = mm.workspace_size(16, 32768, 264)
    assert fixed16 + 7 * 16 * 264 * 4 <= ws16 < fixed16 + 7 * 16 * 264 * 4 + (1 << 16)
    assert mm.workspace_size(16, 12288, 1000) >= 3 * 16 * 12288 + 2 * 512 * 1000
    # T = 8, K = 24576: 16 chunks per slab, S = 2 + 3
    assert mm.workspace_size(8, 24576, 264) >= 3 * 8 * 24576 + 5 * 8 * 264 * 4
    # T * K <= 128 KB (precomputed mode without slabs) and K not a multiple of
    # 1024 keep the matmul's regions
    assert mm.workspace_size(16, 8192, 1000) >= 3 * 16 * 8192 + 2 * 512 * 1000
    assert mm.workspace_size(8, 49168, 1000) >= 3 * 8 * 49168 + 2 * 512 * 1000
    with pytest.raises(mm.Int8mmError) as e:
        mm.workspace_size(16, 60, 48)
    assert e.value.status == mm.E_SHAPE


FAKE = 1 << 40   # 16-byte aligned, never dereferenced by a validation failure


def call_mm(lib, X=FAKE, T=16, K=64, Wq=FAKE, sw=FAKE, W16=FAKE, N=48, tau=6.0, Y=FAKE,
            ws=FAKE, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return lib.int8_mixed_matmul(vp(X) if X else None, T, K, vp(Wq) if Wq else None,
                                 vp(sw) if sw else None, vp(W16) if W16 else None, N, tau,
                                 vp(Y) if Y else None, vp(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=0), 1), (dict(Wq=0), 1), (dict(sw=0), 1), (dict(Y=0), 1), (dict(ws=0), 1),
    (dict(T=0), 2), (dict(K=0), 2), (dict(N=0), 2), (dict(T=-3), 2),
    (dict(K=72), 2),                      # K % 16 != 0
    (dict(N=44), 2),                      # N % 8 != 0
    (dict(K=133136 + 16), 2),             # int32 accumulator bound
    (dict(T=1 << 24), 2),                 # launch-grid bound
    (dict(tau=float("nan")), 3), (dict(tau=-1.0), 3), (dict(tau=-1e-30), 3),
    (dict(X=FAKE + 8), 4), (dict(Wq=FAKE + 1), 4), (dict(Y=FAKE + 2), 4), (dict(W16=FAKE + 4), 4),
    (dict(ws_bytes=100), 5),
])
def test_matmul_validation(mm, kw, status):
    assert call_mm(mm.lib(), **kw) == status


def test_weight_bytes(mm):
    assert mm.weight_bytes(64, 48) == 48 * 64
    assert mm.weight_bytes(80, 200) == 200 * 80
    assert mm.weight_bytes(12288, 49152) == 12288 * 49152
    with pytest.raises(mm.Int8mmError):
        mm.weight_bytes(60, 48)


def test_largest_k_accepted_by_shape_check(mm):
    assert mm.workspace_size(1, 133136, 8) > 0


def test_tau_infinity_is_valid_input(mm):
    # +inf passes validation: the failure reported here is the workspace size
    assert call_mm(mm.lib(), tau=math.inf, ws_bytes=1) == mm.E_WORKSPACE
    assert call_mm(mm.lib(), tau=0.0, ws_bytes=1) == mm.E_WORKSPACE


def test_quantize_weight_validation(mm):
    lib, vp = mm.lib(), ctypes.c_void_p
    assert lib.int8_quantize_weight(None, 64, 48, vp(FAKE), vp(FAKE), None) == mm.E_NULL
    assert lib.int8_quantize_weight(vp(FAKE), 60, 48, vp(FAKE), vp(FAKE), None) == mm.E_SHAPE
    assert lib.int8_quantize_weight(vp(FAKE), 64, 47, vp(FAKE), vp(FAKE), None) == mm.E_SHAPE
    assert lib.int8_quantize_weight(vp(FAKE), 64, 48, vp(FAKE + 3), vp(FAKE), None) == mm.E_ALIGN


def test_quantize_weight_typed_validation(mm):
    lib, vp = mm.lib(), ctypes.c_void_p
    q = lib.int8_quantize_weight_typed
    assert q(None, mm.WEIGHT_F32, 64, 48, vp(FAKE), vp(FAKE), None, None) == mm.E_NULL
    assert q(vp(FAKE), mm.WEIGHT_BF16, 60, 48, vp(FAKE), vp(FAKE), None, None) == mm.E_SHAPE
    assert q(vp(FAKE), 3, 64, 48, vp(FAKE), vp(FAKE), None, None) == mm.E_UNSUPPORTED
    assert q(vp(FAKE), -1, 64, 48, vp(FAKE), vp(FAKE), None, None) == mm.E_UNSUPPORTED
    assert q(vp(FAKE), mm.WEIGHT_F32, 64, 48, vp(FAKE), vp(FAKE), vp(FAKE + 2), None) == mm.E_ALIGN


def test_staged_entry_points_validation(mm):
    lib, vp = mm.lib(), ctypes.c_void_p
    assert lib.int8mm_quantize_activations(None, 16, 64, 48, 6.0, vp(FAKE), 1 << 30, None) == 1
    assert lib.int8mm_quantize_activations(vp(FAKE), 16, 64, 48, float("nan"), vp(FAKE),
                                           1 << 30, None) == 3
    assert lib.int8mm_quantize_activations(vp(FAKE), 16, 64, 48, 6.0, vp(FAKE), 10, None) == 5
    assert lib.int8mm_matmul_prepared(vp(FAKE), 1 << 30, 16, 64, vp(FAKE), vp(FAKE),
                                      vp(FAKE + 2), 48, vp(FAKE), None) == mm.E_ALIGN
    assert lib.int8mm_matmul_prepared(None, 1 << 30, 16, 64, vp(FAKE), vp(FAKE), None, 48,
                                      vp(FAKE), None) == mm.E_NULL
    assert lib.int8mm_matmul_prepared(vp(FAKE), 10, 16, 64, vp(FAKE), vp(FAKE), vp(FAKE), 48,
                                      vp(FAKE), None) == mm.E_WORKSPACE
    assert lib.int8_mixed_matmul_debug(vp(FAKE), 16, 64, vp(FAKE), vp(FAKE), vp(FAKE), 48, 6.0,
                                       vp(FAKE), vp(FAKE), 1 << 30, None, vp(FAKE + 4), None,
                                       None, None, None) == mm.E_ALIGN


def test_binding_rejects_cpu_tensors(mm):
    import torch
    X = torch.zeros(16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        mm.quantize_weight(X)
    Wq = torch.zeros(64 * 48, dtype=torch.int8)
    sw = torch.ones(48, dtype=torch.float32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    for call in (lambda: mm.mixed_matmul(X, Wq, sw, None, 6.0),
                 lambda: mm.quantize_activations(X, 48, 6.0, ws),
                 lambda: mm.matmul_prepared(ws, 16, 64, Wq, sw, None),
                 lambda: mm.quantize_checkpoint(torch.zeros(64, 48))):
        with pytest.raises(ValueError):
            call()
    with pytest.raises(TypeError):
        mm.matmul_prepared(None, 16, 64, Wq, sw, None)


def test_noalloc_validation(mm):
    """The allocation-free entry point checks its arguments and the scratch
    size before it touches a device."""
    lib, vp = mm.lib(), ctypes.c_void_p
    f = lib.int8_mixed_matmul_noalloc
    ok = dict(X=vp(FAKE), T=16, K=64, Wq=vp(FAKE), sw=vp(FAKE), W16=None, N=48, tau=6.0, Y=vp(FAKE))

    def call(**kw):
        a = {**ok, **kw}
        return f(a["X"], a["T"], a["K"], a["Wq"], a["sw"], a["W16"], a["N"], a["tau"], a["Y"], None)

    assert call(X=None) == mm.E_NULL and call(Y=None) == mm.E_NULL
    assert call(K=72) == mm.E_SHAPE and call(T=0) == mm.E_SHAPE
    assert call(tau=float("nan")) == mm.E_TAU
    assert call(Wq=vp(FAKE + 1)) == mm.E_ALIGN and call(W16=vp(FAKE + 8)) == mm.E_ALIGN
    # about 3*T*K bytes of fixed workspace against the 128 MiB scratch:
    # T=2048, K=12288 (75.5 MB) fits, T=4096, K=12288 (151 MB) does not
    assert call(T=4096, K=12288, N=49152) == mm.E_WORKSPACE
    assert call(T=2048, K=49152, N=12288) == mm.E_WORKSPACE
