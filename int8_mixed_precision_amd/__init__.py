"""LLM.int8() mixed-precision matmul for AMD MI355X (gfx950).

Thin ctypes binding over ``libint8mm.so`` (C ABI in ``include/int8mm.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, allocates outputs/workspace with torch and passes
device pointers and the current HIP stream.  There is no CPU fallback: if the
library is missing, importing the binding raises.

The method (LLM.int8() abstract, taxoreview.com page dblp:280/8696, second
paragraph; "LLM.int8(): A Procedure for Int8 Matrix Multiplication in
Transformer Language Models", section "The LLM.int8() Methodology"):
outlier hidden dimensions of X (|x| >= tau in some row) go through a 16-bit
matmul, the rest through an Int8 matmul with one absmax scale per row of X
and per column of W.
"""
from __future__ import annotations

import ctypes
import os

# torch first: it carries the HIP runtime this process uses, and the library
# must bind to that same runtime (same soname) rather than load a second one.
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libint8mm.so")

OK, E_NULL, E_SHAPE, E_TAU, E_ALIGN, E_WORKSPACE, E_UNSUPPORTED, E_HIP = range(8)
WEIGHT_F16, WEIGHT_BF16, WEIGHT_F32 = range(3)
MAX_K = 133136

EXPORTS = [
    "int8mm_status_string",
    "int8_mixed_matmul_workspace_size",
    "int8_quantize_weight_size",
    "int8_quantize_weight",
    "int8_quantize_weight_typed",
    "int8_mixed_matmul",
    "int8_mixed_matmul_debug",
    "int8_mixed_matmul_bf16",
    "int8_mixed_matmul_bf16_debug",
    "int8mm_quantize_activations",
    "int8mm_matmul_prepared",
    "int8_mixed_matmul_noalloc",
]


class Int8mmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run int8_mixed_precision_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, f32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    c_int = ctypes.c_int
    lib.int8mm_status_string.argtypes = [c_int]
    lib.int8mm_status_string.restype = ctypes.c_char_p
    lib.int8_mixed_matmul_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
    lib.int8_quantize_weight_size.argtypes = [i64, i64, ctypes.POINTER(sz)]
    lib.int8_quantize_weight.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.int8_quantize_weight_typed.argtypes = [vp, c_int, i64, i64, vp, vp, vp, vp]
    lib.int8_mixed_matmul.argtypes = [vp, i64, i64, vp, vp, vp, i64, f32, vp, vp, sz, vp]
    lib.int8_mixed_matmul_debug.argtypes = [vp, i64, i64, vp, vp, vp, i64, f32, vp, vp, sz, vp,
                                            vp, vp, vp, vp, vp]
    lib.int8_mixed_matmul_bf16.argtypes = lib.int8_mixed_matmul.argtypes
    lib.int8_mixed_matmul_bf16_debug.argtypes = lib.int8_mixed_matmul_debug.argtypes
    lib.int8mm_quantize_activations.argtypes = [vp, i64, i64, i64, f32, vp, sz, vp]
    lib.int8mm_matmul_prepared.argtypes = [vp, sz, i64, i64, vp, vp, vp, i64, vp, vp]
    lib.int8_mixed_matmul_noalloc.argtypes = [vp, i64, i64, vp, vp, vp, i64, f32, vp, vp]
    for name in EXPORTS[1:]:
        getattr(lib, name).restype = c_int
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    """The loaded C library (for tests that call the ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.int8mm_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Int8mmError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, dtype, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d {dtype} tensor, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _need_ws(ws) -> None:
    """A workspace is a contiguous 1-d uint8 GPU tensor (its size is checked
    by the library against the size query)."""
    _need(ws, torch.uint8, 1, "workspace")


def _need_out(Y, dtype, T: int, N: int) -> None:
    _need(Y, dtype, 2, "out")
    if tuple(Y.shape) != (T, N):
        raise ValueError(f"out must be [{T},{N}], got {tuple(Y.shape)}")


def workspace_size(T: int, K: int, N: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.int8_mixed_matmul_workspace_size(T, K, N, ctypes.byref(out)),
           "int8_mixed_matmul_workspace_size")
    return out.value


def new_workspace(T: int, K: int, N: int, device=None) -> torch.Tensor:
    return torch.empty(workspace_size(T, K, N), dtype=torch.uint8, device=device or "cuda")


def weight_bytes(K: int, N: int) -> int:
    """Bytes of the converted weight (layout in include/int8mm.h)."""
    out = ctypes.c_size_t(0)
    _check(_lib.int8_quantize_weight_size(K, N, ctypes.byref(out)), "int8_quantize_weight_size")
    return out.value


def quantize_weight(W16: torch.Tensor, out: tuple | None = None):
    """W16 fp16 [K,N] -> (Wq int8 [weight_bytes(K,N)], the library's layout
    (the transpose [N,K], panel-blocked as include/int8mm.h describes),
    sw fp32 [N])."""
    _need(W16, torch.float16, 2, "W16")
    K, N = W16.shape
    if out is None:
        Wq = torch.empty(weight_bytes(K, N), dtype=torch.int8, device=W16.device)
        sw = torch.empty(N, dtype=torch.float32, device=W16.device)
    else:
        Wq, sw = out
        _need(Wq, torch.int8, 1, "Wq")
        _need(sw, torch.float32, 1, "sw")
        if Wq.numel() != weight_bytes(K, N) or sw.numel() != N:
            raise ValueError("output buffers have the wrong size")
    _check(_lib.int8_quantize_weight(_ptr(W16), K, N, _ptr(Wq), _ptr(sw), _stream()),
           "int8_quantize_weight")
    return Wq, sw


_WEIGHT_TYPES = {torch.float16: WEIGHT_F16, torch.bfloat16: WEIGHT_BF16,
                 torch.float32: WEIGHT_F32}


def quantize_checkpoint(W: torch.Tensor, fp16_copy: bool = False):
    """A 16- or 32-bit checkpoint weight [K,N] (fp16, bf16 or fp32) ->
    (Wq, sw, W16) with W16 the fp16 copy for the outlier path when
    fp16_copy, else None (for the memory-halved variant)."""
    if not isinstance(W, torch.Tensor) or W.dtype not in _WEIGHT_TYPES:
        raise ValueError("W must be a float16, bfloat16 or float32 tensor")
    _need(W, W.dtype, 2, "W")
    K, N = W.shape
    Wq = torch.empty(weight_bytes(K, N), dtype=torch.int8, device=W.device)
    sw = torch.empty(N, dtype=torch.float32, device=W.device)
    W16 = torch.empty((K, N), dtype=torch.float16, device=W.device) if fp16_copy else None
    _check(_lib.int8_quantize_weight_typed(_ptr(W), _WEIGHT_TYPES[W.dtype], K, N, _ptr(Wq),
                                           _ptr(sw), _ptr(W16), _stream()),
           "int8_quantize_weight_typed")
    return Wq, sw, W16


def _mm_args(X, Wq, sw, W16):
    """Checks the operands; X, W16 and Y share one 16-bit type: float16, or
    bfloat16 for the bf16 variant."""
    if not isinstance(X, torch.Tensor) or X.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("X must be a float16 or bfloat16 tensor")
    _need(X, X.dtype, 2, "X")
    _need(Wq, torch.int8, 1, "Wq")
    _need(sw, torch.float32, 1, "sw")
    T, K = X.shape
    N = sw.shape[0]
    if Wq.numel() != weight_bytes(K, N):
        raise ValueError(f"Wq has {Wq.numel()} bytes, a [{K},{N}] weight needs "
                         f"{weight_bytes(K, N)}")
    if W16 is not None:
        _need(W16, X.dtype, 2, "W16")
        if tuple(W16.shape) != (K, N):
            raise ValueError(f"W16 must be [{K},{N}], got {tuple(W16.shape)}")
    return T, K, N


def mixed_matmul(X, Wq, sw, W16, tau: float, workspace=None, out=None) -> torch.Tensor:
    """Y [T,N] = LLM.int8()(X, W, tau), in X's 16-bit type (float16, or
    bfloat16 for the bf16 variant).  W16 None: memory-halved variant."""
    T, K, N = _mm_args(X, Wq, sw, W16)
    if workspace is None:
        workspace = new_workspace(T, K, N, X.device)
    _need_ws(workspace)
    Y = out if out is not None else torch.empty((T, N), dtype=X.dtype, device=X.device)
    _need_out(Y, X.dtype, T, N)
    fn, name = ((_lib.int8_mixed_matmul_bf16, "int8_mixed_matmul_bf16")
                if X.dtype == torch.bfloat16 else (_lib.int8_mixed_matmul, "int8_mixed_matmul"))
    _check(fn(_ptr(X), T, K, _ptr(Wq), _ptr(sw), _ptr(W16), N, float(tau), _ptr(Y),
              _ptr(workspace), workspace.numel(), _stream()), name)
    return Y


def mixed_matmul_debug(X, Wq, sw, W16, tau: float, workspace=None) -> dict:
    """Y plus the intermediates count, idx, xq, sx and acc (see the header)."""
    T, K, N = _mm_args(X, Wq, sw, W16)
    dev = X.device
    if workspace is None:
        workspace = new_workspace(T, K, N, dev)
    _need_ws(workspace)
    r = {"Y": torch.empty((T, N), dtype=X.dtype, device=dev),
         "count": torch.zeros(4, dtype=torch.int32, device=dev),
         "idx": torch.zeros(K, dtype=torch.int32, device=dev),
         "xq": torch.empty((T, K), dtype=torch.int8, device=dev),
         "sx": torch.empty(T, dtype=torch.float32, device=dev),
         "acc": torch.empty((T, N), dtype=torch.int32, device=dev)}
    fn, name = ((_lib.int8_mixed_matmul_bf16_debug, "int8_mixed_matmul_bf16_debug")
                if X.dtype == torch.bfloat16
                else (_lib.int8_mixed_matmul_debug, "int8_mixed_matmul_debug"))
    _check(fn(_ptr(X), T, K, _ptr(Wq), _ptr(sw), _ptr(W16), N, float(tau), _ptr(r["Y"]),
              _ptr(workspace), workspace.numel(), _stream(), _ptr(r["count"]), _ptr(r["idx"]),
              _ptr(r["xq"]), _ptr(r["sx"]), _ptr(r["acc"])), name)
    return r


def quantize_activations(X, N: int, tau: float, workspace) -> None:
    """Activation-side steps into `workspace` (see int8mm_quantize_activations)."""
    _need(X, torch.float16, 2, "X")
    _need_ws(workspace)
    T, K = X.shape
    _check(_lib.int8mm_quantize_activations(_ptr(X), T, K, N, float(tau), _ptr(workspace),
                                            workspace.numel(), _stream()),
           "int8mm_quantize_activations")


def matmul_prepared(workspace, T: int, K: int, Wq, sw, W16, out=None) -> torch.Tensor:
    """Matmul steps on a prepared workspace (see int8mm_matmul_prepared);
    W16 None: memory-halved variant."""
    _need_ws(workspace)
    _need(Wq, torch.int8, 1, "Wq")
    _need(sw, torch.float32, 1, "sw")
    N = sw.shape[0]
    if Wq.numel() != weight_bytes(K, N):
        raise ValueError("Wq does not match K and N")
    if W16 is not None:
        _need(W16, torch.float16, 2, "W16")
        if tuple(W16.shape) != (K, N):
            raise ValueError(f"W16 must be [{K},{N}], got {tuple(W16.shape)}")
    Y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=Wq.device)
    _need_out(Y, torch.float16, T, N)
    _check(_lib.int8mm_matmul_prepared(_ptr(workspace), workspace.numel(), T, K, _ptr(Wq),
                                       _ptr(sw), _ptr(W16), N, _ptr(Y), _stream()),
           "int8mm_matmul_prepared")
    return Y


def mixed_matmul_noalloc(X, Wq, sw, W16, tau: float, out) -> torch.Tensor:
    """int8_mixed_matmul_noalloc: Y into `out` (float16 [T,N]) with the
    library's per-GPU scratch as the workspace (no allocation in the call;
    calls that overlap on one GPU race, see include/int8mm.h)."""
    if not isinstance(X, torch.Tensor) or X.dtype != torch.float16:
        raise ValueError("X must be a float16 tensor")
    T, K, N = _mm_args(X, Wq, sw, W16)
    _need_out(out, torch.float16, T, N)
    _check(_lib.int8_mixed_matmul_noalloc(_ptr(X), T, K, _ptr(Wq), _ptr(sw), _ptr(W16), N,
                                          float(tau), _ptr(out), _stream()),
           "int8_mixed_matmul_noalloc")
    return out
