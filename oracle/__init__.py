"""ORACLE - TEST INFRASTRUCTURE ONLY.

ctypes wrapper around ``oracle.c``, the plain CPU implementation of the
LLM.int8() mixed-precision matmul (LLM.int8() abstract, taxoreview.com page,
second paragraph; "LLM.int8(): A Procedure for Int8 Matrix Multiplication in
Transformer Language Models", section "The LLM.int8() Methodology").

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

Every function is pinned by ``tests/test_oracle_*.py`` against values that
do not come from the oracle itself: hand-derived examples under
``tests/golden/``, closed forms, invariants and numpy library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle: plain C, -O2, no intrinsics, no BLAS, no
    contraction of multiply-adds, IEEE fp32/fp64 (no fast-math)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float16:
        raise TypeError(f"expected float16, got {a.dtype}")
    return a


HTYPES = {"f16": 0, "bf16": 1}


def _h16(a, htype: str) -> np.ndarray:
    """A 16-bit array of the given type: float16 for "f16", uint16 bit
    patterns for "bf16" (numpy has no bfloat16)."""
    if htype == "f16":
        return _f16(a)
    a = np.ascontiguousarray(a)
    if htype != "bf16" or a.dtype != np.uint16:
        raise TypeError(f"expected {htype} data (uint16 bits for bf16), got {a.dtype}")
    return a


class Oracle:
    """One loaded build of ``oracle.c`` (the default one, or a variant a test
    compiled from an edited copy)."""

    def __init__(self, path: str = _LIB_PATH):
        if path == _LIB_PATH and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        i64, vp, c_int, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_decode.restype = ctypes.c_double
        lib.oracle_f16_encode.argtypes = [ctypes.c_double]
        lib.oracle_f16_encode.restype = ctypes.c_uint16
        lib.oracle_max_threads.restype = c_int
        lib.oracle_quantize_weight.argtypes = [vp, i64, i64, vp, vp, c_int]
        lib.oracle_quantize_weight_typed.argtypes = [vp, c_int, i64, i64, vp, vp, c_int]
        lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_decode.restype = ctypes.c_float
        lib.oracle_detect.argtypes = [vp, i64, i64, f32, vp, c_int]
        lib.oracle_compact.argtypes = [vp, i64, vp]
        lib.oracle_compact.restype = i64
        lib.oracle_quantize_rows.argtypes = [vp, i64, i64, vp, vp, i64, vp, vp, c_int]
        lib.oracle_int8_gemm.argtypes = [vp, i64, i64, vp, i64, vp, c_int]
        lib.oracle_int8_gemm.restype = i64
        lib.oracle_output.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp,
                                      vp, c_int, c_int]
        lib.oracle_dequant_weight_h.argtypes = [ctypes.c_int8, f32, c_int]
        lib.oracle_dequant_weight_h.restype = ctypes.c_uint16
        lib.oracle_bf16_encode.argtypes = [ctypes.c_double]
        lib.oracle_bf16_encode.restype = ctypes.c_uint16
        lib.oracle_dequant_weight.argtypes = [ctypes.c_int8, f32]
        lib.oracle_dequant_weight.restype = ctypes.c_uint16
        lib.oracle_mixed_matmul.argtypes = [vp, i64, i64, vp, vp, vp, i64, f32, vp, i64,
                                            vp, vp, vp, vp, vp, vp, vp, c_int, c_int]
        lib.oracle_mixed_matmul.restype = i64
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()

    def f16_decode(self, bits: int) -> float:
        return self.lib.oracle_f16_decode(bits)

    def f16_encode(self, x: float) -> int:
        return int(self.lib.oracle_f16_encode(float(x)))

    def quantize_weight(self, W: np.ndarray, threads: int = 0):
        """W fp16 [K,N] -> (Wq int8 [N,K], s_w float32 [N])."""
        W = _f16(W)
        K, N = W.shape
        Wq = np.empty((N, K), np.int8)
        sw = np.empty(N, np.float32)
        self.lib.oracle_quantize_weight(_p(W), K, N, _p(Wq), _p(sw), threads)
        return Wq, sw

    WEIGHT_TYPES = {"f16": 0, "bf16": 1, "f32": 2}

    def quantize_weight_typed(self, W: np.ndarray, wtype: str, threads: int = 0):
        """A 16- or 32-bit checkpoint weight [K,N] -> (Wq int8 [N,K], s_w [N]).
        wtype "f16" (float16 array), "bf16" (uint16 array of bfloat16 bits)
        or "f32" (float32 array)."""
        dt = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}[wtype]
        W = np.ascontiguousarray(W)
        if W.dtype != dt:
            raise TypeError(f"{wtype} weight must be {np.dtype(dt)}, got {W.dtype}")
        K, N = W.shape
        Wq = np.empty((N, K), np.int8)
        sw = np.empty(N, np.float32)
        self.lib.oracle_quantize_weight_typed(_p(W), self.WEIGHT_TYPES[wtype], K, N, _p(Wq),
                                              _p(sw), threads)
        return Wq, sw

    def bf16_decode(self, bits: int) -> float:
        return float(self.lib.oracle_bf16_decode(bits))

    def bf16_encode(self, x: float) -> int:
        return int(self.lib.oracle_bf16_encode(float(x)))

    def detect(self, X: np.ndarray, tau: float, htype: str = "f16") -> np.ndarray:
        """Outlier flags uint8 [K]."""
        X = _h16(X, htype)
        T, K = X.shape
        flag = np.empty(K, np.uint8)
        self.lib.oracle_detect(_p(X), T, K, tau, _p(flag), HTYPES[htype])
        return flag

    def compact(self, flag: np.ndarray) -> np.ndarray:
        flag = np.ascontiguousarray(flag, np.uint8)
        idx = np.empty(len(flag), np.int32)
        o = self.lib.oracle_compact(_p(flag), len(flag), _p(idx))
        return idx[:o].copy()

    def quantize_rows(self, X: np.ndarray, flag: np.ndarray, rows=None, htype: str = "f16"):
        """(Xq int8 [M,K], s_x float32 [M]) for the listed rows (all when None)."""
        X = _h16(X, htype)
        T, K = X.shape
        flag = np.ascontiguousarray(flag, np.uint8)
        r = None if rows is None else np.ascontiguousarray(rows, np.int64)
        M = T if r is None else len(r)
        Xq = np.empty((M, K), np.int8)
        sx = np.empty(M, np.float32)
        self.lib.oracle_quantize_rows(_p(X), T, K, _p(flag), _p(r), M, _p(Xq), _p(sx),
                                      HTYPES[htype])
        return Xq, sx

    def int8_gemm(self, Xq: np.ndarray, Wq: np.ndarray, threads: int = 0):
        """acc int32 [M,N] = Xq [M,K] . Wq[N,K]^T; raises if an entry overflows."""
        Xq = np.ascontiguousarray(Xq, np.int8)
        Wq = np.ascontiguousarray(Wq, np.int8)
        M, K = Xq.shape
        N = Wq.shape[0]
        acc = np.empty((M, N), np.int32)
        bad = self.lib.oracle_int8_gemm(_p(Xq), M, K, _p(Wq), N, _p(acc), threads)
        if bad:
            raise OverflowError(f"{bad} accumulators do not fit int32")
        return acc

    def dequant_weight(self, q: int, sw: float, htype: str = "f16") -> int:
        """16-bit bits of the weight value recovered from Int8 code q and
        column scale sw (memory-halved variant)."""
        return int(self.lib.oracle_dequant_weight_h(int(q), float(sw), HTYPES[htype]))

    def output(self, acc, sx, sw, X, W16, idx, rows=None, threads: int = 0, Wq=None,
               htype: str = "f16"):
        """(Y [M,N] (float16, or uint16 bf16 bits), Y64 float64 [M,N] before
        the final rounding).  W16 None: memory-halved variant, outlier rows
        recovered from Wq."""
        X = _h16(X, htype)
        K = X.shape[1]
        if W16 is not None:
            W16 = _h16(W16, htype)
            N = W16.shape[1]
        else:
            Wq = np.ascontiguousarray(Wq, np.int8)
            N = Wq.shape[0]
        acc = np.ascontiguousarray(acc, np.int32)
        M = acc.shape[0]
        idx = np.ascontiguousarray(idx, np.int32)
        r = None if rows is None else np.ascontiguousarray(rows, np.int64)
        Y = np.empty((M, N), np.float16 if htype == "f16" else np.uint16)
        Y64 = np.empty((M, N), np.float64)
        self.lib.oracle_output(_p(acc), _p(np.ascontiguousarray(sx, np.float32)),
                               _p(np.ascontiguousarray(sw, np.float32)), _p(X), _p(W16),
                               _p(Wq if W16 is None else None), _p(r), M, K, N, _p(idx), len(idx),
                               _p(Y), _p(Y64), threads, HTYPES[htype])
        return Y, Y64

    def mixed_matmul(self, X, Wq, sw, W16, tau: float, rows=None, threads: int = 0,
                     htype: str = "f16"):
        """The whole method.  Returns a dict with flag, idx, o, xq, sx, acc,
        Y, Y64 (xq/sx/acc/Y/Y64 for the sampled rows when `rows` is given).
        W16 None: the memory-halved variant.  htype "bf16": X, W16 and Y are
        bfloat16 (uint16 bit arrays)."""
        X = _h16(X, htype)
        T, K = X.shape
        Wq = np.ascontiguousarray(Wq, np.int8)
        if W16 is not None:
            W16 = _h16(W16, htype)
        N = Wq.shape[0]
        sw = np.ascontiguousarray(sw, np.float32)
        r = None if rows is None else np.ascontiguousarray(rows, np.int64)
        M = T if r is None else len(r)
        flag = np.empty(K, np.uint8)
        idx = np.empty(K, np.int32)
        xq = np.empty((M, K), np.int8)
        sx = np.empty(M, np.float32)
        acc = np.empty((M, N), np.int32)
        Y = np.empty((M, N), np.float16 if htype == "f16" else np.uint16)
        Y64 = np.empty((M, N), np.float64)
        o = self.lib.oracle_mixed_matmul(_p(X), T, K, _p(Wq), _p(sw), _p(W16), N, tau, _p(r), M,
                                         _p(flag), _p(idx), _p(xq), _p(sx), _p(acc), _p(Y),
                                         _p(Y64), threads, HTYPES[htype])
        if o == -2:
            raise OverflowError("int32 accumulator overflow")
        if o < 0:
            raise MemoryError("oracle allocation failed")
        return {"flag": flag, "idx": idx[:o].copy(), "o": int(o), "xq": xq, "sx": sx,
                "acc": acc, "Y": Y, "Y64": Y64}


_default = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` as committed."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # oracle.mixed_matmul(...) etc. forward to the default build.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
