"""Seeded synthetic inputs for the LLM.int8() mixed-precision matmul.

A module of its own: both the CPU oracle and the GPU path take their inputs
from here, and it holds none of the method's arithmetic (no thresholding, no
quantization, no products).  Values are drawn on the host by the counter-based
SplitMix64 generator in ``synth.c`` and rounded to fp16 once.

Workloads stand in for the 70B-175B-class feed-forward and attention
projections that the LLM.int8() abstract names (no trained weights or
activations are available): Gaussian or Laplace activations with a few hidden
dimensions scaled up to act as the emergent outlier features the method
isolates, and Gaussian weights.

Streams of one seed: 1 = X base, 2 = W, 3 = choice of outlier dims,
4 = per-dim factor f = 10 + 50u, 5 = row subsets (offset j*T for dim j),
6 = tiny-config outlier magnitudes and signs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

STREAM_X, STREAM_W, STREAM_DIMS, STREAM_FACTORS, STREAM_ROWS, STREAM_TINY = 1, 2, 3, 4, 5, 6


def build() -> str:
    """Compile ``libsynth.so`` with gcc (plain C, no intrinsics)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                           "-ffp-contract=off", "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, u64, dbl, vp, c_int = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_double,
                                ctypes.c_void_p, ctypes.c_int)
    lib.synth_uniform.argtypes = [u64, u64, u64]
    lib.synth_uniform.restype = dbl
    lib.synth_normal.argtypes = [u64, u64, u64]
    lib.synth_normal.restype = dbl
    lib.synth_f64_to_f16.argtypes = [dbl]
    lib.synth_f64_to_f16.restype = ctypes.c_uint16
    lib.synth_matrix_f16.argtypes = [vp, i64, i64, u64, u64, c_int, dbl, c_int, vp, vp, vp, c_int]
    lib.synth_matrix_f16.restype = c_int
    lib.synth_set_columns_f16.argtypes = [vp, i64, i64, u64, u64, c_int, vp, dbl, dbl]
    lib.synth_set_columns_f16.restype = c_int
    lib.synth_choose.argtypes = [u64, u64, i64, i64, u64, vp]
    lib.synth_choose.restype = c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def uniform(seed: int, stream: int, i: int) -> float:
    return _load().synth_uniform(seed, stream, i)


def f64_to_f16_bits(x: float) -> int:
    return int(_load().synth_f64_to_f16(float(x)))


def matrix_f16(rows: int, cols: int, seed: int, stream: int, dist: str, param: float,
               dims=None, factors=None, rowsel=None, threads: int = 0) -> np.ndarray:
    """fp16 matrix [rows, cols]; ``dist`` is "normal" (param = sigma) or
    "laplace" (param = scale b).  Column dims[j] is multiplied by factors[j]
    in the rows where rowsel[j] is true (all rows when rowsel is None)."""
    out = np.empty((rows, cols), dtype=np.float16)
    nd = 0 if dims is None else len(dims)
    d = f = r = None
    if nd:
        d = np.ascontiguousarray(dims, dtype=np.int64)
        f = np.ascontiguousarray(factors, dtype=np.float64)
        if rowsel is not None:
            r = np.ascontiguousarray(rowsel, dtype=np.uint8).reshape(nd, rows)
    rc = _load().synth_matrix_f16(_ptr(out), rows, cols, seed, stream,
                                  0 if dist == "normal" else 1, param, nd,
                                  _ptr(d), _ptr(f), _ptr(r), threads)
    if rc:
        raise ValueError(f"synth_matrix_f16 failed ({rc})")
    return out


def choose(seed: int, stream: int, pool: int, count: int, offset: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    if _load().synth_choose(seed, stream, pool, count, offset, _ptr(out)):
        raise ValueError("synth_choose failed")
    return out


def set_columns(X: np.ndarray, seed: int, stream: int, cols, lo: float, hi: float) -> None:
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if _load().synth_set_columns_f16(_ptr(X), X.shape[0], X.shape[1], seed, stream,
                                     len(c), _ptr(c), lo, hi):
        raise ValueError("synth_set_columns_f16 failed")


@dataclass
class Workload:
    name: str
    T: int
    K: int
    N: int
    tau: float
    seed: int
    x_dist: str = "normal"
    x_param: float = 1.0
    w_sigma: float = 0.02
    n_dims: int = 0               # planted outlier dims
    factor: tuple | float = (10.0, 60.0)   # range for f = 10 + 50u, or a fixed factor
    row_frac: float = 1.0         # fraction of rows in which a planted dim is scaled
    tiny_cols: tuple = ()         # columns replaced by +-(8 + 12u) in every row
    notes: str = ""
    extra: dict = field(default_factory=dict)


# Small case the oracle finishes instantly, then the projection shapes.
WORKLOADS = {
    "tiny": Workload("tiny", 16, 64, 48, 6.0, 1000, w_sigma=0.02, tiny_cols=(3, 17),
                     notes="columns 3 and 17 set to +-(8 + 12u) in every row"),
    "dec": Workload("dec", 8, 8192, 28672, 6.0, 1001, w_sigma=0.02, n_dims=6,
                    notes="decode-shaped FFN up-projection, W pre-quantized"),
    "up": Workload("up", 2048, 12288, 49152, 6.0, 1002, w_sigma=0.015, n_dims=7, row_frac=0.25,
                   notes="prefill 175B-class FFN up-projection"),
    "down": Workload("down", 2048, 49152, 12288, 6.0, 1003, x_dist="laplace", x_param=0.5,
                     w_sigma=0.01, n_dims=24, factor=20.0,
                     notes="prefill FFN down-projection, Laplace activations"),
}

SWEEP_PROJ = {"qkv": (12288, 36864), "out": (12288, 12288), "up": (12288, 49152),
              "down": (49152, 12288)}
SWEEP_DIMS = (0, 8, 64, 256)
for _p, (_k, _n) in enumerate(SWEEP_PROJ.values()):
    for _d, _nd in enumerate(SWEEP_DIMS):
        _name = f"sweep_{list(SWEEP_PROJ)[_p]}_{_nd}"
        WORKLOADS[_name] = Workload(_name, 4096, _k, _n, 6.0, 2000 + 4 * _p + _d,
                                    w_sigma=0.015, n_dims=_nd,
                                    notes="175B-class layer at T=4096, outlier-count sweep")


def planted(w: Workload, T: int | None = None, K: int | None = None):
    """(dims, factors, rowsel) of the planted outlier features."""
    T = w.T if T is None else T
    K = w.K if K is None else K
    if w.n_dims == 0:
        return np.zeros(0, np.int64), np.zeros(0), None
    dims = choose(w.seed, STREAM_DIMS, K, w.n_dims)
    if isinstance(w.factor, tuple):
        lo, hi = w.factor
        factors = np.array([lo + (hi - lo) * uniform(w.seed, STREAM_FACTORS, j)
                            for j in range(w.n_dims)])
    else:
        factors = np.full(w.n_dims, float(w.factor))
    rowsel = None
    if w.row_frac < 1.0:
        nsel = int(round(T * w.row_frac))
        rowsel = np.zeros((w.n_dims, T), np.uint8)
        for j in range(w.n_dims):
            rowsel[j, choose(w.seed, STREAM_ROWS, T, nsel, offset=j * T)] = 1
    return dims, factors, rowsel


def make_x(w: Workload, T: int | None = None, K: int | None = None, threads: int = 0) -> np.ndarray:
    """Activation X fp16 [T, K] of the workload (shape overridable for tests)."""
    T = w.T if T is None else T
    K = w.K if K is None else K
    dims, factors, rowsel = planted(w, T, K)
    X = matrix_f16(T, K, w.seed, STREAM_X, w.x_dist, w.x_param, dims, factors, rowsel, threads)
    if w.tiny_cols:
        set_columns(X, w.seed, STREAM_TINY, w.tiny_cols, 8.0, 20.0)
    return X


def make_w(w: Workload, K: int | None = None, N: int | None = None, threads: int = 0) -> np.ndarray:
    """Weight W fp16 [K, N] ~ N(0, w_sigma)."""
    K = w.K if K is None else K
    N = w.N if N is None else N
    return matrix_f16(K, N, w.seed, STREAM_W, "normal", w.w_sigma, threads=threads)


def random_case(seed: int, T: int, K: int, N: int, x_sigma: float = 1.0, w_sigma: float = 0.05,
                n_dims: int = 0, factor: float = 15.0, x_dist: str = "normal"):
    """Free-form seeded (X, W) pair for tests: n_dims planted columns scaled
    by `factor` in every row."""
    dims = choose(seed, STREAM_DIMS, K, n_dims) if n_dims else None
    facs = np.full(n_dims, factor) if n_dims else None
    X = matrix_f16(T, K, seed, STREAM_X, x_dist, x_sigma, dims, facs)
    W = matrix_f16(K, N, seed, STREAM_W, "normal", w_sigma)
    return X, W
