"""Test-side view of the library's converted weight (documented in
include/int8mm.h): int8 [N,K] row-major.  Used to compare the GPU's
converted weight with the oracle's [N,K] array."""
import numpy as np


def unblock_weight(wq_bytes: np.ndarray, K: int, N: int) -> np.ndarray:
    """Converted-weight bytes -> int8 [N,K]."""
    return np.asarray(wq_bytes, dtype=np.int8).reshape(N, K)


def padding_is_zero(wq_bytes: np.ndarray, K: int, N: int) -> bool:
    """The row-major layout has no padding."""
    return np.asarray(wq_bytes).size == N * K
