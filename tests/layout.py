"""Test-side view of the library's converted weight, as include/int8mm.h
documents it: int8 [N,K] in the panel-blocked layout - rows in panels of
256 (the last one shorter when N % 256 != 0), each panel's K range in
k-tiles of 64 columns (the last one narrower when K % 64 != 0), each
(panel, k-tile) block stored row-major, blocks in k order inside a panel,
panels in row order, no padding.  Written here from that description (it
shares nothing with the library) to compare the GPU's converted weight with
the oracle's [N,K] array."""
import numpy as np

PANEL, KTILE = 256, 64


def unblock_weight(wq_bytes: np.ndarray, K: int, N: int) -> np.ndarray:
    """Converted-weight bytes (N*K of them) -> int8 [N,K]."""
    b = np.asarray(wq_bytes, dtype=np.int8).reshape(-1)
    assert b.size == N * K, f"{b.size} bytes for a [{N},{K}] weight"
    out = np.empty((N, K), dtype=np.int8)
    pos = 0
    for p0 in range(0, N, PANEL):
        rows = min(PANEL, N - p0)
        for k0 in range(0, K, KTILE):
            w = min(KTILE, K - k0)
            out[p0:p0 + rows, k0:k0 + w] = b[pos:pos + rows * w].reshape(rows, w)
            pos += rows * w
    assert pos == N * K
    return out
