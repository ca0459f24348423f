"""The test-side view of the converted weight (tests/layout.py) against the
element formula include/int8mm.h gives for the panel-blocked layout, on
shapes with partial panels and ragged k-tiles (CPU only)."""
import numpy as np
import pytest

from tests.layout import unblock_weight


def header_offset(n, k, N, K):
    # byte of element (n, k): p0*K + k0*rows + (n - p0)*w + (k - k0)
    p0 = n - n % 256
    rows = min(256, N - p0)
    k0 = k - k % 64
    w = min(64, K - k0)
    return p0 * K + k0 * rows + (n - p0) * w + (k - k0)


@pytest.mark.parametrize("N,K", [(8, 16), (256, 64), (264, 80), (520, 144), (16, 1024), (776, 208)])
def test_unblock_matches_header_formula(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    ref = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    blob = np.zeros(N * K, dtype=np.int8)
    seen = np.zeros(N * K, dtype=bool)
    for n in range(N):
        for k in range(K):
            off = header_offset(n, k, N, K)
            assert not seen[off]
            seen[off] = True
            blob[off] = ref[n, k]
    assert seen.all()                       # a bijection onto N*K bytes, no padding
    assert np.array_equal(unblock_weight(blob, K, N), ref)
    # 16 consecutive rows of one full k-tile are one contiguous kilobyte
    if N >= 16 and K >= 64:
        offs = sorted(header_offset(n, k, N, K) for n in range(16) for k in range(64))
        assert offs == list(range(offs[0], offs[0] + 1024))
