"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: the outlier count and index set, Xq, s_x, Wq, s_w and the int32
accumulators.  fp16 output: max|dY| <= 1e-3 * max|Y_oracle| (the output
tolerance of the method's statement; one fp16 ulp at the top binade is
2^-10 < 1e-3 of max|Y|, so independent final roundings fit inside it), and
element by element |dY| <= ulp16 + (o + 8) * 2^-24 * (|y8| + sum_j |x_j w_j|):
both sides round once to fp16 (at most one fp16 ulp apart when their sums
agree), the oracle from the exact sum, the GPU from fp32 arithmetic whose
error is a few fp32 roundings of the dequantized value and one per outlier
product accumulated (the term on the right); and, with at most 1024
outliers, at least 99% of outputs bit-identical: the sums then differ by
about sqrt(o + 6) fp32 roundings (~2e-6 relative at o = 1024), so a
different final rounding needs the exact value that close to an fp16
rounding boundary (2^-11 relative away on average).  With every dimension
an outlier (tau = 0, o = K up to 49152) the fp32 sum of the GPU drifts by
more than that and only the per-element bound applies.

Small shapes are checked element by element everywhere; the full-size
projection workloads are checked in full for every integer tensor the
oracle can produce quickly (outlier set, Xq, s_x, Wq, s_w) and on sampled
rows for acc and Y (the oracle's matmul is the slow part).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.layout import unblock_weight

pytestmark = pytest.mark.gpu

Y_RTOL = 1e-3


@pytest.fixture(scope="module")
def mm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_mixed_precision_amd as mm
    return mm


def say(msg):
    print(msg, flush=True)


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ulp16(v):
    """Spacing of fp16 at |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def term_magnitudes(acc, sx, sw, X, W16, idx):
    """|y8| + sum_j |x_j w_j| per output, in fp64 (X: the rows compared;
    W16 None: recovered weights, bounded by |w^| <= s_w)."""
    y8 = np.abs(acc.astype(np.float64)) * sx.astype(np.float64)[:, None] * \
        sw.astype(np.float64)[None, :] / 16129.0
    if len(idx) == 0:
        return y8
    xa = np.abs(X[:, idx].astype(np.float64))
    if W16 is None:
        return y8 + xa.sum(axis=1)[:, None] * sw.astype(np.float64)[None, :]
    return y8 + xa @ np.abs(W16[idx, :].astype(np.float64))


def check_y(y_gpu, y_ref, what, mag=None, o=0):
    yg = y_gpu.astype(np.float64)
    yr = y_ref.astype(np.float64)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite output"
    scale = np.abs(yr).max()
    err = np.abs(yg - yr).max()
    assert err <= Y_RTOL * scale, f"{what}: max|dY| = {err:.3e} > 1e-3 * {scale:.3e}"
    if mag is not None:
        d = np.abs(yg - yr)
        bound = ulp16(np.maximum(np.abs(yg), np.abs(yr))) + (o + 8) * 2.0 ** -24 * mag
        bad = np.flatnonzero(d > bound)
        assert bad.size == 0, (f"{what}: {bad.size} outputs beyond one fp16 ulp + the fp32 slack, "
                               f"first at {np.unravel_index(bad[0], d.shape)}: "
                               f"{yg.flat[bad[0]]} vs {yr.flat[bad[0]]}")
        same = np.mean(y_gpu.view(np.uint16) == y_ref.view(np.uint16))
        assert o > 1024 or same >= 0.99, f"{what}: only {same:.4f} of outputs bit-identical"
    return err / max(scale, 1e-30)


def run_case(mm, name, X, W, tau, rows=None, plain_too=True, halved=False):
    """halved: the memory-halved variant (no 16-bit weight passed; outlier
    rows recovered from the Int8 weight on both sides)."""
    T, K = X.shape
    N = W.shape[1]
    say(f"[case] {name}: T={T} K={K} N={N} tau={tau}{' (memory-halved)' if halved else ''}")
    Xd, Wd = gpu(X), gpu(W)
    Wq, sw = mm.quantize_weight(Wd)
    W16 = None if halved else Wd
    r = mm.mixed_matmul_debug(Xd, Wq, sw, W16, tau)
    Yp = mm.mixed_matmul(Xd, Wq, sw, W16, tau) if plain_too else None
    torch.cuda.synchronize()
    say(f"[case] {name}: GPU done")

    Wq_o, sw_o = oracle.quantize_weight(W)
    wq_gpu = Wq.cpu().numpy()
    assert np.array_equal(unblock_weight(wq_gpu, K, N), Wq_o), f"{name}: Wq differs"
    assert np.array_equal(sw.cpu().numpy(), sw_o), f"{name}: s_w differs"

    flag = oracle.detect(X, tau)
    idx_o = oracle.compact(flag)
    o = int(r["count"][0].item())
    assert o == len(idx_o), f"{name}: o = {o}, oracle {len(idx_o)}"
    assert np.array_equal(r["idx"][:o].cpu().numpy(), idx_o), f"{name}: outlier set differs"
    xq_o, sx_o = oracle.quantize_rows(X, flag)
    assert np.array_equal(r["sx"].cpu().numpy(), sx_o), f"{name}: s_x differs"
    assert np.array_equal(r["xq"].cpu().numpy(), xq_o), f"{name}: Xq differs"

    sel = np.arange(T) if rows is None else np.asarray(rows)
    ref = oracle.mixed_matmul(X, Wq_o, sw_o, None if halved else W, tau,
                              rows=None if rows is None else sel)
    sel_t = torch.from_numpy(sel).cuda()
    acc = r["acc"].index_select(0, sel_t).cpu().numpy()
    assert np.array_equal(acc, ref["acc"]), f"{name}: acc differs in {np.sum(acc != ref['acc'])}"
    Y = r["Y"].index_select(0, sel_t).cpu().numpy()
    mag = term_magnitudes(ref["acc"], ref["sx"], sw_o, X[sel], None if halved else W, idx_o)
    rel = check_y(Y, ref["Y"], name, mag, o)
    if Yp is not None:
        Yp_s = Yp.index_select(0, sel_t).cpu().numpy()
        if T > 16:
            # same kernels as the debug entry point
            assert np.array_equal(Yp_s.view(np.uint16), Y.view(np.uint16)), f"{name}: plain != debug"
        else:
            check_y(Yp_s, ref["Y"], name + " (plain)", mag, o)
    say(f"[case] {name}: ok, o={o}, rel err {rel:.2e}")
    return r, ref


def test_tiny_config(mm):
    w = synth.WORKLOADS["tiny"]
    X, W = synth.make_x(w), synth.make_w(w)
    r, _ = run_case(mm, "tiny", X, W, w.tau)
    assert r["idx"][:2].cpu().tolist() == [3, 17]


@pytest.mark.parametrize("T,K,N,nd,dist", [
    (1, 16, 8, 0, "normal"), (37, 80, 200, 2, "normal"), (129, 272, 136, 5, "laplace"),
    (300, 1040, 520, 3, "normal"), (17, 4096, 264, 40, "normal"), (260, 528, 1032, 20, "laplace"),
    # shapes on the large-tile kernel (T > 128, K % 64 == 0): one and two
    # k-tiles, ragged T and N against the 256x256 tile, many outliers
    (129, 64, 8, 1, "normal"), (513, 128, 264, 2, "normal"), (300, 1024, 520, 3, "laplace"),
    (257, 2048, 1000, 70, "normal"),
    # K split in two halves (K >= 24576 and few tiles): ragged T and N, and
    # 200 outliers through the second half's epilogue
    (300, 24576, 520, 3, "normal"), (129, 24576, 264, 200, "laplace"),
    # past 256 rows the split starts at K = 8192
    (300, 8192, 520, 3, "normal"), (513, 12288, 264, 70, "laplace"),
    # the mid-size-T tiles (32x128x256, 64x128x256, 64x128x128) with K not a
    # multiple of their k-tile, and T = 130 (K % 64 != 0) on 128x128x64
    (32, 1040, 264, 4, "normal"), (50, 1296, 520, 3, "laplace"), (100, 1104, 392, 5, "normal"),
    (128, 2064, 136, 2, "normal"), (130, 1040, 264, 3, "laplace"),
    # the streaming kernels (K % 128 == 0): 64x64 tiles up to T = 64, 128x128
    # up to 128; one k-tile, fewer k-tiles than ring stages, ragged T and N
    (37, 256, 200, 2, "normal"), (50, 1152, 520, 3, "laplace"), (64, 2048, 136, 1, "normal"),
    (17, 128, 72, 1, "normal"), (100, 1280, 392, 4, "normal"), (128, 4096, 1000, 6, "laplace"),
    (65, 384, 8, 2, "normal"), (100, 2048, 264, 70, "laplace"), (64, 1024, 200, 40, "normal"),
    # 9..16 rows go to the matmul kernels unless K is long
    (16, 8192, 1000, 6, "normal"), (12, 5120, 520, 3, "laplace"), (16, 12288, 264, 20, "normal"),
    # 17..32 rows (detection without the clearing kernel), K past a whole
    # 2048-column segment
    (24, 2064, 136, 3, "normal"), (32, 6144, 264, 9, "laplace"), (19, 4112, 72, 2, "normal"),
    # 129..256 rows on the 256x128 streaming tile (one k-tile; ragged T and
    # N; many outliers through the LDS stage)
    (129, 128, 72, 1, "normal"), (200, 1152, 392, 5, "laplace"), (256, 2048, 264, 80, "normal"),
])
def test_ragged_shapes(mm, T, K, N, nd, dist):
    X, W = synth.random_case(10_000 + T + K + N, T, K, N, n_dims=nd, x_dist=dist)
    run_case(mm, f"ragged {T}x{K}x{N}", X, W, 6.0)


@pytest.mark.parametrize("T,K,nd,dist", [
    # register-resident row quantizer (rows in registers, partial bitmaps of
    # the detection in row groups), one case per row shape, at its longest
    # row or with K % 64 != 0 (byte addressing of the last k-tile), T odd
    # against the rows per workgroup
    (131, 4096, 3, "normal"),     # 2 waves per row, 4 chunks per lane, 2 rows per workgroup
    (200, 8192, 4, "laplace"),    # 4 waves x 4 chunks
    (151, 10000, 5, "normal"),    # 4 waves x 6 chunks, the last k-tile 16 wide
    (130, 16384, 5, "normal"),    # 8 waves x 4 chunks: every word held
    (130, 16400, 5, "normal"),    # 8 waves x 6 chunks, most of the last ones past the row;
                                  # detection blocks of 256 columns, the last one 16 wide
    (133, 30000, 6, "normal"),    # 4 waves x 16 chunks, ragged
    (140, 32768, 9, "laplace"),   # 4 waves x 16 chunks, every word held
    (129, 49152, 40, "laplace"),  # persistent rows of 8 waves x 12 chunks, one row per
                                  # workgroup (grid = T), every word held, many outliers
    (131, 40016, 5, "normal"),    # the same, ragged; detection blocks of 256 columns, the last
                                  # one 80 wide
    (1000, 40016, 9, "laplace"),  # persistent rows, 512 workgroups (rows 2k and 2k+1 paired),
                                  # two rows per workgroup for most, ragged rows and last panel
    (2048, 36864, 30, "normal"),  # persistent rows, four per workgroup, whole k-tiles
    (256, 49152, 12, "laplace"),  # persistent rows, grid = T = 256 with the row pairing
    (2000, 36880, 6, "normal"),   # persistent rows, a partial last round, ragged k-tiles
    (2049, 49152, 8, "normal"),   # past the persistent kernel's row limit: 2 rows per workgroup
    (129, 49168, 7, "normal"),    # past the registers: one bitmap, separate compaction, two-pass rows
    (1100, 12288, 6, "normal"),   # three row groups in the detection
    (1100, 24576, 6, "normal"),   # 8 waves x 6 chunks, three row groups
])
def test_row_quantizer_limits(mm, T, K, nd, dist):
    """The activation pass for more than 128 rows at the row lengths where
    the row quantizer changes form."""
    X, W = synth.random_case(60_000 + K, T, K, 136, n_dims=nd, x_dist=dist)
    run_case(mm, f"row quantizer {T}x{K}x136", X, W, 6.0)


def _row_max_in_outlier_column(T, K, seed):
    """Rows whose largest magnitude below tau sits in a column that another
    row makes an outlier: column 777 holds 7.0 in row 0 (an outlier) and
    5.5 in every other row (above the rest of those rows, |x| < 3), so the
    row scale must skip it; column 40 is >= tau in every row; column 41
    holds exactly the row maximum in a non-outlier column for even rows
    (5.5 again), where the scale is 5.5."""
    rng = np.random.default_rng(seed)
    X = np.clip(rng.standard_normal((T, K)), -2.9, 2.9)
    X[:, 777] = 5.5
    X[0, 777] = 7.0
    X[:, 40] = -6.5
    X[::2, 41] = -5.5
    return X.astype(np.float16)


@pytest.mark.parametrize("T,K", [(700, 49152), (1400, 24576), (300, 20480), (200, 8192)])
def test_row_max_in_outlier_column(mm, T, K):
    """Row scales over the non-outlier columns when a row's largest value
    below tau is in a column that other rows make an outlier (a pass that
    took the row maximum before knowing the outlier set would get it
    wrong)."""
    X = _row_max_in_outlier_column(T, K, 70_000 + K)
    W = synth.random_case(71_000 + K, 1, K, 8)[1]
    r, _ = run_case(mm, f"row max in an outlier column {T}x{K}", X, W, 6.0)
    assert int(r["count"][0]) == 2


@pytest.mark.parametrize("T,K", [(1100, 32768), (150, 20480)])
def test_many_outlier_dims(mm, T, K):
    """120 outlier dimensions spread over the row (more than 32 flagged
    bitmap words per row)."""
    X, W = synth.random_case(72_000 + K, T, K, 8, n_dims=120)
    run_case(mm, f"120 outlier dimensions {T}x{K}", X, W, 6.0)


def _random_shapes(n=24, seed=2024, max_macs=6e8):
    """Seeded shapes spread over every route of the library: row counts of
    the decode kernel, the streaming tiles and the large-tile kernel, K with
    and without a multiple of 1024 / 128 / 64, ragged N; each with a few
    planted outlier dimensions, every other one the memory-halved variant."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.choice([rng.integers(1, 9), rng.integers(9, 33), rng.integers(33, 129),
                            rng.integers(129, 400)]))
        K = int(rng.choice([1024 * rng.integers(1, 17), 128 * rng.integers(1, 80),
                            16 * rng.integers(1, 600)]))
        N = int(8 * rng.integers(1, 160))
        if T * K * N > max_macs:
            continue
        out.append((T, K, N, int(rng.integers(0, 9)), len(out) % 2 == 1))
    return out


@pytest.mark.parametrize("T,K,N,nd,halved", _random_shapes())
def test_random_shapes(mm, T, K, N, nd, halved):
    X, W = synth.random_case(50_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_case(mm, f"random {T}x{K}x{N}{' halved' if halved else ''}", X, W, 6.0, halved=halved)


def _random_long_rows(n=10, seed=77, max_macs=6e8):
    """Seeded shapes for the long-row activation kernels and the large-tile
    matmul: 300-2600 rows, K past 16384 (multiples of 16, of 64 or of 1024),
    narrow ragged N."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(300, 2600))
        K = int(rng.choice([16 * rng.integers(1025, 3073), 64 * rng.integers(257, 769),
                            1024 * rng.integers(17, 49)]))
        N = int(8 * rng.integers(1, 40))
        if T * K * N > max_macs:
            continue
        out.append((T, K, N, int(rng.integers(0, 40)), len(out) % 3 == 2))
    return out


@pytest.mark.parametrize("T,K,N,nd,halved", _random_long_rows())
def test_random_long_rows(mm, T, K, N, nd, halved):
    X, W = synth.random_case(51_000 + T + K + N + nd, T, K, N, n_dims=nd, x_dist="laplace")
    run_case(mm, f"long rows {T}x{K}x{N}{' halved' if halved else ''}", X, W, 6.0, halved=halved)


@pytest.mark.parametrize("T,K,N,nd,halved", [
    # streaming matmul's 128x128 tiles with K cut into slabs (tiles on at
    # most half of the CUs): 8 slabs, 6, 4 and 2 (ragged rows and columns),
    # many outliers, memory-halved
    (72, 49152, 264, 3, False), (128, 12288, 1032, 6, False), (100, 8192, 776, 4, False),
    (65, 4096, 136, 40, False), (96, 12288, 520, 20, True),
    # 64x64 tiles on at most a quarter of the slots: partial sums [S][T][N]
    # and the finishing kernel (8, 6 and 2 slabs; o > 16; memory-halved)
    (40, 12288, 1032, 3, False), (64, 49152, 4096, 5, False), (17, 4096, 264, 40, False),
    (33, 49152, 520, 20, True),
    # 256x128 tiles (129..256 rows) on at most half of the CUs: 6, 8 and 4 slabs
    (200, 12288, 1032, 4, False), (160, 16384, 520, 20, True), (256, 8192, 2056, 3, False),
])
def test_stream_k_split(mm, T, K, N, nd, halved):
    X, W = synth.random_case(34_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_case(mm, f"stream K split {T}x{K}x{N}", X, W, 6.0, halved=halved)


def test_stream_k_split_out_projection(mm):
    """The 175B-class out-projection at 128 rows (96 tiles of 128x128 on 256
    CUs, K split in two), checked on sampled rows."""
    X, W = synth.random_case(35_128, 128, 12288, 12288, n_dims=6)
    run_case(mm, "stream K split 128x12288x12288 (sampled rows)", X, W, 6.0,
             rows=[0, 1, 37, 64, 101, 127])


@pytest.mark.parametrize("T,K,N,nd,tau", [
    (1, 4096, 1000, 3, 6.0), (3, 4096, 8, 0, 6.0), (8, 8192, 2056, 6, 6.0),
    (16, 4096, 520, 5, 6.0), (8, 8192, 264, 300, 6.0),   # o > 256: values read from X
    (2, 4096, 136, 0, 0.0),                              # every dimension an outlier
    # 9 and 12 (the most) 16-row blocks per workgroup; 49160 columns: 3073
    # blocks, one more workgroup holding a half block
    (2, 4096, 36864, 3, 6.0), (1, 4096, 49160, 2, 6.0),
    # the decode workload's width with a half last block, more outliers than
    # the W16 values kept in LDS at that width, and 9 blocks per workgroup
    # with K = 4096 (4 chunks per block)
    (4, 8192, 28680, 5, 6.0), (8, 8192, 28672, 40, 6.0), (16, 4096, 36864, 3, 6.0),
])
def test_decode_path(mm, T, K, N, nd, tau):
    """Shapes on the single-kernel decode path (T <= 16, K in {4096, 8192})."""
    X, W = synth.random_case(30_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_case(mm, f"decode path {T}x{K}x{N} tau={tau}", X, W, tau)


@pytest.mark.parametrize("T,K,N,nd,tau,halved", [
    (8, 16384, 1000, 6, 6.0, False), (8, 16384, 1000, 6, 6.0, True),   # T*K = 128 KB
    (6, 5120, 520, 3, 6.0, False),                                     # K = 5 x 1024
    (8, 12288, 1000, 40, 6.0, False), (8, 12288, 264, 40, 6.0, True),  # o > 16
    (4, 16384, 264, 100, 6.0, False),                                  # o > 64: X from the workspace
    (1, 1024, 8, 0, 0.0, False), (1, 1024, 8, 0, 0.0, True),           # every dimension an outlier
    # 12 and 10 blocks per workgroup (W16 values and codes of 192 rows)
    (4, 1024, 49152, 5, 6.0, False), (4, 1024, 49152, 5, 6.0, True),
    (3, 2048, 36872, 20, 6.0, False), (3, 2048, 36872, 20, 6.0, True),
])
def test_decode_precomputed(mm, T, K, N, nd, tau, halved):
    """Few rows (T <= 8) off the single-kernel path: the activation-pass
    kernels, then the decode kernel's weight stream with the activation side
    read from the workspace."""
    X, W = synth.random_case(32_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_case(mm, f"decode (precomputed) {T}x{K}x{N} tau={tau}", X, W, tau, halved=halved)


@pytest.mark.parametrize("T,K,N,nd,tau", [
    (37, 80, 200, 2, 6.0), (300, 1040, 520, 3, 6.0),          # staged kernels
    (257, 2048, 1000, 70, 6.0), (129, 64, 8, 1, 6.0),          # large-tile kernel
    (1, 4096, 1000, 3, 6.0), (8, 8192, 264, 300, 6.0),         # decode kernel, o > 16
    (16, 4096, 520, 20, 6.0), (300, 24576, 520, 3, 6.0),      # K split in two
    (70, 1024, 136, 0, 0.0), (2, 4096, 136, 0, 0.0),           # every dimension an outlier
    (257, 1024, 264, 0, 0.0),       # o = 1024 > 512: rows recovered inside the matmul
    (300, 2048, 520, 600, 6.0),     # about 600 outliers, the same
    (64, 2048, 264, 600, 6.0), (100, 2048, 520, 40, 6.0),   # streaming kernel, W rows through LDS
    (30, 2048, 136, 0, 0.0),        # 30 rows, every dimension an outlier
    (160, 2048, 264, 300, 6.0),     # 256x128 streaming tile, recovered rows
    (300, 8192, 264, 40, 6.0),      # K split in two past 256 rows
    (8, 8192, 28680, 40, 6.0),      # decode kernel, half last block, o > 16
])
def test_memory_halved(mm, T, K, N, nd, tau):
    """W16 = NULL: outlier rows recovered from the Int8 weight."""
    X, W = synth.random_case(50_000 + T + K + N + nd, T, K, N, n_dims=nd)
    r, ref = run_case(mm, f"memory-halved {T}x{K}x{N} tau={tau}", X, W, tau, halved=True)
    if tau == 0.0:
        assert int(r["count"][0]) == K


def test_tau_zero_every_dimension_outlier(mm):
    X, W = synth.random_case(21, 70, 1024, 136)
    r, ref = run_case(mm, "tau=0", X, W, 0.0)
    assert int(r["count"][0]) == 1024 and not r["xq"].any()
    # the result is the 16-bit matmul
    y16 = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16)
    check_y(r["Y"].cpu().numpy(), y16, "tau=0 vs fp16 matmul")


def test_tau_infinity_pure_int8(mm):
    X, W = synth.random_case(22, 65, 320, 96, n_dims=4)
    r, _ = run_case(mm, "tau=inf", X, W, float("inf"))
    assert int(r["count"][0]) == 0


def test_zero_rows_and_exact_tie(mm):
    X, W = synth.random_case(23, 40, 128, 64)
    X[5] = 0                      # zero row: s_x = 0, Xq row 0
    X[7, :] = 0
    X[7, 9] = 6.0                 # row whose only nonzero is an outlier at the tie
    X[11, 33] = -6.0              # exact tie, negative
    r, _ = run_case(mm, "zero rows + ties", X, W, 6.0)
    idx = r["idx"][:int(r["count"][0])].cpu().tolist()
    assert 9 in idx and 33 in idx
    assert float(r["sx"][7]) == 0.0 and float(r["sx"][5]) == 0.0


def test_largest_k(mm):
    """K at the int32 bound with every quantized value at +-127: the largest
    accumulator magnitude 127^2 * K must come out exactly."""
    K = 133136
    X = np.ones((3, K), np.float16)
    X[1] = -1
    W = np.full((K, 16), 0.125, np.float16)   # Y = +-K/8 stays finite in fp16
    r, _ = run_case(mm, "largest K", X, W, 6.0)
    acc = r["acc"].cpu().numpy()
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K


def test_largest_accumulator_in_slabs(mm):
    """The same extreme accumulators with K = 130 x 1024 on the decode
    kernel's K slabs: every slab's partial sum and their total exact."""
    K = 133120
    X = np.ones((3, K), np.float16)
    X[1] = -1
    W = np.full((K, 16), 0.125, np.float16)
    r, _ = run_case(mm, "largest K in slabs", X, W, 6.0)
    acc = r["acc"].cpu().numpy()
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K


@pytest.mark.parametrize("T,K,N,nd,tau,halved", [
    (8, 49152, 1000, 10, 6.0, False), (8, 49152, 264, 10, 6.0, True),   # 48 chunks, >= 3 slabs
    (16, 32768, 1000, 20, 6.0, False),                                  # 32 chunks, >= 4 slabs
    (12, 33792, 520, 3, 6.0, True),                                     # slabs of unequal length
    (12, 32768, 1032, 5, 6.0, False),                                   # half a block at the end
    (8, 24576, 264, 4, 6.0, True),                                      # 8 rows: from 16 KB of Xq on
    (1, 133120, 8, 2, 6.0, False),                                      # the longest K in slabs
    (9, 32768, 136, 0, 0.0, False),                                     # every dimension an outlier
])
def test_decode_slabs(mm, T, K, N, nd, tau, halved):
    """Few rows whose Xq exceeds the decode kernel's LDS: K streamed in slabs
    by separate workgroups, partial sums added by a second kernel."""
    X, W = synth.random_case(34_000 + T + K + N + nd, T, K, N, n_dims=nd)
    run_case(mm, f"decode (K slabs) {T}x{K}x{N} tau={tau}", X, W, tau, halved=halved)


@pytest.mark.parametrize("T,K,N1,N2", [(96, 512, 264, 136), (300, 24576, 520, 264),
                                       (16, 8192, 1000, 264), (8, 49152, 1000, 264)])
def test_staged_entry_points_match(mm, T, K, N1, N2):
    # the second shape runs the matmul with K split in two halves
    X, W = synth.random_case(24, T, K, N1, n_dims=3)
    W2 = synth.random_case(25, 1, K, N2)[1]
    say(f"[case] staged entry points T={T} K={K} N={N1},{N2}")
    Xd, Wd, W2d = gpu(X), gpu(W), gpu(W2)
    Wq, sw = mm.quantize_weight(Wd)
    Wq2, sw2 = mm.quantize_weight(W2d)
    ws = mm.new_workspace(T, K, N1)
    mm.quantize_activations(Xd, N1, 6.0, ws)
    Y1 = mm.matmul_prepared(ws, T, K, Wq, sw, Wd)
    Y2 = mm.matmul_prepared(ws, T, K, Wq2, sw2, W2d)   # one pass of X, two weights
    Y1b = mm.matmul_prepared(ws, T, K, Wq, sw, Wd)     # and the first again
    H2 = mm.matmul_prepared(ws, T, K, Wq2, sw2, None)  # memory-halved
    R1 = mm.mixed_matmul(Xd, Wq, sw, Wd, 6.0)
    R2 = mm.mixed_matmul(Xd, Wq2, sw2, W2d, 6.0)
    RH2 = mm.mixed_matmul(Xd, Wq2, sw2, None, 6.0)
    torch.cuda.synchronize()
    assert torch.equal(Y1, R1) and torch.equal(Y2, R2) and torch.equal(Y1b, R1)
    assert torch.equal(H2, RH2)


# ----------------------------------------------------------- full-size workloads

def test_split_whole_and_half_tiles(mm):
    """More 256x256 tiles than compute units with K split in two: one round
    of tiles runs all of K and only the rest are split in halves (9 x 29 =
    261 tiles; on 256 CUs the split ones are tiles 256..260, in the last
    column of tiles, rows 1024 on).  Rows checked in whole and split tiles."""
    X, W = synth.random_case(73_000, 2304, 8192, 7424, n_dims=5)
    run_case(mm, "whole and split tiles 2304x8192x7424", X, W, 6.0,
             rows=[0, 255, 256, 1000, 1024, 2047, 2048, 2300, 2303])


def _sample_rows(T, rowsel, n=12, seed=0):
    """Rows to check against the oracle: first, last, random, and rows that
    carry planted outliers."""
    rng = np.random.default_rng(seed)
    rows = {0, T - 1, *rng.choice(T, n, replace=False).tolist()}
    if rowsel is not None:
        for j in range(min(3, len(rowsel))):
            rows.add(int(np.flatnonzero(rowsel[j])[0]))
    return sorted(rows)


def test_decode_config(mm):
    w = synth.WORKLOADS["dec"]
    X, W = synth.make_x(w), synth.make_w(w)
    r, _ = run_case(mm, "dec (full)", X, W, w.tau)
    assert sorted(r["idx"][:int(r["count"][0])].cpu().tolist()) == sorted(synth.planted(w)[0].tolist())


@pytest.mark.parametrize("name", ["up", "down"])
def test_prefill_config(mm, name):
    w = synth.WORKLOADS[name]
    X, W = synth.make_x(w), synth.make_w(w)
    dims, _, rowsel = synth.planted(w)
    r, _ = run_case(mm, f"{name} (sampled rows)", X, W, w.tau,
                    rows=_sample_rows(w.T, rowsel), plain_too=True)
    idx = set(r["idx"][:int(r["count"][0])].cpu().tolist())
    assert set(dims.tolist()) <= idx


@pytest.mark.parametrize("name", ["sweep_qkv_256", "sweep_out_0"])
def test_sweep_config(mm, name):
    w = synth.WORKLOADS[name]
    X, W = synth.make_x(w), synth.make_w(w)
    r, _ = run_case(mm, f"{name} (sampled rows)", X, W, w.tau, rows=_sample_rows(w.T, None, n=8))
    assert int(r["count"][0]) >= w.n_dims


@pytest.mark.parametrize("name", ["dec", "up"])
def test_memory_halved_config(mm, name):
    """The memory-halved variant (no 16-bit weight) on the decode and prefill
    up-projection workloads at full size (acc and Y on sampled rows for the
    prefill one)."""
    w = synth.WORKLOADS[name]
    X, W = synth.make_x(w), synth.make_w(w)
    dims, _, rowsel = synth.planted(w)
    rows = None if w.T <= 16 else _sample_rows(w.T, rowsel, n=6)
    r, _ = run_case(mm, f"{name} memory-halved", X, W, w.tau, rows=rows, halved=True)
    assert set(dims.tolist()) <= set(r["idx"][:int(r["count"][0])].cpu().tolist())


@pytest.mark.parametrize("name", ["sweep_up_64", "sweep_down_8"])
def test_sweep_config_more(mm, name):
    """Two more projections of the 175B-class block sweep (T = 4096)."""
    w = synth.WORKLOADS[name]
    X, W = synth.make_x(w), synth.make_w(w)
    r, _ = run_case(mm, f"{name} (sampled rows)", X, W, w.tau, rows=_sample_rows(w.T, None, n=6))
    assert int(r["count"][0]) >= w.n_dims
