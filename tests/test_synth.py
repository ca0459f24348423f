"""The seeded input generator: determinism, thread-count independence, fp16
rounding, and the workload recipes.  CPU only."""
import numpy as np

import synth


def test_thread_count_independent():
    a = synth.matrix_f16(300, 700, 42, synth.STREAM_X, "normal", 1.0, threads=1)
    b = synth.matrix_f16(300, 700, 42, synth.STREAM_X, "normal", 1.0, threads=7)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    c = synth.matrix_f16(300, 700, 43, synth.STREAM_X, "normal", 1.0)
    assert not np.array_equal(a, c)


def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(5000) * 10.0 ** rng.integers(-9, 6, 5000)
    v = np.concatenate([v, [65504.0, 65519.9, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, -0.0]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([synth.f64_to_f16_bits(x) for x in v], np.uint16)
    assert np.array_equal(got, ref)


def test_distributions():
    x = synth.matrix_f16(500, 800, 9, 1, "normal", 0.02).astype(np.float64)
    assert abs(x.std() - 0.02) < 0.0005 and abs(x.mean()) < 0.0005
    y = synth.matrix_f16(500, 800, 9, 1, "laplace", 0.5).astype(np.float64)
    assert abs(np.abs(y).mean() - 0.5) < 0.01 and abs(y.std() - 0.5 * 2 ** 0.5) < 0.02


def test_tiny_recipe():
    w = synth.WORKLOADS["tiny"]
    X = synth.make_x(w)
    assert X.shape == (16, 64)
    mags = np.abs(X[:, [3, 17]].astype(np.float64))
    assert mags.min() >= 8.0 and mags.max() <= 20.0
    others = np.delete(X.astype(np.float64), [3, 17], axis=1)
    assert np.abs(others).max() < 6.0
    assert synth.make_w(w).shape == (64, 48)


def test_planted_dims_and_rows():
    w = synth.WORKLOADS["up"]
    dims, factors, rowsel = synth.planted(w)
    assert len(set(dims.tolist())) == 7 and dims.min() >= 0 and dims.max() < w.K
    assert np.all((factors >= 10) & (factors <= 60))
    assert rowsel.shape == (7, 2048) and np.all(rowsel.sum(1) == 512)
    X = synth.make_x(w, T=2048, K=w.K)
    xf = np.abs(X[:, dims].astype(np.float32))
    for j in range(7):
        # the scaled rows are exactly the selected ones (factor >= 10 makes
        # them large on average, the others stay N(0,1))
        assert xf[rowsel[j] == 1, j].mean() > 5 * xf[rowsel[j] == 0, j].mean()


def test_choose_distinct():
    c = synth.choose(5, 3, 100, 100)
    assert sorted(c.tolist()) == list(range(100))
