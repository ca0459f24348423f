"""Pins for the CPU oracle: checks against values that do not come from the
oracle itself.

Each ``pin_*`` takes a loaded oracle build and raises AssertionError when it
disagrees with:
  - hand-derived worked examples (tests/golden/*.json, derivations inside);
  - closed forms and invariants of absmax quantization (error at most half a
    quantization step, the absmax element maps to +-127, signs kept);
  - library routines the special cases reduce to (numpy int64 / float64
    matmul, numpy's float16 conversion);
  - metamorphic relations (power-of-two scaling, joint permutation of the
    hidden dimension).

Sources of the method: LLM.int8() abstract (taxoreview.com page, second
paragraph) and "LLM.int8(): A Procedure for Int8 Matrix Multiplication in
Transformer Language Models", section "The LLM.int8() Methodology".
"""
from __future__ import annotations

import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
# |x - q*s/127| <= s/254 * (1 + SLACK): the two fp32 roundings in
# x * fp32(127/s) move the product by at most 127 * 2^-23 quantization steps,
# i.e. 3.03e-5 of the half step; 2^-14 = 6.1e-5 leaves margin.
SLACK = 2.0 ** -14


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _case(seed, T, K, N, n_dims=0, factor=15.0, x_dist="normal", w_sigma=0.05):
    return synth.random_case(seed, T, K, N, n_dims=n_dims, factor=factor, x_dist=x_dist,
                             w_sigma=w_sigma)


# ------------------------------------------------------------------ fp16 codec

def pin_f16_codec(orc):
    """Decode every binary16 pattern and encode doubles, against numpy."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([orc.f16_decode(int(b)) for b in bits[fin][::7]])
    assert np.array_equal(got, ref[fin][::7]), "fp16 decode"
    for b in (0x7C00, 0xFC00):
        assert np.isinf(orc.f16_decode(b))
    rng = np.random.default_rng(7)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000)
    # exact ties between neighbours, both parities, and the range edges
    grid = np.arange(0, 64, dtype=np.float64)
    ties = (1024 + grid + 0.5) * 2.0 ** -10 * 4            # halfway points in [4, 8)
    sub_ties = (grid + 0.5) * 2.0 ** -24                   # halfway points among subnormals
    edges = np.array([65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                      2.0 ** -14 - 2.0 ** -25, 0.0, -0.0])
    v = np.concatenate([v, ties, -ties, sub_ties, edges])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([orc.f16_encode(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref), f"fp16 encode: {np.flatnonzero(got != ref)[:5]}"


# -------------------------------------------------------- hand-worked examples

def pin_hand_example(orc):
    g = _load("hand_2x4x2.json")
    X = np.array(g["X"], np.float16)
    W = np.array(g["W"], np.float16)
    Wq, sw = orc.quantize_weight(W)
    assert np.array_equal(Wq, np.array(g["Wq_NK"], np.int8)), "hand Wq"
    assert np.array_equal(sw, np.array(g["sw"], np.float32)), "hand sw"
    r = orc.mixed_matmul(X, Wq, sw, W, g["tau"])
    assert r["idx"].tolist() == g["idx"], "hand idx"
    assert np.array_equal(r["sx"], np.array(g["sx"], np.float32)), "hand sx"
    assert np.array_equal(r["xq"], np.array(g["Xq"], np.int8)), "hand Xq"
    assert np.array_equal(r["acc"], np.array(g["acc"], np.int32)), "hand acc"
    num = np.array([a / b + c for a, b, c in g["Y64_num"]]).reshape(2, 2)
    assert np.allclose(r["Y64"], num, rtol=1e-14, atol=0), "hand Y64"
    assert np.array_equal(r["Y"].astype(np.float64), np.array(g["Y"])), "hand Y"


def pin_hand_memory_halved(orc):
    """The hand example without the 16-bit weight (outlier row recovered
    from the Int8 weight)."""
    g = _load("hand_2x4x2.json")
    h = g["memory_halved"]
    X = np.array(g["X"], np.float16)
    W = np.array(g["W"], np.float16)
    Wq, sw = orc.quantize_weight(W)
    for n in range(2):
        bits = orc.dequant_weight(int(Wq[n, 3]), float(sw[n]))
        assert orc.f16_decode(bits) == h["What_row3"][n], "hand recovered weight"
    r = orc.mixed_matmul(X, Wq, sw, None, g["tau"])
    assert np.array_equal(r["acc"], np.array(g["acc"], np.int32)), "hand acc (memory-halved)"
    num = np.array([a / b + c for a, b, c in h["Y64_num"]]).reshape(2, 2)
    assert np.allclose(r["Y64"], num, rtol=1e-14, atol=0), "hand Y64 (memory-halved)"
    assert np.array_equal(r["Y"].astype(np.float64), np.array(h["Y"])), "hand Y (memory-halved)"


def pin_dequant_weight(orc):
    """Recovered weight values: within half an fp16 step (plus the two fp32
    roundings) of q * s_w / 127, odd in q, monotone in q, exact for
    s_w = 127 (the codes themselves), 0 for q = 0."""
    rng = np.random.default_rng(7)
    scales = [127.0, 2.0, 0.015, 3.0e-5, 0.4990234375, 1000.0] + list(rng.uniform(1e-3, 50, 6))
    for s in scales:
        s = float(np.float32(s))
        vals = np.array([orc.f16_decode(orc.dequant_weight(q, s)) for q in range(-127, 128)])
        exact = np.arange(-127, 128) * s / 127.0
        # half an fp16 ulp of the value (2^-11 relative, 2^-25 absolute below
        # the normal range) plus the fp32 divide and multiply (2^-23 each)
        bound = np.abs(exact) * (2.0 ** -11 + 2.0 ** -22) + 2.0 ** -25
        assert np.all(np.abs(vals - exact) <= bound), f"recovered weight error, s_w={s}"
        assert vals[127] == 0.0, "q = 0"
        assert np.array_equal(vals[::-1], -vals), "odd in q"
        assert np.all(np.diff(vals) >= 0), "monotone in q"
        if s == 127.0:
            assert np.array_equal(vals, np.arange(-127, 128, dtype=np.float64)), "s_w = 127"


def pin_memory_halved_tau_zero(orc):
    """tau = 0, memory-halved: every dimension is an outlier and Xq is 0, so
    Y is the fp16 matmul of X with the recovered weight, rounded once
    (numpy float64 matmul; the recovered values come from
    pin_dequant_weight's function)."""
    for seed, (T, K, N) in enumerate([(5, 32, 16), (17, 48, 24)]):
        X, W = _case(300 + seed, T, K, N, n_dims=2, factor=9.0)
        Wq, sw = orc.quantize_weight(W)
        What = np.empty((K, N), np.float64)
        for n in range(N):
            for k in range(K):
                What[k, n] = orc.f16_decode(orc.dequant_weight(int(Wq[n, k]), float(sw[n])))
        r = orc.mixed_matmul(X, Wq, sw, None, 0.0)
        ref = X.astype(np.float64) @ What
        assert r["o"] == K and not r["xq"].any(), "tau = 0 isolates everything"
        assert np.allclose(r["Y64"], ref, rtol=1e-13, atol=1e-300), "memory-halved tau=0 Y64"
        assert np.array_equal(r["Y"], ref.astype(np.float16)), "memory-halved tau=0 Y"


def pin_memory_halved_exact_weight(orc):
    """When every weight is its own Int8 code (integer values with a 127 in
    each column, so s_w = 127 and W^ = W exactly), the memory-halved result
    equals the result with the 16-bit weight, bit for bit."""
    rng = np.random.default_rng(11)
    for T, K, N in [(6, 32, 16), (9, 64, 8)]:
        X, _ = _case(400 + K, T, K, N, n_dims=3, factor=9.0)
        W = rng.integers(-127, 128, size=(K, N)).astype(np.float16)
        W[rng.integers(0, K, size=N), np.arange(N)] = 127.0
        Wq, sw = orc.quantize_weight(W)
        assert np.all(sw == 127.0) and np.array_equal(Wq.T.astype(np.float16), W)
        a = orc.mixed_matmul(X, Wq, sw, W, 6.0)
        b = orc.mixed_matmul(X, Wq, sw, None, 6.0)
        assert a["o"] > 0
        assert np.array_equal(a["Y"], b["Y"]) and np.array_equal(a["Y64"], b["Y64"]), \
            "memory-halved with exact weights"


def pin_bf16_decode(orc):
    """Every bfloat16 bit pattern widens exactly as torch converts it."""
    import torch
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    mine = np.array([orc.bf16_decode(int(b)) for b in bits], np.float32)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all(), "bf16 decode"


def pin_typed_weight_hand(orc):
    """Hand-derived conversions of an fp32 and a bf16 checkpoint column."""
    g = _load("typed_weight.json")
    f = g["f32"]
    col = np.array(f["column"], np.float32)
    assert col[0] == np.float32(1.0 - 2.0 ** -20)
    Wq, sw = orc.quantize_weight_typed(col.reshape(-1, 1), "f32")
    assert float(sw[0]) == f["sw"] and Wq[0].tolist() == f["q"], f"fp32 column: {Wq[0].tolist()}"
    Wq16, _ = orc.quantize_weight(col.astype(np.float16).reshape(-1, 1))
    assert Wq16[0].tolist() == f["q_if_fp16"], "the same column in fp16"
    b = g["bf16"]
    bits = np.array(b["column_bits"], np.uint16)
    assert [orc.bf16_decode(int(x)) for x in bits] == b["column"]
    Wq, sw = orc.quantize_weight_typed(bits.reshape(-1, 1), "bf16")
    assert float(sw[0]) == b["sw"] and Wq[0].tolist() == b["q"], f"bf16 column: {Wq[0].tolist()}"


def pin_typed_weight_containers(orc):
    """The conversion depends on the values, not on the container: fp16
    weights stored as fp32 (always exact) and as bf16 (when exact there)
    give the fp16 result; fp32 weights satisfy the quantizer invariants."""
    rng = np.random.default_rng(5)
    for K, N in [(64, 48), (128, 24)]:
        W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
        ref = orc.quantize_weight(W)
        got = orc.quantize_weight_typed(W.astype(np.float32), "f32")
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), "fp32 container"
        # values with at most 8 significant bits are exact in bf16 and fp16
        Wb = (np.round(rng.standard_normal((K, N)) * 64) / 256).astype(np.float16)
        bits = (Wb.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(bits.astype(np.uint32) << 16, Wb.astype(np.float32).view(np.uint32))
        ref = orc.quantize_weight(Wb)
        got = orc.quantize_weight_typed(bits, "bf16")
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), "bf16 container"
        # fp32 values: absmax element -> +-127, |x - q s/127| <= s/254 (1 + 2^-14)
        W32 = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
        Wq, sw = orc.quantize_weight_typed(W32, "f32")
        assert np.array_equal(sw, np.abs(W32).max(axis=0)), "fp32 scale"
        amax = np.abs(W32).argmax(axis=0)
        assert np.array_equal(np.abs(Wq[np.arange(N), amax]), np.full(N, 127)), "absmax -> 127"
        err = np.abs(W32.T.astype(np.float64) - Wq * (sw.astype(np.float64)[:, None] / 127.0))
        assert np.all(err <= sw[:, None] / 254.0 * (1 + 2.0 ** -14)), "fp32 quantization error"


def _bf16_bits(a):
    """float32 values that are exact in bf16 -> their bf16 bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def pin_bf16_encode(orc):
    """Rounding to bfloat16: every finite pattern round-trips; exact
    midpoints go to the even neighbour and anything off the midpoint to
    the nearer one; the overflow and underflow edges; and on fp32 inputs
    the integer round-half-even of the bit pattern."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)              # +0 .. max finite
    vals = np.array([orc.bf16_decode(int(b)) for b in pos], np.float64)
    for b, v in zip(pos[::97], vals[::97]):
        assert orc.bf16_encode(v) == b and orc.bf16_encode(-v) == (b | 0x8000), f"round trip {b:#x}"
    for i in range(0, len(pos) - 1, 89):
        lo, hi = vals[i], vals[i + 1]
        mid = (lo + hi) / 2                                   # exact in double
        even = int(pos[i]) if pos[i] % 2 == 0 else int(pos[i + 1])
        assert orc.bf16_encode(mid) == even, f"midpoint above {pos[i]:#x}"
        d = (hi - lo) / 1024
        assert orc.bf16_encode(mid - d) == pos[i] and orc.bf16_encode(mid + d) == pos[i + 1]
    top = (2 - 2.0 ** -8) * 2.0 ** 127
    assert orc.bf16_encode(top) == 0x7F80 and orc.bf16_encode(np.nextafter(top, 0)) == 0x7F7F
    assert orc.bf16_encode(2.0 ** -134) == 0 and orc.bf16_encode(1.5 * 2.0 ** -134) == 1
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-130, 120, 4000))).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)   # integer RNE
    mine = np.array([orc.bf16_encode(float(v)) for v in x], np.uint16)
    assert np.array_equal(mine, ref), "rounding of fp32 values"


def pin_hand_bf16(orc):
    """The hand example in the bf16 variant."""
    g = _load("hand_2x4x2.json")
    X = _bf16_bits(np.array(g["X"], np.float32))
    W = np.array(g["W"], np.float32)
    Wq, sw = orc.quantize_weight_typed(_bf16_bits(W), "bf16")
    assert np.array_equal(Wq, np.array(g["Wq_NK"], np.int8)) and sw.tolist() == g["sw"]
    r = orc.mixed_matmul(X, Wq, sw, _bf16_bits(W), g["tau"], htype="bf16")
    assert r["idx"].tolist() == g["idx"] and np.array_equal(r["xq"], np.array(g["Xq"], np.int8))
    assert np.array_equal(r["acc"], np.array(g["acc"], np.int32)), "hand acc (bf16)"
    num = np.array([a / b + c for a, b, c in g["Y64_num"]]).reshape(2, 2)
    assert np.allclose(r["Y64"], num, rtol=1e-14, atol=0), "hand Y64 (bf16)"
    Y = np.array([[orc.bf16_decode(int(b)) for b in row] for row in r["Y"]])
    assert np.array_equal(Y, np.array(g["bf16"]["Y"])), f"hand Y (bf16): {Y.tolist()}"


def pin_bf16_same_values(orc):
    """Inputs exact in both fp16 and bf16: the bf16 variant gives the same
    outlier set, Xq, s_x, acc and Y64 as the fp16 path, and Y is the bf16
    rounding of Y64; tau = 0 gives the float64 matmul of the inputs."""
    rng = np.random.default_rng(9)
    for T, K, N in [(6, 48, 16), (13, 64, 24)]:
        # at most 8 significant bits and small exponents: exact in both types
        X = (np.round(rng.standard_normal((T, K)) * 32) / 32).astype(np.float32)
        X[:, 5] *= 8
        W = (np.round(rng.standard_normal((K, N)) * 64) / 2048).astype(np.float32)
        Xh, Wh = X.astype(np.float16), W.astype(np.float16)
        Xb, Wb = _bf16_bits(X), _bf16_bits(W)
        Wq, sw = orc.quantize_weight(Wh)
        for tau in (6.0, 0.0, float("inf")):
            a = orc.mixed_matmul(Xh, Wq, sw, Wh, tau)
            b = orc.mixed_matmul(Xb, Wq, sw, Wb, tau, htype="bf16")
            for key in ("idx", "xq", "sx", "acc", "Y64"):
                assert np.array_equal(a[key], b[key]), f"bf16 variant {key}, tau={tau}"
            enc = np.array([[orc.bf16_encode(v) for v in row] for row in b["Y64"]], np.uint16)
            assert np.array_equal(b["Y"], enc), "bf16 rounding of Y64"
            if tau == 0.0:
                assert np.allclose(b["Y64"], X.astype(np.float64) @ W.astype(np.float64),
                                   rtol=1e-13, atol=1e-300), "tau = 0 (bf16)"


def pin_quant_ties(orc):
    g = _load("quant_ties.json")
    for c in g["cases"]:
        row = np.array([c["row"]], np.float16)
        flag = np.zeros(row.shape[1], np.uint8)
        q, s = orc.quantize_rows(row, flag)
        assert float(s[0]) == c["s"], f"scale {c['note']}"
        assert q[0].tolist() == c["q"], f"row quant {c['note']}: {q[0].tolist()}"
        # the same values as one weight column
        wq, sw = orc.quantize_weight(row.T.copy())
        assert float(sw[0]) == c["s"] and wq[0].tolist() == c["q"], f"weight {c['note']}"


# --------------------------------------------------------------- outlier set

def tiny_scale_cases():
    """The hand-derived tiny-scale cases (tests/golden/tiny_scale.json) as
    arrays: a bf16 activation row (uint16 bit patterns) and an fp32
    checkpoint column, each with its scale and codes."""
    g = _load("tiny_scale.json")
    b = g["bf16_row"]
    # bf16 subnormal k * 2^-133 has bit pattern k (sign in bit 15)
    assert b["unit_log2"] == -133
    row_bits = np.array([abs(u) | (0x8000 if u < 0 else 0) for u in b["x_units"]], np.uint16)
    c = g["f32_column"]
    col = np.array([u * 2.0 ** c["unit_log2"] for u in c["x_units"]], np.float32)
    assert all(float(v) == u * 2.0 ** c["unit_log2"] for v, u in zip(col, c["x_units"]))
    return (row_bits, b["s_units"] * 2.0 ** b["unit_log2"], b["q"],
            col, c["s_units"] * 2.0 ** c["unit_log2"], c["q"])


def pin_tiny_scale(orc):
    """Scales whose fp32 reciprocal 127/s would overflow: the reciprocal is
    read with an unbounded exponent (tests/golden/tiny_scale.json)."""
    row_bits, s_row, q_row, col, s_col, q_col = tiny_scale_cases()
    K = 16
    X = np.zeros((1, K), np.uint16)
    X[0, :len(row_bits)] = row_bits
    Xq, sx = orc.quantize_rows(X, np.zeros(K, np.uint8), htype="bf16")
    assert float(sx[0]) == s_row, "tiny bf16 row scale"
    assert Xq[0, :len(q_row)].tolist() == q_row and not Xq[0, len(q_row):].any(), \
        f"tiny bf16 row codes {Xq[0].tolist()}"
    W = np.zeros((K, 8), np.float32)
    W[:len(col), 0] = col
    W[:, 1:] = 1.0                      # other columns: plain values
    Wq, sw = orc.quantize_weight_typed(W, "f32")
    assert float(sw[0]) == s_col, "tiny fp32 column scale"
    assert Wq[0, :len(q_col)].tolist() == q_col and not Wq[0, len(q_col):].any(), \
        f"tiny fp32 column codes {Wq[0].tolist()}"
    assert (Wq[1:] == 127).all() and (sw[1:] == 1.0).all()


def pin_detect(orc):
    for seed, (T, K) in enumerate([(16, 64), (37, 80), (5, 304), (64, 128)]):
        X, _ = _case(100 + seed, T, K, 8, n_dims=3, factor=9.0)
        for tau in (6.0, 3.5, 1.0):
            ref = np.any(np.abs(X.astype(np.float32)) >= np.float32(tau), axis=0)
            assert np.array_equal(orc.detect(X, tau).astype(bool), ref), f"detect tau={tau}"
        assert orc.detect(X, 0.0).all(), "tau = 0 flags every dimension"
        assert not orc.detect(X, float("inf")).any(), "tau = inf flags none"
    # exact tie at the threshold counts as crossing; the next fp16 below does not
    X = np.zeros((3, 16), np.float16)
    X[1, 5] = 6.0
    X[2, 9] = -6.0
    X[0, 11] = np.float16(6.0) - np.float16(2.0 ** -8)     # 5.99609375
    f = orc.detect(X, 6.0)
    assert f.tolist() == [1 if k in (5, 9) else 0 for k in range(16)], "tie handling"


def pin_compact(orc):
    rng = np.random.default_rng(3)
    for K in (1, 16, 100, 1000):
        for p in (0.0, 0.1, 0.5, 1.0):
            flag = (rng.random(K) < p).astype(np.uint8)
            assert np.array_equal(orc.compact(flag), np.flatnonzero(flag)), "compact"


def pin_tiny_config(orc):
    w = synth.WORKLOADS["tiny"]
    X = synth.make_x(w)
    flag = orc.detect(X, w.tau)
    assert orc.compact(flag).tolist() == [3, 17], "tiny config outlier set"


# ----------------------------------------------------- quantizer invariants

def _check_absmax_rows(Xf, q, s, excluded):
    """Invariants of symmetric absmax quantization of each row of Xf (float64)
    over the columns not in `excluded` (bool per column)."""
    keep = ~excluded
    ref_s = np.abs(Xf[:, keep]).max(axis=1) if keep.any() else np.zeros(len(Xf))
    assert np.array_equal(s.astype(np.float64), ref_s), "scale = absmax over kept columns"
    assert np.all(q[:, excluded] == 0), "excluded columns are zero"
    assert np.all(np.abs(q.astype(np.int32)) <= 127), "range [-127, 127]"
    for t in range(len(Xf)):
        if s[t] == 0:
            assert not q[t].any(), "zero scale gives zero row"
            continue
        xk = Xf[t, keep]
        qk = q[t, keep].astype(np.float64)
        am = np.argmax(np.abs(xk))
        assert qk[am] == np.sign(xk[am]) * 127, "absmax element maps to +-127"
        assert np.all((np.sign(qk) == np.sign(xk)) | (qk == 0)), "sign kept or zero"
        err = np.abs(xk - qk * float(s[t]) / 127.0)
        assert np.all(err <= float(s[t]) / 254.0 * (1 + SLACK)), "error above half a step"
        # values far from a rounding boundary quantize to the nearest integer
        exact = xk * 127.0 / float(s[t])
        safe = np.abs(exact - np.floor(exact) - 0.5) > 1e-3
        assert np.array_equal(qk[safe], np.rint(exact[safe])), "nearest level"


def pin_quant_invariants(orc):
    for seed, (T, K, nd, dist) in enumerate([(16, 64, 2, "normal"), (33, 96, 5, "laplace"),
                                             (7, 160, 0, "normal"), (20, 48, 48, "normal")]):
        X, W = _case(200 + seed, T, K, 40, n_dims=nd, x_dist=dist)
        X[3 % T] = 0                                    # an all-zero row
        flag = orc.detect(X, 6.0)
        q, s = orc.quantize_rows(X, flag)
        _check_absmax_rows(X.astype(np.float64), q, s, flag.astype(bool))
        Wq, sw = orc.quantize_weight(W)
        assert Wq.shape == (W.shape[1], W.shape[0]), "Wq stored [N,K]"
        _check_absmax_rows(W.T.astype(np.float64), Wq, sw, np.zeros(K, bool))
    # grid values quantize exactly: x = j * s / 127 with s = 127 -> q = j
    j = np.arange(-127, 128, dtype=np.float64)
    row = np.array([j], np.float16)
    q, s = orc.quantize_rows(row, np.zeros(row.shape[1], np.uint8))
    assert np.array_equal(q[0].astype(np.float64), j) and s[0] == 127.0, "grid values"
    # a row whose largest entry sits in an outlier column takes its scale
    # from the remaining columns
    X = np.array([[1.0, -3.0, 50.0, 2.0]], np.float16)
    q, s = orc.quantize_rows(X, np.array([0, 0, 1, 0], np.uint8))
    assert s[0] == 3.0 and q[0].tolist() == [42, -127, 0, 85], "outlier excluded from scale"


# ------------------------------------------------------------- int8 matmul

def pin_gemm(orc):
    rng = np.random.default_rng(11)
    for M, K, N in [(1, 1, 1), (3, 17, 5), (16, 64, 48), (9, 256, 33)]:
        a = rng.integers(-127, 128, (M, K)).astype(np.int8)
        b = rng.integers(-127, 128, (N, K)).astype(np.int8)
        ref = a.astype(np.int64) @ b.astype(np.int64).T
        assert np.array_equal(orc.int8_gemm(a, b).astype(np.int64), ref), "int8 gemm"
    # the extreme sum 127*127*K fits int32 up to K = 133144 and not beyond
    a = np.full((1, 133144), 127, np.int8)
    assert int(orc.int8_gemm(a, a)[0, 0]) == 127 * 127 * 133144, "largest in-range sum"
    a = np.full((1, 133145), 127, np.int8)
    try:
        orc.int8_gemm(a, a)
    except OverflowError:
        pass
    else:
        raise AssertionError("overflow past 133144 not reported")


# --------------------------------------------------- the whole method's Y

def pin_tau_inf(orc):
    """No outliers: Y is the plain vector-wise int8 matmul, i.e. the product
    of the dequantized operands (numpy float64 matmul)."""
    for seed, (T, K, N) in enumerate([(16, 64, 48), (21, 96, 40)]):
        X, W = _case(300 + seed, T, K, N, n_dims=2)
        Wq, sw = orc.quantize_weight(W)
        r = orc.mixed_matmul(X, Wq, sw, W, float("inf"))
        assert r["o"] == 0
        xd = r["xq"].astype(np.float64) * r["sx"].astype(np.float64)[:, None] / 127.0
        wd = Wq.astype(np.float64) * sw.astype(np.float64)[:, None] / 127.0
        ref = xd @ wd.T
        assert np.allclose(r["Y64"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), "tau=inf"
        assert np.array_equal(r["Y"], ref.astype(np.float16)), "tau=inf fp16"


def pin_tau_zero(orc):
    """Every dimension an outlier: Y is the 16-bit matmul (numpy float64,
    then one rounding to fp16)."""
    for seed, (T, K, N) in enumerate([(16, 64, 48), (5, 80, 24)]):
        X, W = _case(400 + seed, T, K, N)
        Wq, sw = orc.quantize_weight(W)
        r = orc.mixed_matmul(X, Wq, sw, W, 0.0)
        assert r["o"] == K and not r["xq"].any() and not r["sx"].any()
        ref = X.astype(np.float64) @ W.astype(np.float64)
        assert np.allclose(r["Y64"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), "tau=0"
        assert np.array_equal(r["Y"], ref.astype(np.float16)), "tau=0 fp16"


def pin_error_bound(orc):
    """|Y64 - X W| <= sum over non-outlier k of |x| e_w + |w_hat| e_x, with
    e = s/254 (1 + SLACK) the per-element quantization bound (x w - xh wh =
    x (w - wh) + wh (x - xh)); outlier dimensions contribute no error."""
    for seed, (T, K, N, nd) in enumerate([(16, 64, 48, 2), (24, 128, 56, 6), (8, 96, 32, 0)]):
        X, W = _case(500 + seed, T, K, N, n_dims=nd)
        Wq, sw = orc.quantize_weight(W)
        r = orc.mixed_matmul(X, Wq, sw, W, 6.0)
        Xf, Wf = X.astype(np.float64), W.astype(np.float64)
        keep = ~r["flag"].astype(bool)
        ex = r["sx"].astype(np.float64) / 254 * (1 + SLACK)
        ew = sw.astype(np.float64) / 254 * (1 + SLACK)
        wh = Wq.T.astype(np.float64) * sw.astype(np.float64)[None, :] / 127
        bound = (np.abs(Xf[:, keep]).sum(1)[:, None] * ew[None, :]
                 + ex[:, None] * np.abs(wh[keep]).sum(0)[None, :])
        exact = Xf @ Wf
        err = np.abs(r["Y64"] - exact)
        assert np.all(err <= bound + 1e-12 * np.abs(Xf) @ np.abs(Wf)), "quantization error bound"
        if nd:
            assert r["o"] >= nd


def pin_metamorphic_scale(orc):
    """X * 2^e with tau * 2^e: same outliers, Xq and acc; s_x and Y scale by 2^e."""
    X, W = _case(600, 12, 64, 24, n_dims=2)
    Wq, sw = orc.quantize_weight(W)
    base = orc.mixed_matmul(X, Wq, sw, W, 6.0)
    for e in (-3, 2):
        Xs = (X.astype(np.float64) * 2.0 ** e).astype(np.float16)
        r = orc.mixed_matmul(Xs, Wq, sw, W, 6.0 * 2.0 ** e)
        assert np.array_equal(r["idx"], base["idx"]) and np.array_equal(r["xq"], base["xq"])
        assert np.array_equal(r["acc"], base["acc"])
        assert np.array_equal(r["sx"], base["sx"] * np.float32(2.0 ** e))
        assert np.allclose(r["Y64"], base["Y64"] * 2.0 ** e, rtol=1e-13, atol=0)


def pin_permutation(orc):
    """Permuting the hidden dimension of X's columns and W's rows together
    permutes the outlier set and leaves s_x, s_w, acc and Y unchanged."""
    X, W = _case(700, 10, 80, 16, n_dims=3)
    Wq, sw = orc.quantize_weight(W)
    base = orc.mixed_matmul(X, Wq, sw, W, 6.0)
    perm = np.random.default_rng(5).permutation(80)
    Xp, Wp = X[:, perm].copy(), W[perm].copy()
    Wqp, swp = orc.quantize_weight(Wp)
    assert np.array_equal(swp, sw) and np.array_equal(Wqp, Wq[:, perm])
    r = orc.mixed_matmul(Xp, Wqp, swp, Wp, 6.0)
    inv = np.argsort(perm)
    assert sorted(perm[r["idx"]].tolist()) == base["idx"].tolist()
    assert sorted(inv[base["idx"]].tolist()) == r["idx"].tolist()
    assert np.array_equal(r["sx"], base["sx"]) and np.array_equal(r["acc"], base["acc"])
    assert np.allclose(r["Y64"], base["Y64"], rtol=1e-12, atol=1e-12)


def pin_row_sample(orc):
    """Sampled rows reproduce the same rows of the full computation (the
    outlier set is still taken over all rows)."""
    X, W = _case(800, 30, 64, 20, n_dims=2)
    Wq, sw = orc.quantize_weight(W)
    full = orc.mixed_matmul(X, Wq, sw, W, 6.0)
    rows = np.array([29, 0, 7, 7, 13])
    r = orc.mixed_matmul(X, Wq, sw, W, 6.0, rows=rows)
    assert np.array_equal(r["idx"], full["idx"])
    for key in ("xq", "sx", "acc", "Y"):
        assert np.array_equal(r[key], full[key][rows]), key


ALL_PINS = [pin_f16_codec, pin_hand_example, pin_quant_ties, pin_tiny_scale, pin_detect, pin_compact,
            pin_tiny_config, pin_quant_invariants, pin_gemm, pin_tau_inf, pin_tau_zero,
            pin_error_bound, pin_metamorphic_scale, pin_permutation, pin_row_sample,
            pin_hand_memory_halved, pin_dequant_weight, pin_memory_halved_tau_zero,
            pin_memory_halved_exact_weight, pin_bf16_decode, pin_typed_weight_hand,
            pin_typed_weight_containers, pin_bf16_encode, pin_hand_bf16, pin_bf16_same_values]
