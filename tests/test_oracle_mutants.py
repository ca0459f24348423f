"""Each plausible mistake planted in a copy of the oracle must be caught by
at least one pin.  The mutants are compiled from edited copies of oracle.c
into a temporary directory; the committed oracle is never touched.  CPU only."""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("threshold_strict", "fabsf(h_f32(ht, X[t * K + k])) >= tau", "fabsf(h_f32(ht, X[t * K + k])) > tau"),
    ("threshold_signed", "fabsf(h_f32(ht, X[t * K + k])) >= tau", "h_f32(ht, X[t * K + k]) >= tau"),
    ("round_half_away", "float q = rintf(p);", "float q = roundf(p);"),
    ("round_truncate", "float q = rintf(p);", "float q = truncf(p);"),
    ("range_128", "frexp(127.0 / (double)s, &e)", "frexp(128.0 / (double)s, &e)"),
    ("reciprocal_overflows", "double r = ldexp((double)(float)m, e);", "double r = (double)(127.0f / s);"),
    ("reciprocal_unrounded", "double r = ldexp((double)(float)m, e);", "double r = ldexp(m, e);"),
    ("product_unrounded", "float p = (float)((double)x * r);             /* exact 48-bit product, rounded to fp32 once */\n    float q = rintf(p);",
     "double p = (double)x * r;\n    float q = (float)rint(p);"),
    ("row_scale_includes_outliers", "if (flag[k]) continue;", ";"),
    ("outlier_column_kept", "flag[k] ? 0 : quant_one", "0 ? 0 : quant_one"),
    ("drop_16bit_part", "double y = y8 + y16;", "double y = y8;"),
    ("dequant_wrong_constant", "/ 16129.0", "/ 16384.0"),
    ("dequant_one_scale", "(double)c->sx[m] * (double)c->sw[n]", "(double)c->sx[m] * (double)c->sw[0]"),
    ("int32_wraparound", "int64_t s = 0;\n            for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)b[k];\n            if (s > INT32_MAX",
     "int32_t s = 0;\n            for (int64_t k = 0; k < c->K; ++k) s += (int32_t)a[k] * (int32_t)b[k];\n            if (s > INT32_MAX"),
    ("compact_reversed", "idx[o++] = (int32_t)k;", "idx[o++] = (int32_t)(K - 1 - k);"),
    ("f16_ties_away", "(frac == 0.5 && fmod(fl, 2.0) != 0.0)", "(frac == 0.5)"),
    ("weight_scale_first_rows", "for (int64_t k = 0; k < c->K; ++k) {\n            float a = fabsf(w_value(c, k * c->N + n));",
     "for (int64_t k = 0; k < c->K / 2; ++k) {\n            float a = fabsf(w_value(c, k * c->N + n));"),
    ("outlier_value_from_wrong_row", "h_decode(c->ht, c->X[t * c->K + k]) * h_decode(c->ht, w)",
     "h_decode(c->ht, c->X[k]) * h_decode(c->ht, w)"),
    ("recovered_weight_unrounded", "y16 += h_decode(c->ht, c->X[t * c->K + k]) * h_decode(c->ht, w);",
     "y16 += h_decode(c->ht, c->X[t * c->K + k]) * (c->W16 ? h_decode(c->ht, w) : (double)((float)c->Wq[n * c->K + k] * (c->sw[n] / 127.0f)));"),
    ("recovered_weight_128", "const float d = sw / 127.0f;", "const float d = sw / 128.0f;"),
    ("bf16_decode_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("f32_weight_read_as_f16", "if (c->type == 2) return ((const float*)c->W)[i];",
     "if (c->type == 3) return ((const float*)c->W)[i];"),
    ("f32_weight_rounded_to_f16", "if (c->type == 2) return ((const float*)c->W)[i];",
     "if (c->type == 2) return oh_f32(oh_encode((double)((const float*)c->W)[i]));"),
    ("recovered_weight_transposed", "oracle_dequant_weight_h(c->Wq[n * c->K + k], c->sw[n], c->ht)",
     "oracle_dequant_weight_h(c->Wq[(k * c->N + n) % (c->N * c->K)], c->sw[n], c->ht)"),
    ("recovered_weight_ignored", ": oracle_dequant_weight_h(c->Wq[n * c->K + k], c->sw[n], c->ht);",
     ": (uint16_t)0;"),
    ("bf16_output_rounded_as_fp16", "c->Y[m * c->N + n] = h_encode(c->ht, y);",
     "c->Y[m * c->N + n] = h_encode(0, y);"),
    ("bf16_encode_ties_away", "double n = fl;\n    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;\n    float r",
     "double n = fl;\n    if (frac >= 0.5) n = fl + 1.0;\n    float r"),
    ("bf16_input_read_as_fp16", "static float h_f32(int ht, uint16_t b) { return (float)h_decode(ht, b); }",
     "static float h_f32(int ht, uint16_t b) { (void)ht; return (float)oh_decode(b); }"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in oracle.c"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / f"liboracle_{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, OverflowError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
