"""The pins catch planted mistakes: each case copies the oracle's C source,
plants one plausible mistake (a wrong divisor, tie rule, operand, order,
sign, guard or index), builds the copy, and runs a fast battery of the pins
of this suite against it. Every mutant must fail at least one pin, and the
unmodified copy must pass them all. The mutants live in a temporary
directory; the oracle itself is never modified.
"""
import itertools
import os
import re
import shutil
import pytest

import oracle
import test_oracle_blocks as blocks
import test_oracle_bruteforce as brute
import test_oracle_formats as formats
import test_oracle_invariants as inv

SRC = os.path.join(os.path.dirname(oracle.__file__), "fos_oracle.c")

# (name, regex, replacement): each regex must match the source at least once;
# a mutation applies to the first match only (the quantizer's own code comes
# before the decode and grouped helpers that reuse some of its lines)
MUTATIONS = [
    ("map-to-4 divisor 3", r"(encode_candidate\(xb, nrows, a, )4\.0f(, S_enc, S_dec, cfg, 1, &c4\);\n        /\* keep)",
     r"\g<1>3.0f\g<2>"),
    ("ties keep map-to-4", r"if \(c4\.err < c6\.err\)", "if (c4.err <= c6.err)"),
    ("decode multiplier uses S_enc", r"float D = sigma \* S_dec;", "float D = sigma * S_enc;"),
    ("decode multiplier divides", r"float D = sigma \* S_dec;", "float D = sigma / S_enc;"),
    ("block scale order of operations", r"float t = \(a / c\) \* S_enc;", "float t = a * (S_enc / c);"),
    ("FP16-error mode ignored", r"if \(cfg->err_prec == ORC_ERR_FP16\) ref =", "if (0) ref ="),
    ("MAE and MSE swapped", r"\? fabsf\(e\) : e \* e", "? e * e : fabsf(e)"),
    ("tree strides reversed", r"for \(int stride = 8; stride >= 1; stride /= 2\)",
     "for (int stride = 1; stride <= 8; stride *= 2)"),
    ("sequential order reversed", r"float s = u\[0\];\n    for \(int i = 1; i < 16; i\+\+\) s = s \+ u\[i\];",
     "float s = u[15];\n    for (int i = 14; i >= 0; i--) s = s + u[i];"),
    ("16x16 rows summed sequentially", r"out->err = oracle_tree16\(rows\);", "out->err = oracle_seq16(rows);"),
    ("E2M1 ties to the odd code",
     r"(oracle_e2m1_value\(c\)\);\n        if \(d < best_d \|\| \(d == best_d && \(c & 1\) == )0", r"\g<1>1"),
    ("E4M3 ties to the odd code",
     r"(oracle_e4m3_value\(c\)\);\n        if \(d < best_d \|\| \(d == best_d && \(c & 1\) == )0", r"\g<1>1"),
    ("E4M3 saturates one code low", r"if \(t >= 448\.0f\) return 0x7E;", "if (t >= 448.0f) return 0x7D;"),
    ("NaN element encodes to 0", r"if \(isnan\(v\)\) return 0x7;", "if (isnan(v)) return 0x0;"),
    ("global scale maps the amax to 4", r"float s = \(6\.0f \* \(float\)bound\) / A;",
     "float s = (4.0f * (float)bound) / A;"),
    ("no zero-amax guard", r"if \(!\(A > 0\.0f\) \|\| isinf\(A\)\) return 1\.0f;", "if (isinf(A)) return 1.0f;"),
    ("S_dec not the reciprocal", r"float S_dec = 1\.0f / S_enc;", "float S_dec = S_enc;"),
    ("nibbles swapped", r"\(uint8_t\)\(\(q\[16 \* i \+ 2 \* j\] & 0xF\) \| \(\(q\[16 \* i \+ 2 \* j \+ 1\] & 0xF\) << 4\)\)",
     "(uint8_t)((q[16 * i + 2 * j + 1] & 0xF) | ((q[16 * i + 2 * j] & 0xF) << 4))"),
    ("amax keeps NaN", r"if \(isnan\(x\)\) return acc;", "if (isnan(x)) return x;"),
    ("amax without absolute value", r"float m = fabsf\(x\);", "float m = x;"),
    ("per-row amax indexed by tensor", r"\? amax\[0\] : amax\[r0\];", "? amax[0] : amax[0];"),
    ("grouped padding not cleared", r"memset\(codes \+ M \* \(K / 2\), 0,", "memset(codes + M * (K / 2), 1,"),
    ("binary16 rounding truncates", r"return nearbyint\(a / q\) \* q;", "return trunc(a / q) * q;"),
    ("per-row dequantize reads the first S_dec", r"\? sdec\[0\] : sdec\[r\];", "? sdec[0] : sdec[0];"),
    ("16x16 decoded values all go to the tile's first row",
     r"xhat_out\[r \* K \+ cb \* 16 \+ j\] = xhat\[16 \* i \+ j\]",
     "xhat_out[r0 * K + cb * 16 + j] = xhat[16 * i + j]"),
    ("fp32 outputs rounded through bf16", r"\(\(float\*\)y\)\[idx\] = v;",
     "((float*)y)[idx] = oracle_bf16_bits_to_f32(oracle_f32_to_bf16_rne(v));"),
]


def _battery(orc):
    """A fast subset of the pins, each called with the oracle under test."""
    for blk, key, metric in (p.values for p in blocks._cases()):
        blocks.test_hand_block(orc, blk, key, metric)
    formats.test_e2m1_grid_matches_ocp(orc)
    formats.test_e2m1_hand_thresholds(orc)
    formats.test_e2m1_specials(orc)
    formats.test_e4m3_matches_torch_cast(orc)
    formats.test_e4m3_saturation_and_zero(orc)
    formats.test_f16_rounding_matches_numpy(orc)
    formats.test_tree16_exact_value(orc)
    formats.test_seq16_exact_values(orc)
    for A, B, want in [(2688.0, 448, 1.0), (3.0, 448, 896.0), (0.0, 448, 1.0), (float("nan"), 256, 1.0)]:
        formats.test_global_encode_scale_closed_forms(orc, A, B, want)
    formats.test_global_decode_scale_is_reciprocal(orc)
    for dtype, family, block, gran, bound in [("bf16", "normal", "1x16", "tensor", 448),
                                              ("fp32", "outlier", "1x16", "row", 256),
                                              ("bf16", "special", "16x16", "row", 448),
                                              ("fp16", "weight", "16x16", "tensor", 256)]:
        brute.test_oracle_matches_exact_model(orc, dtype, family, block, gran, bound)
    brute.test_fp16_error_mode_exercised(orc, "mse", "fp16")
    brute.test_specials_match_exact_model(orc)
    brute.test_sequential_order_matches_exact_model(orc, "bf16", "outlier", "tensor")
    brute.test_block_scale_rounding_order(orc)
    for block, gran in itertools.product(("1x16", "16x16"), ("tensor", "row")):
        inv.test_selection_keeps_lower_recomputed_error(orc, "bf16", "outlier", block, gran)
    inv.test_zero_blocks(orc)
    inv.test_amax_modes(orc, "bf16")
    inv.test_qdq_is_dequantize_of_quantize(orc, "bf16", "4over6", "mse", "fp16", 448)
    inv.test_grouped_equals_per_group(orc)
    for out_dtype, gran in (("fp32", "row"), ("bf16", "tensor")):
        inv.test_dequantize_matches_independent_decode(orc, out_dtype, gran)
    for dtype, block, gran in (("fp32", "1x16", "tensor"), ("bf16", "16x16", "row"), ("fp16", "1x16", "row")):
        inv.test_qdq_every_dtype_block_and_granularity(orc, dtype, block, gran)


def _build(tmp_path, source, name):
    d = tmp_path / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "fos_oracle.h"), d / "fos_oracle.h")
    (d / "fos_oracle.c").write_text(source)
    return oracle.Oracle(oracle.build(force=True, out=str(d / "liboracle.so"), src=str(d / "fos_oracle.c")))


def test_unmodified_copy_passes_the_battery(tmp_path):
    _battery(_build(tmp_path, open(SRC).read(), "control"))


@pytest.mark.parametrize("name,pattern,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, pattern, repl):
    src = open(SRC).read()
    mutated, n = re.subn(pattern, repl, src, count=1)
    assert n >= 1, f"mutation '{name}' no longer matches the oracle source"
    orc = _build(tmp_path, mutated, "mutant")
    with pytest.raises((AssertionError, ValueError)):
        _battery(orc)
