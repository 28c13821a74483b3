"""Plant plausible mistakes in a scratch copy of the oracle (CPU only) and check
that the pin battery catches every one of them.  The committed oracle is never
modified; each mutant is compiled into a temporary directory."""
import os

import pytest

import oracle
import oracle_pins as P

# (id, exact text in oracle.c, replacement)
MUTATIONS = [
    ("e4m3_mantissa_width", "double quantum = ldexp(1.0, ex - 3);", "double quantum = ldexp(1.0, ex - 2);"),
    ("e4m3_no_saturation", "if (r > 448.0) r = 448.0;", ""),
    ("e4m3_ties_away", "double r = rint(a / quantum) * quantum;\n    if (r > 448.0)",
     "double r = round(a / quantum) * quantum;\n    if (r > 448.0)"),
    ("e4m3_subnormal_range", "if (ex < -6) ex = -6;", "if (ex < -7) ex = -7;"),
    ("e4m3_negative_zero_lost", "uint8_t sign = signbit(y) ? 0x80 : 0x00;", "uint8_t sign = (y < 0) ? 0x80 : 0x00;"),
    ("mx_emax_off_by_one", "floor_log2(amax) - 8;", "floor_log2(amax) - 7;"),
    ("mx_no_low_clamp", "if (shared < -127) shared = -127;", "if (shared < -200) shared = -200;"),
    ("mx_inf_not_poisoning", "if (!is_finite_d(v[i])) return 0xFF;", "if (isnan(v[i])) return 0xFF;"),
    ("mx_scale_index_transposed", "s[m * nb + b] = c;", "s[b * M + m] = c;"),
    ("mx_dequant_scale_index", "s[m * nb + k / 32]", "s[m * nb + k % nb]"),
    ("bf16_no_subnormal_binade", "if (ex < -126) ex = -126;", ""),
    ("bf16_ties_away", "double r = rint(a / quantum) * quantum;   /* a/quantum is exact; rint = ties-to-even */",
     "double r = round(a / quantum) * quantum;"),
    ("e8m0_nan_code_finite", "if (code == 0xFF) return NAN;", ""),
    ("group_fnuz_max", "volatile float s = 448.0f / denom;", "volatile float s = 240.0f / denom;"),
    ("group_single_rounding", "volatile float p = f32_of_bf16(xbits) * s;",
     "volatile double p = (double)f32_of_bf16(xbits) * (double)s;"),
    ("group_col_layout_wrong", "else q[k * M + r] = c;", "else q[r * K + k] = c;"),
    ("group_start_not_advanced", "        start = end;\n    }", "    }"),
    ("group_decreasing_end_kept", "if (end < start) end = start;", ""),
    ("mm_block_scale_index", "e8m0[wsrow[k / 32]]", "e8m0[wsrow[k % KB]]"),
    ("mm_token_scale_row", "const uint8_t* xsrow = xs + r * KB;", "const uint8_t* xsrow = xs + (r / 2) * KB;"),
    ("mm_weight_group_ignored", "wq + ((int64_t)grp * N + n) * K;", "wq + ((int64_t)0 * N + n) * K;"),
    ("mm_weight_uses_token_scale", "double wv = e4m3[wrow[k]] * e8m0[wsrow[k / 32]];",
     "double wv = e4m3[wrow[k]] * e8m0[xsrow[k / 32]];"),
    ("mm_tail_rows_in_group0", "int32_t grp = -1;", "int32_t grp = 0;"),
    ("mm_group_end_inclusive", "if (r >= start && r < end) { grp = g; break; }",
     "if (r >= start && r <= end) { grp = g; break; }"),
    ("transpose_identity", "out[j * R + i] = in[i * C + j];", "out[i * C + j] = in[i * C + j];"),
    ("rceil_boundary_inclusive", "while (amax > 448.0 * ldexp(1.0, e)) ++e;", "while (amax >= 448.0 * ldexp(1.0, e)) ++e;"),
    ("rceil_wrong_max", "while (amax > 448.0 * ldexp(1.0, e)) ++e;", "while (amax > 480.0 * ldexp(1.0, e)) ++e;"),
    ("rceil_is_floor", "} else if (rule == 0) {", "} else if (rule >= 0) {"),
    ("rceil_floor_emax", "e = -8 + floor_log2(amax);", "e = -7 + floor_log2(amax);"),
    ("axis0_block_rows", "(a * 32 + i) * K + b;", "(a + i) * K + b;"),
    ("axis0_dequant_scale_row", "s[(m / 32) * K + k]", "s[(m % 32) * K + k]"),
    ("axis1_ex_dequant_scale", "s[m * (K / 32) + k / 32]", "s[m * (K / 32) + k % 32]"),
    ("group_pow2_rounds_up", "return ldexpf(1.0f, e - 1);", "return ldexpf(1.0f, e);"),
    ("group_pow2_ignored", "if (flags & 1) mult = group_pow2_floor(mult);", "if (flags & 4) mult = group_pow2_floor(mult);"),
    ("group_inverse_not_stored", "stored = (flags & 2) ? one / mult : mult;", "stored = mult;"),
    ("pack_not_stable", "for (int64_t p = 0; p < P; ++p) {\n            if (ids[p] != e) continue;",
     "for (int64_t p = P - 1; p >= 0; --p) {\n            if (ids[p] != e) continue;"),
    ("pack_scales_in_front", "oracle_mx_quantize(x + (p / topk) * K, 1, K, row, row + K);",
     "oracle_mx_quantize(x + (p / topk) * K, 1, K, row + K / 32, row);"),
    ("pack_token_index", "oracle_mx_quantize(x + (p / topk) * K, 1, K, row, row + K);",
     "oracle_mx_quantize(x + (p % M) * K, 1, K, row, row + K);"),
    ("pack_end_exclusive", "group_end[e] = (int32_t)r;", "group_end[e] = (int32_t)(r > 0 ? r - 1 : 0);"),
    ("group_codes_from_stored_scale", "oracle_group_encode_element(x[r * K + k], mult)",
     "oracle_group_encode_element(x[r * K + k], stored)"),
]


@pytest.mark.parametrize("mid,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, mid, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {mid} not found exactly once"
    mutant_c = os.path.join(tmp_path, "mutant.c")
    with open(mutant_c, "w") as f:
        f.write(src.replace(old, new))
    so = oracle.compile_source(mutant_c, os.path.join(tmp_path, "libmutant.so"))
    failed = P.run_battery(oracle.Oracle(so))
    assert failed, f"mutation {mid} was not caught by any pin"
