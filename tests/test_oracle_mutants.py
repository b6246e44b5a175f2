"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/oracle.c, applies one plausible mistake (a dropped
term, a wrong index, a wrong sign, a wrong exponent bias, ...), builds the copy
with the same gcc flags into a temporary library, routes the oracle wrappers to
it and runs the pin tests of test_oracle_pins.py.  At least one pin must fail
for every mutant.  All of this runs on the CPU; nothing here touches the GPU
library.
"""
import pytest

import oracle
from tests import test_oracle_cast_pins as cast_pins
from tests import test_oracle_pins as pins
from tests import test_oracle_ue8m0_pins as ue8m0_pins
from tests import test_oracle_layout_pins as layout_pins
from tests import test_oracle_mqa_pins as mqa_pins

MUTANTS = {
    "exponent_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                      "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "subnormal_scale": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "nan_code": ("if (e == 15 && m == 7)", "if (e == 15 && m == 6)"),
    "dropped_accumulation": ("acc += s * p;                                 /* promotion",
                             "acc = s * p;                                 /* promotion"),
    "sfb_ignores_n_block": ("sfb[(n / KBLK) * KB + kb]", "sfb[kb]"),
    "sfb_transposed": ("sfb[(n / KBLK) * KB + kb]", "sfb[kb * ((N + KBLK - 1) / KBLK) + n / KBLK]"),
    "sfa_ignores_stride": ("double s = (double)sa_row[kb * sa_stride]", "double s = (double)sa_row[kb]"),
    "b_index_shifted": ("p += g_dec[a_row[k]] * g_dec[b_row[k]];",
                        "p += g_dec[a_row[k]] * g_dec[b_row[(k + 1) % K]];"),
    "c_sign": ("out[n] = acc + (c_row ? (double)c_row[n] : 0.0);",
               "out[n] = acc - (c_row ? (double)c_row[n] : 0.0);"),
    "block_sum_in_float": ("double p = 0.0;                               /* exact block sum */\n"
                           "            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)\n"
                           "                p += g_dec[a_row[k]] * g_dec[b_row[k]];",
                           "float p = 0.0f;                               /* exact block sum */\n"
                           "            for (int64_t k = kb * KBLK; k < (kb + 1) * KBLK; ++k)\n"
                           "                p += (float)(g_dec[a_row[k]] * g_dec[b_row[k]]);"),
    "scale_block_off_by_one": ("double s = (double)sa_row[kb * sa_stride]",
                               "double s = (double)sa_row[((kb + 1) % KB) * sa_stride]"),
    "contiguous_expert_zero": ("nt_row(a + r * K, sfa + r, M_tot, b + e * N * K, sfb + e * NB * KB,",
                               "nt_row(a + r * K, sfa + r, M_tot, b, sfb + e * NB * KB,"),
    "masked_off_by_one": ("if (r >= mm) {", "if (r > mm) {"),
    "masked_no_clamp": ("if (mm > M_max) mm = M_max;", "if (mm > M_max) mm = 1;"),
    "tn_sfb_row_only": ("(double)sfb[kb * N + n];", "(double)sfb[kb * N];"),
    "tn_group_start": ("for (int64_t kb = k0 / KBLK; kb < k1 / KBLK; ++kb) {",
                       "for (int64_t kb = 0; kb < k1 / KBLK; ++kb) {"),
    "tn_c_dropped": ("acc += s * p;\n            }\n            out[i * N + n] = acc + (c ? (double)c[(g * M + m) * N + n] : 0.0);",
                     "acc += s * p;\n            }\n            out[i * N + n] = acc;"),
    "kgu_c_dropped": ("ue8m0_scale(sfb + (w0 + j / 4) * N, N, n, j % 4) * p;\n            }\n            out[i * N + n] = acc + (c ? (double)c[(g * M + m) * N + n] : 0.0);",
                      "ue8m0_scale(sfb + (w0 + j / 4) * N, N, n, j % 4) * p;\n            }\n            out[i * N + n] = acc;"),
    # FP8 casting
    "cast_fnuz_max": ("float s = amax / 448.0f;", "float s = amax / 240.0f;"),
    "cast_ties_away": ("code = (lo % 2 == 0) ? lo : hi;", "code = hi;"),
    "cast_truncates": ("if (below < above)", "if (below < above || 1)"),
    "cast_zero_unsigned": ("const uint8_t sign = signbit(y) ? 0x80 : 0x00;",
                           "const uint8_t sign = y < 0 ? 0x80 : 0x00;"),
    "cast_sf_row_major": ("sf[(g * KB + kb) * R + r] = s;", "sf[(g * R + r) * KB + kb] = s;"),
    "cast_multiply_by_reciprocal": ("float q = x / s;", "float q = x * (1.0f / s);"),
    "cast_pow2_rounds_down": ("s = (float)ldexp(1.0, e);", "s = (float)ldexp(1.0, e - 1);"),
    "cast_blocks_drop_tail_rows": ("const int64_t n1 = (nb + 1) * KBLK < N ? (nb + 1) * KBLK : N;",
                                   "const int64_t n1 = (nb + 1) * KBLK < N ? (nb + 1) * KBLK : N - 1;"),
    "ue8m0_bias": ("return e == 0xFF ? NAN : ldexp(1.0, e - 127);",
                   "return e == 0xFF ? NAN : ldexp(1.0, e - 128);"),
    "ue8m0_byte_order": ("const int e = (int)((w >> (8 * (kb % 4))) & 0xFF);",
                         "const int e = (int)((w >> (8 * (3 - kb % 4))) & 0xFF);"),
    "ue8m0_b_per_block": ("ue8m0_scale(sfb, N, n, kb)", "ue8m0_scale(sfb, N, (n / KBLK) * KBLK, kb)"),
    "ue8m0_pack_offset": ("const int e = x - 1 + 127;                /* s = 2^(x-1)",
                          "const int e = x + 127;                /* s = 2^(x-1)"),
    "kgu_pack_offset": ("const int e = x - 1 + 127;\n                    if", "const int e = x + 127;\n                    if"),
    "ue8m0_pack_broadcast": ("sf[(mn / KBLK) * KB + kb]", "sf[kb]"),
    "layout_a_ignores_storage": ("const uint8_t av = a_stored_mk ? a[m * K + k] : a[k * M + m];",
                                 "const uint8_t av = a[m * K + k];"),
    "layout_b_ignores_storage": ("const uint8_t bv = b_stored_nk ? b[n * K + k] : b[k * N + n];",
                                 "const uint8_t bv = b[k * N + n];"),
    "layout_sfa_transposed": ("acc += ((double)sfa[kb * M + m] * (double)sfb[kb * N + n]) * p;",
                              "acc += ((double)sfa[m * KB + kb] * (double)sfb[kb * N + n]) * p;"),
    "layout_sfb_transposed": ("acc += ((double)sfa[kb * M + m] * (double)sfb[kb * N + n]) * p;",
                              "acc += ((double)sfa[kb * M + m] * (double)sfb[n * KB + kb]) * p;"),
    "layout_drops_c": ("(double)sfb[kb * N + n]) * p;\n            }\n            out[i * N + n] = acc + (c ? (double)c[m * N + n] : 0.0);",
                       "(double)sfb[kb * N + n]) * p;\n            }\n            out[i * N + n] = acc;"),
    "mqa_no_relu": ("logit += (s > 0.0 ? s : 0.0) * (double)w[i * H + h];",
                    "logit += s * (double)w[i * H + h];"),
    "mqa_sf_of_query": ("const double s = dot * (double)sf[j];", "const double s = dot * (double)sf[i % S_kv];"),
    "mqa_weight_index": ("logit += (s > 0.0 ? s : 0.0) * (double)w[i * H + h];",
                         "logit += (s > 0.0 ? s : 0.0) * (double)w[(h * S + i) % (S * H)];"),
    "mqa_range_inclusive": ("if (j < lo || j >= hi) {", "if (j < lo || j > hi) {"),
    "mqa_clean_zero": ("out[r * S_kv + j] = clean ? -INFINITY : NAN;", "out[r * S_kv + j] = clean ? 0.0 : NAN;"),
    "kgu_global_word_rows": ("acc += ue8m0_scale(sfa + (w0 + j / 4) * M, M, m, j % 4)",
                             "acc += ue8m0_scale(sfa + (kb / 4) * M, M, m, kb % 4)"),
    "kgu_b_word_rows": ("* ue8m0_scale(sfb + (w0 + j / 4) * N, N, n, j % 4) * p;",
                        "* ue8m0_scale(sfb + (j / 4) * N, N, n, j % 4) * p;"),
    "kgu_pack_drops_group_offset": ("const double s = sf[(kb0 + 4 * k4 + i) * MN + mn];",
                                    "const double s = sf[(4 * k4 + i) * MN + mn];"),
    "cast_zero_scale": ("if (amax == 0.0f)\n        return 1.0f;", "if (amax == 0.0f)\n        return 0.5f;"),
}


def _pin_suite():
    """The pins, as plain calls; returns the names of those that failed."""
    checks = [
        ("decode_all", pins.test_decode_all_codes_match_torch),
        ("decode_448", lambda: pins.test_decode_special_values(0x7E, 448.0)),
        ("decode_sub", lambda: pins.test_decode_special_values(0x01, 2.0 ** -9)),
        ("dense_exact_0", lambda: pins.test_dense_matches_exact_rationals(0, 3, 5, 128)),
        ("dense_exact_1", lambda: pins.test_dense_matches_exact_rationals(1, 4, 3, 256)),
        ("dense_exact_2", lambda: pins.test_dense_matches_exact_rationals(2, 2, 130, 384)),
        ("all_ones", lambda: pins.test_all_ones_gives_K(512)),
        ("pow2_scales", pins.test_power_of_two_scales_pick_the_right_blocks),
        ("one_hot_b", pins.test_one_hot_b_selects_a_column),
        ("one_hot_a", pins.test_one_hot_a_selects_a_row_of_b),
        ("f64_matmul", pins.test_dense_against_float64_matmul),
        ("golden", pins.test_hand_worked_golden),
        ("contiguous", pins.test_contiguous_matches_exact_rationals),
        ("masked", pins.test_masked_matches_exact_rationals_and_masks_rows),
        ("k_grouped", pins.test_k_grouped_matches_exact_rationals_with_empty_group),
        ("encode_codes", cast_pins.test_encode_round_trips_every_finite_code),
        ("encode_midpoints", cast_pins.test_encode_midpoints_tie_to_even_and_neighbours_round_to_nearest),
        ("encode_torch", cast_pins.test_encode_matches_torch_cast),
        ("cast_golden", cast_pins.test_cast_rows_hand_worked_golden),
        ("cast_nearest", cast_pins.test_cast_rows_is_the_nearest_code_of_the_fp32_quotient),
        ("cast_layout", cast_pins.test_cast_rows_scale_layout_and_block_max),
        ("cast_zero", cast_pins.test_cast_rows_zero_block),
        ("cast_gen_rows", cast_pins.test_cast_rows_matches_generator_quantiser),
        ("cast_pow2", cast_pins.test_cast_rows_pow2_scales),
        ("cast_gen_blocks", cast_pins.test_cast_blocks_matches_generator_quantiser_with_ragged_n),
        ("cast_blocks_nearest", cast_pins.test_cast_blocks_is_the_nearest_code_of_the_fp32_quotient),
        ("ue8m0_pack", ue8m0_pins.test_pack_matches_frexp_and_byte_order),
        ("ue8m0_broadcast", ue8m0_pins.test_pack_broadcasts_block_scales_to_rows),
        ("ue8m0_exact", lambda: ue8m0_pins.test_gemm_ue8m0_matches_exact_rationals(53, 4, 6, 640)),
        ("ue8m0_vs_fp32", ue8m0_pins.test_gemm_ue8m0_equals_fp32_scale_definition_on_block_constant_b),
        ("layout_nn_exact", lambda: layout_pins.test_layouts_match_exact_rationals("nn", 71, 4, 3, 384)),
        ("layout_tt_exact", lambda: layout_pins.test_layouts_match_exact_rationals("tt", 71, 4, 3, 384)),
        ("layout_tn_exact", lambda: layout_pins.test_layouts_match_exact_rationals("tn", 71, 4, 3, 384)),
        ("layout_transposes", layout_pins.test_nn_and_tt_are_nt_on_transposed_storage),
        ("layout_one_hot_nn", lambda: layout_pins.test_one_hot_b_selects_an_element_of_a("nn")),
        ("mqa_exact", mqa_pins.test_matches_exact_rationals),
        ("kgu_pack", ue8m0_pins.test_k_grouped_pack_layout_and_byte_order),
        ("kgu_vs_fp32", ue8m0_pins.test_k_grouped_ue8m0_equals_the_fp32_scale_definition),
        ("mqa_numpy", mqa_pins.test_matches_float64_numpy_formula),
        ("mqa_relu", mqa_pins.test_relu_zeroes_negative_logits_and_one_hot_weights),
        ("mqa_ranges", mqa_pins.test_ranges_clean_and_unclean_clamped_and_empty),
    ]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC_PATH) as f:
        return f.read()


def test_unmutated_copy_passes_every_pin(tmp_path, source):
    src = tmp_path / "oracle_copy.c"
    src.write_text(source)
    lib = oracle.compile_source(str(src), str(tmp_path / "liboracle_copy.so"))
    with oracle.use_library(lib):
        assert _pin_suite() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle.compile_source(str(src), str(tmp_path / f"liboracle_{name}.so"))
    with oracle.use_library(lib):
        failed = _pin_suite()
    assert failed, f"mutant {name} passed every pin"
