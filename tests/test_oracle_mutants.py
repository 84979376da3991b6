"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source -- a flipped
tie rule, a dropped normalisation, swapped gate/up, a transposed weight, a
wrong index into the permutation, an unstable order, a wrong segment key --
builds it, routes the oracle module to that build, and runs the pin checks
of tests/test_oracle_pins.py.  At least one pin must fail for every mutant;
the unmodified source must pass them all.
"""
import os

import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = {
    "ties_to_higher_index": ("if (best < 0 || row[e] > row[best]) best = e;",
                             "if (best < 0 || row[e] >= row[best]) best = e;"),
    "weights_not_normalised": ("exp((double)row[sel[j]] - l0) / denom)", "exp((double)row[sel[j]] - l0))"),
    "weights_unshifted_slot": ("topk_w[t * k + j] = (float)(exp((double)row[sel[j]] - l0) / denom);",
                               "topk_w[t * k + j] = (float)(exp((double)row[sel[0]] - l0) / denom);"),
    "gate_up_swapped": ("double a = silu(g) * u;", "double a = silu(u) * g;"),
    "silu_sign": ("static double silu(double z) { return z / (1.0 + exp(-z)); }",
                  "static double silu(double z) { return z / (1.0 + exp(z)); }"),
    "no_bf16_rounding": ("hact[f] = act_fp8 ? (double)(float)a : ((dtype == ORC_BF16) ? orc_round_to_bf16(a) : a);",
                         "hact[f] = act_fp8 ? (double)(float)a : a;"),
    "bf16_rounds_to_zero": ("double r = nearbyint(scaled);", "double r = trunc(scaled);"),
    "down_transposed": ("for (int f = 0; f < F; ++f) acc += hact[f] * load_elem(w_down, dtype, wrow + f);",
                        "for (int f = 0; f < F; ++f) acc += hact[f] * load_elem(w_down, dtype, eHF + (int64_t)f * H + n);"),
    "gate_transposed": ("g += xrow[h] * load_elem(w_gate, dtype, wrow + h);",
                        "g += xrow[h] * load_elem(w_gate, dtype, eHF + (int64_t)h * F + f);"),
    "combine_slot0_weight": ("acc += (double)topk_w_sub[i * k + j] * y_rows[(i * k + j) * H + n];",
                             "acc += (double)topk_w_sub[i * k] * y_rows[(i * k + j) * H + n];"),
    "combine_drops_last_slot": ("for (int j = 0; j < k; ++j)\n        if (!kept",
                                "for (int j = 0; j + 1 < k; ++j)\n        if (!kept"),
    "unstable_permutation": ("for (int64_t f = 0; f < R; ++f)\n      if (seg_of(topk_idx, src_block, base, EL, k, f) == g)",
                             "for (int64_t f = R - 1; f >= 0; --f)\n      if (seg_of(topk_idx, src_block, base, EL, k, f) == g)"),
    "segment_key_unscaled": ("return s * EL + e;", "return s + e;"),
    "local_filter_ignores_base": ("int64_t e = (int64_t)topk_idx[f] - base;", "int64_t e = (int64_t)topk_idx[f];"),
    "local_filter_one_past": ("if (e < 0 || e >= EL) return -1;", "if (e < 0 || e > EL) return -1;"),
    "local_tail_not_cleared": ("for (; r < R; ++r) sorted_to_flat[r] = -1;", ""),
    "local_dropped_not_marked": ("for (int64_t f = 0; f < R; ++f) flat_to_sorted[f] = -1;",
                                 "for (int64_t f = 0; f < R; ++f) flat_to_sorted[f] = 0;"),
    "epilogue_ignores_residual": ("double v = acc[i] + (residual ? load_elem(residual, res_dtype, i) : 0.0);",
                                  "double v = acc[i];"),
    "epilogue_not_rounded": ("out[i] = (out_dtype == ORC_BF16) ? orc_round_to_bf16(v) : v;", "out[i] = v;"),
    "mx_scale_exponent_off_by_one": ("X = e - 1 - 8;", "X = e - 8;"),
    "mx_ties_to_odd": ("if (dh < dl || (dh == dl && (hi & 1) == 0)) lo = hi;",
                       "if (dh < dl || (dh == dl && (hi & 1) == 1)) lo = hi;"),
    "mx_rounds_down": ("if (dh < dl || (dh == dl && (hi & 1) == 0)) lo = hi;", ""),
    "mx_amax_skips_last": ("for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[i]));",
                           "for (int i = 0; i < 31; ++i) amax = fmax(amax, fabs(v[i]));"),
    "mx_down_scale_index": ("int64_t wrow = (int64_t)e * H + n;", "int64_t wrow = (int64_t)n;"),
    "mx_value_wrong_block": ("scales[mx_scale_index(r, c / 32, cols)]", "scales[mx_scale_index(r, c / 128, cols)]"),
    "mx_layout_transposed": ("return ((r / 32) * (cols / 128) + b / 4) * 128 + (r % 32) * 4 + (b % 4);",
                             "return ((r / 32) * (cols / 128) + b / 4) * 128 + (b % 4) * 32 + (r % 32);"),
    "mx_act_not_quantised": ("for (int i = 0; i < 32; ++i) hact[b * 32 + i] = ldexp(orc_e4m3_value(codes[i]), (int)sc - 127);",
                             ""),
    "epilogue_rounds_acc_first": ("double v = acc[i] + (residual ? load_elem(residual, res_dtype, i) : 0.0);",
                                  "double v = ((out_dtype == ORC_BF16) ? orc_round_to_bf16(acc[i]) : acc[i]) + "
                                  "(residual ? load_elem(residual, res_dtype, i) : 0.0);"),
    "expert_from_block_index": ("int e = (int)(g % E);", "int e = (int)((g / E) % E);"),
    "ffn_reads_flat_row": ("int64_t t = sorted_to_flat[r] / k;\n    double* xrow", "int64_t t = r / k;\n    double* xrow"),
    "dispatch_wrong_token": ("int64_t t = sorted_to_flat[r] / k;\n    memcpy", "int64_t t = sorted_to_flat[r] % k;\n    memcpy"),
    "inverse_not_inverted": ("flat_to_sorted[sorted_to_flat[q]] = (int32_t)q;", "flat_to_sorted[q] = sorted_to_flat[q];"),
    "dispatch_dropped_rows_not_zeroed": ("      memset((char*)x_perm + (size_t)r * row, 0, row);\n", ""),
    "offsets_inclusive": ("offsets[g + 1] = offsets[g] + counts[g];", "offsets[g + 1] = offsets[g] + counts[g] + (g == 0);"),
}


def _checks():
    """The pin checks, as callables that raise on failure."""
    return [
        ("bf16", pins.test_bf16_rounding_matches_torch),
        ("route_E8", lambda: pins.test_route_matches_python_sort(8, 2)),
        ("route_E64", lambda: pins.test_route_matches_python_sort(64, 4)),
        ("k2_closed_form", pins.test_route_weights_closed_form_k2),
        ("softmax", pins.test_route_weights_full_softmax_renormalised),
        ("k1", pins.test_route_k1_weight_is_exactly_one),
        ("segments_S1", lambda: pins.test_segments_and_permutation_brute_force(37, 8, 2, 1)),
        ("segments_S8", lambda: pins.test_segments_and_permutation_brute_force(96, 16, 8, 8)),
        ("dispatch", pins.test_dispatch_is_bitwise_row_copy),
        ("dispatch_held", lambda: pins.test_dispatch_with_held_experts_zero_fills_past_kept_pairs("bf16", 4, 4, 1)),
        ("dense_f32", lambda: pins.test_layer_matches_dense_brute_force("f32", 4, 2)),
        ("dense_bf16", lambda: pins.test_layer_matches_dense_brute_force("bf16", 6, 3)),
        ("dense_src_blocks", pins.test_layer_with_source_blocks_matches_dense),
        ("single_ffn", pins.test_top1_single_expert_is_one_dense_swiglu_ffn),
        ("local_segments", lambda: pins.test_local_segments_brute_force(60, 16, 4, 1, 4, 4)),
        ("local_segments_S4", lambda: pins.test_local_segments_brute_force(96, 32, 8, 4, 0, 8)),
        ("local_last_expert", lambda: pins.test_local_segments_brute_force(33, 16, 2, 1, 15, 1)),
        ("local_dense", lambda: pins.test_local_layer_matches_dense_partial("bf16", 16, 4, 12, 4)),
        ("local_partition", pins.test_local_partition_sums_to_full_layer),
        ("epilogue_hand", pins.test_epilogue_hand_values),
        ("epilogue_torch", pins.test_epilogue_bf16_matches_torch_rounding_of_f32_sums),
        ("e4m3_round", pins.test_e4m3_rounding_matches_torch_below_448),
        ("e4m3_clamp", pins.test_e4m3_rounding_clamps_to_448),
        ("mx_hand", pins.test_mx_block_hand_values),
        ("mx_round_trip", pins.test_mx_round_trip_within_half_a_step),
        ("mx_layout", pins.test_mx_scale_storage_layout),
        ("mx_layer", pins.test_mx_layer_matches_dense_quantised_evaluation),
    ]


def _failures():
    failed = []
    for name, fn in _checks():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_source_passes_every_check(workdir):
    path = oracle.build_variant(oracle.source_text(), os.path.join(workdir, "orc_clean.so"))
    with oracle.use_library(path):
        assert _failures() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(workdir, name):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation anchor not unique for {name}"
    path = oracle.build_variant(src.replace(old, new), os.path.join(workdir, f"orc_{name}.so"))
    with oracle.use_library(path):
        failed = _failures()
    assert failed, f"no pin caught the planted mistake {name}"
