"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's C source,
builds the copy in a temporary directory, points the oracle wrapper at it and
runs the pins: at least one pin must fail.  The real oracle is never edited.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

from oracle import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "idx_oracle.c")

MUTANTS = {
    "relu-dropped": ("logit += (dot > 0.0 ? dot : 0.0) * (double)w_row[h];",
                     "logit += dot * (double)w_row[h];"),
    "q-transposed": ("dot += k[d] * q_row[(int64_t)h * D + d];",
                     "dot += k[d] * q_row[(int64_t)d * H + h];"),
    "fp8-bias-8": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                   "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8-no-subnormal": ("mag = ldexp((double)m, -9);", "mag = 0.0;"),
    "scale-magnitude-only": ("k[d] = oracle_e4m3_value(key_row[d]) * scale;",
                             "k[d] = oracle_e4m3_value(key_row[d]) * fabs(scale);"),
    "scale-big-endian": ("uint32_t bits = (uint32_t)p[0] | ((uint32_t)p[1] << 8) |",
                         "uint32_t bits = (uint32_t)p[3] | ((uint32_t)p[2] << 8) |"),
    "limit-off-by-one": ("if (entry >= limits[b])", "if (entry > limits[b])"),
    "ties-to-higher-column": ("return (a->c > b->c) - (a->c < b->c);",
                              "return (a->c < b->c) - (a->c > b->c);"),
    "nan-selectable": ("if (isnan(v) || v == -INFINITY)", "if (v == -INFINITY)"),
    "weights-dropped": ("logit += (dot > 0.0 ? dot : 0.0) * (double)w_row[h];",
                        "logit += (dot > 0.0 ? dot : 0.0);"),
    "encode-ties-to-lower": ("if (d < best_d || (d == best_d && (c & 1) == 0)) {",
                             "if (d < best_d) {"),
    "encode-sign-dropped": ("return (uint8_t)(best | (signbit(y) ? 0x80 : 0));",
                            "return (uint8_t)best;"),
    "encode-truncates": ("double d = fabs(oracle_e4m3_value((uint8_t)c) - a);",
                         "double d = oracle_e4m3_value((uint8_t)c) <= a ? a - oracle_e4m3_value((uint8_t)c) : INFINITY;"),
    "writer-scale-447": ("scale = amax / 448.0f;", "scale = amax / 447.0f;"),
    "writer-amax-ignores-negatives": ("if (fabsf(v) > amax)\n            amax = fabsf(v);",
                                      "if (v > amax)\n            amax = v;"),
    "writer-bad-slot-not-counted": ("            ++bad;\n", ""),
    "level1-max-is-min": ("                    if (x > s)\n", "                    if (x < s)\n"),
    "level1-mean-not-divided": ("s = sum / (float)L;", "s = sum;"),
    "level1-threshold-exclusive": ("if (s >= threshold)", "if (s > threshold)"),
    "level1-ties-to-higher-page": ("return (a->page > b->page) - (a->page < b->page);",
                                   "return (a->page < b->page) - (a->page > b->page);"),
    "level1-recent-off-by-one": ("if (p < n_sink || p >= P - n_recent)", "if (p < n_sink || p > P - n_recent)"),
    "level1-entries-past-limit": ("for (e = 0; e < hist; ++e) {", "for (e = 0; e < P * 64 && e < n_cols; ++e) {"),
    "level1-nothing-forced": ("                pr[p].rank = 2;\n", "                pr[p].rank = pr[p].density > 0;\n"),
    "q8-scale-ignored": ("qd[(int64_t)h * D + d] = oracle_e4m3_value(qrow[d]) * qs;",
                         "qd[(int64_t)h * D + d] = oracle_e4m3_value(qrow[d]);"),
    "q8-head-stride-wrong": ("const uint8_t *qrow = q8 + ((int64_t)b * H + h) * row_bytes;",
                             "const uint8_t *qrow = q8 + ((int64_t)b * H + h) * D;"),
    "level1-empty-pages-eligible": ("pr[p].rank = pr[p].density > 0 ? 1 : 0;", "pr[p].rank = 1;"),
    "block-row-stride-64": ("prow = pblk * block_size + s;", "prow = pblk * 64 + s % 64;"),
    "sigmoid-sign-flipped": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "sigmoid-half-slope": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(-0.5 * x));"),
    "chunk-entry-stride-64": ("e = chunk_ids[(int64_t)b * max_chunks + j] * block_size + s;",
                              "e = chunk_ids[(int64_t)b * max_chunks + j] * 64 + s;"),
    "mx-ties-to-larger": ("if (d < best_d || (d == best_d && (c & 1) == 0 && (best_c & 1) == 1)) {",
                          "if (d <= best_d) {"),
    "mx-ties-to-smaller": ("if (d < best_d || (d == best_d && (c & 1) == 0 && (best_c & 1) == 1)) {",
                           "if (d < best_d) {"),
    "mx-sign-dropped": ("return x < 0.0 ? -best : best;", "return best;"),
    "mx-exponent-ceil": ("e = (ex - 1) - 2;                    /* floor(log2(amax)) - 2 */",
                         "e = ex - 2;"),
    "mx-exponent-minus-3": ("e = (ex - 1) - 2;                    /* floor(log2(amax)) - 2 */",
                            "e = (ex - 1) - 3;"),
    "mx-no-low-clamp": ("    if (e < -127)\n        e = -127;\n", ""),
    "mx-key-not-rounded": ("        oracle_mxfp4_round(k, D, k);\n", ""),
    "mx-query-not-rounded": ("                    oracle_mxfp4_round(qd + (int64_t)h * D, D, qd + (int64_t)h * D);",
                             "                    (void)h;"),
    "mx-key-rounded-after-scale": ("            k[d] = oracle_e4m3_value(key_row[d]);\n        oracle_mxfp4_round(k, D, k);\n        for (d = 0; d < D; ++d)\n            k[d] = k[d] * scale;",
                                   "            k[d] = oracle_e4m3_value(key_row[d]) * scale;\n        oracle_mxfp4_round(k, D, k);"),
    "mx-blocks-of-16": ("        x = ldexp(1.0, oracle_mxfp4_exponent(amax));\n        for (i = 0; i < 32; ++i)",
                        "        x = ldexp(1.0, oracle_mxfp4_exponent(amax));\n        for (i = 0; i < 16; ++i)"),
}

PIN_TESTS = [
    lambda: pins.test_e4m3_all_bytes_match_torch_e4m3fn(),
    lambda: [pins.test_e4m3_closed_form_points(u, v) for u, v in
             [(0x38, 1.0), (0x01, 2.0 ** -9), (0x7E, 448.0)]],
    lambda: pins.test_scale_is_little_endian_fp32_after_head_dim((0, 0, 0, 0x3F), 0.5),
    pins.test_one_hot_closed_form,
    pins.test_relu_applies_per_head_before_weighting,
    pins.test_negative_scale_is_applied_before_relu,
    lambda: pins.test_integer_case_matches_numpy_matmul(0),
    pins.test_limits_mask_exactly_and_poison_never_leaks,
    lambda: pins.test_topk_matches_brute_force_with_ties(0),
    pins.test_e4m3_encode_matches_torch_cast_at_values_and_midpoints,
    pins.test_e4m3_encode_ties_and_saturation_closed_form,
    pins.test_quantize_row_with_amax_448_is_the_plain_cast,
    lambda: pins.test_quantize_row_scale_is_rounded_amax_over_448_and_error_is_half_a_step(0),
    pins.test_write_keys_places_rows_and_skips_padding_and_bad_slots,
    pins.test_level1_densest_pages_closed_form,
    pins.test_level1_threshold_is_inclusive_and_mean_rounds_in_binary32,
    pins.test_level1_history_bounds,
    lambda: pins.test_level1_matches_brute_force(0),
    pins.test_level1_layer_order_and_single_layer,
    pins.test_quantised_query_equals_plain_query_when_quantisation_is_exact,
    pins.test_quantised_query_closed_form,
    pins.test_16_row_blocks_are_a_relabelling,
    pins.test_16_row_chunk_lists_read_the_listed_small_blocks,
    pins.test_sigmoid_values_closed_form,
    pins.test_e2m1_round_closed_form,
    pins.test_mxfp4_exponent_closed_form,
    pins.test_mxfp4_round_worked_blocks,
    pins.test_mxfp4_round_is_identity_on_the_grid,
    pins.test_mxfp4_scores_equal_plain_scores_when_rounding_is_exact,
    pins.test_mxfp4_score_closed_form,
]


def _build_mutant(old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = os.path.join(tmp, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmp, "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", path,
                    "-o", so, "-lm"], check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(old, new, tmp)
        real = oracle._load()
        monkeypatch.setattr(oracle, "_LIB", so)
        monkeypatch.setattr(oracle, "_lib", None)
        try:
            oracle._load()
            caught = []
            for t in PIN_TESTS:
                try:
                    t()
                except AssertionError:
                    caught.append(t)
            assert caught, f"mutant {name} passed every pin"
        finally:
            monkeypatch.setattr(oracle, "_lib", real)


def test_unmutated_oracle_passes_the_same_pins():
    for t in PIN_TESTS:
        t()
