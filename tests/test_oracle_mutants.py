"""Planted mistakes in the oracle must fail its pins (no GPU).

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a dropped
term, a wrong index, a wrong sign, a wrong rounding rule, lost stability),
built with gcc into a temporary directory.  The full pin suite runs against
it in a child process (so a mutant that crashes cannot take the test runner
down); the mutant is "caught" when that process fails.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "count_ignores_padding": ("off += round_up(count[e], row_align);", "off += count[e];"),
    "token_index_mod": ("input_perm[r] = (int32_t)(i / k);", "input_perm[r] = (int32_t)(i % k);"),
    "pick_instead_of_token": ("input_perm[r] = (int32_t)(i / k);", "input_perm[r] = (int32_t)i;"),
    "blockscale_uses_row_align": ("bs += round_up(count[e], bs_align);",
                                  "bs += round_up(count[e], row_align);"),
    "segment_right_aligned": ("cursor[e] = off;",
                              "cursor[e] = off + round_up(count[e], row_align) - count[e];"),
    "unstable_reverse_within_expert": (
        "int64_t r = cursor[e]++;",
        "int64_t seen = cursor[e]++ - expert_offsets[e]; "
        "int64_t r = expert_offsets[e] + count[e] - 1 - seen;"),
    "combine_drops_accumulator": ("acc = fmaf(v, w, acc);", "acc = fmaf(v, w, 0.0f);"),
    "combine_wrong_sign": ("acc = fmaf(v, w, acc);", "acc = fmaf(v, -w, acc);"),
    "combine_unfused": ("acc = fmaf(v, w, acc);", "acc = (float)(v * w) + acc;"),
    "factor_index_t_plus_j": ("load_elem(factors, f_dtype, t * k + j)",
                              "load_elem(factors, f_dtype, t + j)"),
    "combine_reads_transposed_column": ("load_elem(y, y_dtype, r * H + h)",
                                        "load_elem(y, y_dtype, r * H + (H - 1 - h))"),
    "bf16_ties_away_from_zero": ("if (rest > 0x8000u || (rest == 0x8000u && (t & 1u)))",
                                 "if (rest >= 0x8000u)"),
    "bf16_truncates": ("t += 1;", "t += 0;"),
    "bf16_nan_not_quieted": ("if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);",
                             "if (isnan(f)) return (uint16_t)(u >> 16);"),
    "f16_subnormal_scale": ("float q = rintf(a * 0x1p24f);", "float q = rintf(a * 0x1p23f);"),
    "f16_bias_off_by_one": ("(((ex + 15) << 10)", "(((ex + 14) << 10)"),
    "f16_widen_bias": ("v = ldexpf((float)(1024 + fr), ex - 25);",
                       "v = ldexpf((float)(1024 + fr), ex - 24);"),
    "problem_sizes2_swaps_n_k": ("ps2[3 * e + 1] = g2_n; ps2[3 * e + 2] = g2_k;",
                                 "ps2[3 * e + 1] = g2_k; ps2[3 * e + 2] = g2_n;"),
    "problem_sizes1_takes_gemm2": ("ps1[3 * e + 1] = g1_n; ps1[3 * e + 2] = g1_k;",
                                   "ps1[3 * e + 1] = g2_n; ps1[3 * e + 2] = g2_k;"),
    "unused_rows_zero": ("for (int64_t r = 0; r < r_max; ++r) input_perm[r] = -1;",
                         "for (int64_t r = 0; r < r_max; ++r) input_perm[r] = 0;"),
    "ids_shifted_by_one": (
        "        int64_t e = read_id(ids, id_bytes, i);\n        if (e >= 0 && e < E) count[e] += 1;",
        "        int64_t e = read_id(ids, id_bytes, i) - 1;\n        if (e >= 0 && e < E) count[e] += 1;"),
    "f16_widen_drops_sign": ("    return sign ? -v : v;\n}", "    return sign > 1 ? -v : v;\n}"),
    "f16_widen_subnormal_scale": ("v = ldexpf((float)fr, -24);", "v = ldexpf((float)fr, -25);"),
    "f16_widen_inf_as_nan": ("v = fr ? NAN : INFINITY;", "v = NAN;"),
    "weights_read_as_y_dtype": ("float w = factors ? load_elem(factors, f_dtype, t * k + j) : 1.0f;",
                                "float w = factors ? load_elem(factors, y_dtype, t * k + j) : 1.0f;"),
    "absent_weights_zero": ("float w = factors ? load_elem(factors, f_dtype, t * k + j) : 1.0f;",
                            "float w = factors ? load_elem(factors, f_dtype, t * k + j) : 0.0f;"),
    "f16_output_rounded_as_bf16": ("    case OR_F16: ((uint16_t*)base)[idx] = f32_to_f16(v); break;",
                                   "    case OR_F16: ((uint16_t*)base)[idx] = f32_to_bf16(v); break;"),
    "shuffle_accepts_last_plus_one": ("if (s < 0 || s >= n_src) continue;",
                                      "if (s < 0 || s > n_src) continue;"),
    "invalid_id_kept_as_expert0": ("output_perm[i] = -1;\n",
                                   "output_perm[i] = 0;\n"),
    "memset_needs_all_picks": ("if (expanded_to_permuted[t * k + j] >= 0) any = 1;",
                               "if (expanded_to_permuted[t * k + j] >= 0) any = 1; else { any = 0; break; }"),
    "sort_limit_is_segment_end": ("tile_limit[q] = (int32_t)(first[g] + count[g]);",
                                  "tile_limit[q] = (int32_t)first[g + 1];"),
    "sort_rows_hold_tokens": ("permuted_to_expanded[r] = (int32_t)i;",
                              "permuted_to_expanded[r] = (int32_t)(i / k);"),
    "sort_tile_count_off_by_one": ("*num_tiles = (int32_t)(total / tile);",
                                   "*num_tiles = (int32_t)((total + tile) / tile);"),
    "sort_window_ignores_offset": ("        int64_t g = read_id(ids, id_bytes, i) - local_offset;\n        if (g >= 0 && g < num_local) count[g] += 1;",
                                   "        int64_t g = read_id(ids, id_bytes, i);\n        if (g >= 0 && g < num_local) count[g] += 1;"),
    "e4m3_bias_off_by_one": ("uint8_t code = (uint8_t)(((ex + 7) << 3) | ((int)q - 8));",
                             "uint8_t code = (uint8_t)(((ex + 8) << 3) | ((int)q - 8));"),
    "e4m3_subnormal_scale": ("float q = rintf(a * 0x1p9f);", "float q = rintf(a * 0x1p8f);"),
    "fp8_scale_uses_240": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                           "float scale = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    "fp8_amax_keeps_nan": ("                if (v > amax) amax = v;",
                           "                if (!(v <= amax)) amax = v;"),
    "fp8_group_amax_first_only": ("                if (v > amax) amax = v;",
                                  "                if (e == 0) amax = v;"),
    "blockscale_from_padded_counts": ("bs += round_up(count[e], bs_align);",
                                      "bs += round_up(round_up(count[e], row_align), bs_align);"),
    "problem_size_is_padded": ("ps1[3 * e] = (int32_t)count[e];",
                               "ps1[3 * e] = (int32_t)round_up(count[e], row_align);"),
    "combine_starts_from_negative_zero": ("float acc = 0.0f;", "float acc = -0.0f;"),
    "combine_reverse_pick_order": (
        "            for (int32_t j = 0; j < k; ++j) {\n                int64_t r = perm[t * k + j];",
        "            for (int32_t j = k - 1; j >= 0; --j) {\n                int64_t r = perm[t * k + j];"),
    "f16_ties_away_from_zero": ("float q = rintf(ldexpf(a, 10 - ex));",
                                "float q = roundf(ldexpf(a, 10 - ex));"),
    "e4m3_ties_away_from_zero": ("float q = rintf(ldexpf(a, 3 - ex));",
                                 "float q = roundf(ldexpf(a, 3 - ex));"),
    "fp8_multiplies_by_reciprocal": (
        "q[t * H + g * block + e] = f32_to_e4m3(bf16_to_f32(xs[e]) / scale);",
        "q[t * H + g * block + e] = f32_to_e4m3(bf16_to_f32(xs[e]) * (1.0f / scale));"),
    "padding_zeroes_rows_of_token0": ("if (input_perm[r] < 0) memset(",
                                      "if (input_perm[r] <= 0) memset("),
    "sort_tiles_round_down": ("first[g + 1] = first[g] + (count[g] + tile - 1) / tile * tile;",
                              "first[g + 1] = first[g] + count[g] / tile * tile;"),
    "sort_unused_tiles_group_zero": (
        "for (int64_t q = 0; q < max_tiles; ++q) { tile_group[q] = -1; tile_limit[q] = -1; }",
        "for (int64_t q = 0; q < max_tiles; ++q) { tile_group[q] = 0; tile_limit[q] = -1; }"),
    "sort_first_tile_skipped": ("for (int64_t q = first[g] / tile; q < first[g + 1] / tile; ++q) {",
                                "for (int64_t q = first[g] / tile + 1; q < first[g + 1] / tile; ++q) {"),
    "sort_group_is_expert_id": ("tile_group[q] = g;", "tile_group[q] = g + local_offset;"),
    "sort_unstable_within_group": ("int64_t r = next[g]++;",
                                   "int64_t r = first[g] + count[g] - 1 - (next[g]++ - first[g]);"),
    "memset_ignores_pick_0": ("for (int32_t j = 0; j < k; ++j)\n            if (expanded_to_permuted",
                              "for (int32_t j = 1; j < k; ++j)\n            if (expanded_to_permuted"),
    "padding_zeroes_valid_rows": ("if (input_perm[r] < 0) memset(", "if (input_perm[r] >= 0) memset("),
    "fp8_zero_group_scale_zero": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                                  "float scale = amax > 0.0f ? amax / 448.0f : 0.0f;"),
    "padding_ignores_total": ("int64_t limit = expert_offsets ? expert_offsets[E] : n_rows;",
                              "int64_t limit = n_rows;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} is not unique in oracle.c"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = oracle.build(out_path=str(tmp_path / "liboracle_mutant.so"), src_path=str(mutant_c))
    env = dict(os.environ, PYTHONPATH=ROOT)
    proc = subprocess.run([sys.executable, "-c",
                           f"import tests.oracle_pins as p; p.run_all({lib!r})"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """The same harness accepts the real oracle (so a failure above is the
    mutation, not the harness)."""
    lib = oracle.build(out_path=str(tmp_path / "liboracle_copy.so"))
    env = dict(os.environ, PYTHONPATH=ROOT)
    proc = subprocess.run([sys.executable, "-c",
                           f"import tests.oracle_pins as p; p.run_all({lib!r})"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr[-2000:]
