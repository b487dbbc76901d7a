"""Mutation check of the oracle's pins: each plausible mistake planted in a copy of
oracle.c (a dropped term, a wrong index, sign or operand) must make at least one pin
test fail. The mutants are built with gcc into a temporary directory and loaded by a
separate pytest process through EP_ORACLE_LIB; the real oracle is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("rne_no_tie_to_even", "u += 0x7fffu + kept_lsb;", "u += 0x7fffu;"),
    ("rne_truncates", "u += 0x7fffu + kept_lsb;", "u += 0u * kept_lsb;"),
    ("rne_rounds_half_up", "u += 0x7fffu + kept_lsb;", "u += 0x8000u + 0u * kept_lsb;"),
    ("rank_by_modulo", "row[e / experts_per_rank] = 1;", "row[e % R] = 1;"),
    ("masked_id_counted_bad", "            if (e == -1)\n                continue;\n            if (e < -1 || e >= E) {",
     "            if (e < 0 || e >= E) {"),
    ("bad_id_no_flag", "                flag = 1;\n", "                flag = 0;\n"),
    ("rank_count_per_slot", "        for (int r = 0; r < R; ++r)\n            if (row[r])\n                count_r[r] += 1;",
     "        for (int j = 0; j < k; ++j)\n            if (topk_idx[t * k + j] >= 0 && topk_idx[t * k + j] < E)\n                count_r[topk_idx[t * k + j] / experts_per_rank] += 1;"),
    ("node_count_per_rank", "            if (any)\n                count_n[n] += 1;",
     "            for (int q = 0; q < ranks_per_node; ++q)\n                if (row[n * ranks_per_node + q])\n                    count_n[n] += 1;\n            (void)any;"),
    ("inclusive_rank_offset", "rank_offset[r + 1] = rank_offset[r] + count_r[r];",
     "rank_offset[r + 1] = rank_offset[r] + count_r[r] + (r == 0 ? count_r[0] : 0);"),
    ("slot_off_by_one", "token_slot[t * R + r] = rank_offset[r] + filled[r];",
     "token_slot[t * R + r] = rank_offset[r] + filled[r] + (filled[r] > 0 ? 1 : 0);"),
    ("slot_rank_major_fill", "token_slot[t * R + r] = rank_offset[r] + filled[r];",
     "token_slot[t * R + r] = rank_offset[r] + (count_r[r] - 1 - filled[r]);"),
    ("expert_offset_shifted", "expert_offset[e + 1] = expert_offset[e] + count_e[e];",
     "expert_offset[e + 1] = expert_offset[e] + count_e[e > 0 ? e - 1 : 0];"),
    ("local_id_not_rebased", "local = e - (int64_t)r * experts_per_rank;", "local = e;"),
    ("weight_kept_off_rank", "recv_w[s * k + j] = local >= 0 ? w_row[j] : 0.0f;",
     "recv_w[s * k + j] = w_row[j];"),
    ("src_is_slot", "recv_src[s] = src;", "recv_src[s] = (int32_t)s;"),
    ("row_copy_short", "memcpy(recv_x + s * H, x + t * H, (size_t)H * sizeof(uint16_t));",
     "memcpy(recv_x + s * H, x + t * H, (size_t)(H - 1) * sizeof(uint16_t));"),
    ("restripe_uses_T_stride", "out[((int64_t)n * Tmax + t) * P + p] = prob[(t * N + n) * P + p];",
     "out[((int64_t)n * T + t) * P + p] = prob[(t * N + n) * P + p];"),
    ("restripe_transposed_source", "out[((int64_t)n * Tmax + t) * P + p] = prob[(t * N + n) * P + p];",
     "out[((int64_t)n * Tmax + t) * P + p] = prob[(n * T + t) * P + p];"),
    ("combine_skips_first_rank", "        for (int r = 0; r < R; ++r) {\n            int64_t s = token_slot[t * R + r];\n            if (s < 0)\n                continue;\n            if (s >= rows) {",
     "        for (int r = 1; r < R; ++r) {\n            int64_t s = token_slot[t * R + r];\n            if (s < 0)\n                continue;\n            if (s >= rows) {"),
    ("combine_rounds_each_add", "acc[h] = acc[h] + oracle_bf16_to_f32(partial[s * H + h]);",
     "acc[h] = oracle_bf16_to_f32(oracle_f32_to_bf16(acc[h] + oracle_bf16_to_f32(partial[s * H + h])));"),
    ("combine_subtracts", "acc[h] = acc[h] + oracle_bf16_to_f32(partial[s * H + h]);",
     "acc[h] = acc[h] - oracle_bf16_to_f32(partial[s * H + h]);"),
    ("e4m3_truncates", "float q = rintf(ldexpf(a, 3 - ex));", "float q = truncf(ldexpf(a, 3 - ex));"),
    ("e4m3_no_subnormal_range", "    if (ex < -6)\n        ex = -6;", "    if (ex < -9)\n        ex = -9;"),
    ("e4m3_bias_off_by_one", "return sign | (uint8_t)(((ex + 7) << 3) | ((int)q - 8));",
     "return sign | (uint8_t)(((ex + 8) << 3) | ((int)q - 8));"),
    ("fp8_scale_not_divided", "const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
     "const float scale = amax > 0.0f ? amax : 1.0f;"),
    ("fp8_inverse_scale_swapped", "const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;",
     "const float inv = amax > 0.0f ? amax / 448.0f : 1.0f;"),
    ("fp8_dispatch_scales_shifted", "memcpy(recv_scales + s * G, scales + t * G, (size_t)G * sizeof(float));",
     "memcpy(recv_scales + s * G, scales + (t > 0 ? t - 1 : 0) * G, (size_t)G * sizeof(float));"),
    ("expert_slot_unstable", "expert_slot[t * k + j] = offset[e] + filled[e];",
     "expert_slot[t * k + j] = offset[e] + (offset[e + 1] - offset[e] - 1 - filled[e]);"),
    ("expert_slot_offset_inclusive", "offset[e + 1] += offset[e];", "offset[e + 1] += offset[e] + (e == 0);"),
    ("permute_weight_first_slot", "perm_w[q] = topk_w[t * k + j];", "perm_w[q] = topk_w[t * k];"),
    ("node_slot_by_rank", "on[e / experts_per_node] = 1;", "on[(e / experts_per_node) % N] = 1; on[0] |= (N > 1 && e % 2);"),
    ("sparse_restripe_dense_row", "out[((int64_t)n * Tmax + s) * P + p] = prob[(t * N + n) * P + p];",
     "out[((int64_t)n * Tmax + t) * P + p] = prob[(t * N + n) * P + p];"),
    ("combine_truncates_output", "out[t * H + h] = oracle_f32_to_bf16(acc[h]);",
     "{ uint32_t bits; memcpy(&bits, &acc[h], 4); out[t * H + h] = (uint16_t)(bits >> 16); }"),
    ("hook_send_dense_row", "const int64_t q = (int64_t)n * Tmax + ns;\n            memcpy(stage_x + q * H",
     "const int64_t q = (int64_t)n * Tmax + t;\n            memcpy(stage_x + q * H"),
    ("hook_send_first_weight", "stage_w[q * k + j] = topk_w[t * k + j];", "stage_w[q * k + j] = topk_w[t * k];"),
    ("hook_recv_skips_first_row", "for (int64_t ns = 0; ns < count_n[n]; ++ns) {",
     "for (int64_t ns = 1; ns < count_n[n]; ++ns) {"),
    ("hook_recv_view_of_node_rank", "experts_per_rank, r, s, recv_idx, recv_w, recv_src);\n            }\n        }\n    }",
     "experts_per_rank, n * ranks_per_node, s, recv_idx, recv_w, recv_src);\n            }\n        }\n    }"),
    ("hook_combine_send_all_ranks",
     "for (int r = n * ranks_per_node; r < (n + 1) * ranks_per_node; ++r) {\n                const int64_t s = token_slot[t * R + r];\n                if (s < 0)\n                    continue;\n                if (s >= rows) {",
     "for (int r = 0; r < R; ++r) {\n                const int64_t s = token_slot[t * R + r];\n                if (s < 0)\n                    continue;\n                if (s >= rows) {"),
    ("hook_combine_recv_skips_node0", "sum[h] = 0.0f;\n        for (int n = 0; n < N; ++n) {",
     "sum[h] = 0.0f;\n        for (int n = 1; n < N; ++n) {"),
    ("hook_combine_send_scaled", "stage[q * H + h] = oracle_f32_to_bf16(sum[h]);",
     "stage[q * H + h] = oracle_f32_to_bf16(sum[h] * 1.0078125f);"),
    ("e4m3_decode_bias_off", "v = ldexpf((float)(8 + m), ef - 7 - 3);",
     "v = ldexpf((float)(8 + m), ef - 8 - 3);"),
    ("e4m3_decode_subnormal_scale", "v = ldexpf((float)m, -9);", "v = ldexpf((float)m, -10);"),
    ("e4m3_saturates_late", "if (a >= 464.0f)", "if (a >= 480.0f)"),
    ("fp8_amax_signed", "const float a = fabsf(oracle_bf16_to_f32(xg[c]));",
     "const float a = oracle_bf16_to_f32(xg[c]);"),
    ("fp8_zero_group_scale", "const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
     "const float scale = amax > 0.0f ? amax / 448.0f : 0.0f;"),
    ("permute_src_is_row", "perm_src[q] = (int32_t)t;", "perm_src[q] = (int32_t)q;"),
    ("node_slot_counts_unrouted", "node_slot[t * N + n] = on[n] ? filled[n]++ : -1;",
     "node_slot[t * N + n] = on[n] ? filled[n]++ : (filled[n]++, -1);"),
    ("node_slot_starts_at_one", "node_slot[t * N + n] = on[n] ? filled[n]++ : -1;",
     "node_slot[t * N + n] = on[n] ? ++filled[n] : -1;"),
    ("sparse_restripe_wrong_node_block",
     "out[((int64_t)n * Tmax + s) * P + p] = prob[(t * N + n) * P + p];",
     "out[((int64_t)((n + 1) % N) * Tmax + s) * P + p] = prob[(t * N + n) * P + p];"),
    ("node_count_first_rank_only", "if (row[n * ranks_per_node + q])",
     "if (row[n * ranks_per_node])"),
    ("permute_row_of_next_token", "memcpy(perm_x + q * H, x + t * H, (size_t)H * sizeof(uint16_t));",
     "memcpy(perm_x + q * H, x + ((t + 1) % T) * H, (size_t)H * sizeof(uint16_t));"),
]

# The quick pins (no exhaustive enumeration): enough to kill every mutant above.
PIN_ARGS = ["tests/test_oracle_layout.py", "tests/test_oracle_dispatch.py",
            "tests/test_oracle_fp8.py", "tests/test_oracle_permute.py",
            "tests/test_oracle_sparse.py", "tests/test_oracle_hook.py",
            "tests/test_oracle_restripe.py", "tests/test_oracle_combine.py",
            "tests/test_golden_pages.py", "-x", "-q", "-p", "no:cacheprovider",
            "-k", "not exhaustive"]


def test_every_mutation_appears_in_the_source():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    mutated = src.replace(old, new)
    assert mutated != src
    (tmp_path / "oracle.c").write_text(mutated)
    (tmp_path / "oracle.h").write_text(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-shared", "-fPIC",
                    str(tmp_path / "oracle.c"), "-o", str(lib)], check=True)
    env = dict(os.environ, EP_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_ARGS], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"
