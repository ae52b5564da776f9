"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, a transposed
index, a wrong rounding rule ...) in a copy of oracle.c on the CPU, builds
that copy in a temporary directory and runs the pin tests against it; the
pins must fail.  Slow (one pytest run per mistake): FP_SLOW_TESTS=1.
"""

import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

MUTATIONS = {
    "padding_not_zero": ("out[k] = 0;", "out[k] = 1;"),
    "padded_size_rounded_down": ("((t + world - 1) / world)", "((t) / world)"),
    "view_offset_in_flat_not_shard": ("buf_offset[i] = lo - (int64_t)rank * s;", "buf_offset[i] = lo - o;"),
    "view_tensor_offset_wrong": ("tensor_offset[i] = lo - o;", "tensor_offset[i] = lo - (int64_t)rank * s;"),
    "reduce_drops_rank_1": ("for (int32_t q = 1; q < world; ++q)\n            sum",
                            "for (int32_t q = 2; q < world; ++q)\n            sum"),
    "reduce_starts_from_plus_zero": ("float sum = or_bf16_to_f32(grads[0][i]);\n        for (int32_t q = 1;",
                                     "float sum = 0.0f;\n        for (int32_t q = 0;"),
    "reduce_wrong_rank_index": ("sum = sum + or_bf16_to_f32(grads[q][i]);",
                                "sum = sum + or_bf16_to_f32(grads[world - q][i]);"),
    "reduce_ignores_accumulate": ("float y = sum * scale;\n        if (accumulate)\n            acc[i] = acc[i] + y;",
                                  "float y = sum * scale;\n        if (accumulate)\n            acc[i] = y;"),
    "hybrid_ignores_accumulate": ("float y = total * scale;\n        if (accumulate)\n            acc[i] = acc[i] + y;",
                                  "float y = total * scale;\n        if (accumulate)\n            acc[i] = y;"),
    "reduce_sums_instead_of_mean": ("float y = sum * scale;", "float y = sum;"),
    "adamw_no_bias_correction_1": ("double m_hat = m / bias1;", "double m_hat = m;"),
    "adamw_no_bias_correction_2": ("double v_hat = v / bias2;", "double v_hat = v;"),
    "adamw_decay_sign": ("theta * (1.0 - lr * weight_decay)", "theta * (1.0 + lr * weight_decay)"),
    "adamw_eps_inside_sqrt": ("(sqrt(v_hat) + eps)", "sqrt(v_hat + eps)"),
    "adamw_beta_swapped": ("(1.0 - beta2) * g * g", "(1.0 - beta1) * g * g"),
    "adamw_update_sign": ("theta = theta - lr * m_hat", "theta = theta + lr * m_hat"),
    "adamw_no_decay": ("theta = theta * (1.0 - lr * weight_decay);\n", ""),
    "adamw_skip_ignored": ("if (skip)\n        return;", ""),
    "bf16_ties_away_from_zero": ("(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    "bf16_truncates": ("upper += 1u;", "upper += 0u;"),
    "unshard_transposed": ("full[(int64_t)q * shard + j] = shards[q][j];", "full[j * world + q] = shards[q][j];"),
    "memory_stage2_drops_grads": ("case 2: return 2.0 * psi + (2.0 * psi + k * psi) / n;",
                                  "case 2: return 2.0 * psi + (k * psi) / n;"),
    "memory_stage1_shards_grads": ("case 1: return 2.0 * psi + 2.0 * psi + k * psi / n;",
                                   "case 1: return 2.0 * psi + 2.0 * psi / n + k * psi / n;"),
    "overflow_check_misses_nan": ("if (!isfinite(acc[i]))", "if (isinf(acc[i]))"),
    "norm_squares_in_fp32": ("s = s + (double)acc[i] * (double)acc[i];", "s = s + (double)(acc[i] * acc[i]);"),
    "locate_offset_by_one": ("offset[j] = pos[j] - start;\n        } else", "offset[j] = pos[j] - start + 1;\n        } else"),
    "shard0_chunk_rounded_down": ("rows[i] = (d0 + world - 1) / world;", "rows[i] = d0 / world + (d0 % world ? 0 : 0);"),
    "shard0_padding_first": ("out[off[i] * elem_size + k] = in[k];", "out[off[i] * elem_size + (c[i] * r[i] - real) * elem_size + k] = in[k];"),
    "shard0_rank_offset_in_rows_not_elements": ("(int64_t)rank * c[i] * r[i] * elem_size;", "(int64_t)rank * c[i] * elem_size;"),
    "shard0_unpack_row_order": ("int64_t q = j / c[i], jj = j % c[i];", "int64_t q = j % world, jj = j / world;"),
    "shard0_row_length_wrong": ("for (int32_t k = 1; k < ndims[i]; ++k)", "for (int32_t k = 2; k < ndims[i]; ++k)"),
    "local_accumulate_overwrites": ("local[i] = accumulate ? local[i] + g : g;", "local[i] = g;"),
    "local_finish_drops_last_micro_batch": ("out[i] = or_f32_to_bf16(accumulate ? local[i] + g : g);",
                                            "out[i] = or_f32_to_bf16(accumulate ? local[i] : g);"),
    "local_finish_truncates": ("out[i] = or_f32_to_bf16(accumulate ? local[i] + g : g);",
                               "{ float v = accumulate ? local[i] + g : g; uint32_t u; memcpy(&u, &v, 4); out[i] = (uint16_t)(u >> 16); }"),
    "grad_coef_norm_not_unscaled": ("double norm = sqrt(sq_norm) * inv;", "double norm = sqrt(sq_norm);"),
    "grad_coef_clip_not_clamped": ("return clip < 1.0 ? inv * clip : inv;", "return inv * clip;"),
    "grad_coef_no_epsilon": ("max_norm / (norm + 1e-6)", "max_norm / norm"),
    "scaler_backoff_keeps_count": ("*clean_steps = 0;\n        return;", "return;"),
    "scaler_grows_every_step": ("if (*clean_steps == growth_interval) {", "if (1) {"),
    "scaler_backoff_is_growth": ("*scale = *scale * backoff_factor;", "*scale = *scale * growth_factor;"),
    "adamw_coef_ignored": ("double g = (double)grad[i] * coef;", "double g = (double)grad[i];"),
    "hybrid_total_from_plus_zero": ("total = g == 0 ? part : total + part;", "total = total + part;"),
    "hybrid_strided_groups": ("grads[g * group + j][i]", "grads[j * n_groups + g][i]"),
    "hybrid_sum_not_mean": ("float y = total * scale;", "float y = total;"),
    "reshard_old_rank_by_new_size": ("old_shards[e / s_old]", "old_shards[e / s_new]"),
    "reshard_copies_old_padding": ("if (e < t) {\n                const unsigned char* src", "if (e < (int64_t)world_old * s_old) {\n                const unsigned char* src"),
    "reshard_offset_in_old_wrong": ("(e % s_old) * elem_size", "(e % s_new) * elem_size"),
    "reshard_new_size_rounded_down": ("int64_t s_new = (t + world_new - 1) / world_new;", "int64_t s_new = t / world_new;"),
    "hybrid_last_group_dropped": ("for (int32_t g = 0; g < n_groups; ++g) {", "for (int32_t g = 0; g < n_groups - (n_groups > 1); ++g) {"),
}

PIN_FILES = ["tests/test_oracle_pack.py", "tests/test_oracle_reduce.py",
             "tests/test_oracle_adamw.py", "tests/test_oracle_bf16_memory.py",
             "tests/test_oracle_shard0.py", "tests/test_oracle_nosync_scaler.py",
             "tests/test_oracle_hybrid.py", "tests/test_oracle_reshard.py"]


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, "mutation site not found"
    for sub in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch {name}:\n{r.stdout[-2000:]}"
