"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c, applies one plausible mistake (a dropped term, a
wrong sign, index or base, a wrong head map, a shifted mask), builds the copy
with gcc and runs the pin suite against it in a child process.  The pins pass
on the real oracle (test_oracle.py); here at least one of them must fail for
every mutant.  Everything runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "head_map_modulo": ("int g = h / group;\n            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * kv_len",
                        "int g = h % Hkv;\n            kv_view kv = {k, v, dt, D, ((int64_t)b * Hkv + g) * kv_len"),
    "causal_off_by_one": ("int64_t vis_end = causal ? i + 1 + delta : (int64_t)kv_len;\n            attend_one(q, r",
                          "int64_t vis_end = causal ? i + delta : (int64_t)kv_len;\n            attend_one(q, r"),
    "causal_top_left": ("int64_t vis_end = causal ? i + 1 + delta : (int64_t)kv_len;\n            attend_one(q, r",
                        "int64_t vis_end = causal ? i + 1 : (int64_t)kv_len;\n            attend_one(q, r"),
    "lse_base_two": ("double L = m + log(z);", "double L = m + log2(z);"),
    "scale_dropped": ("s[t - lo] = scale * acc;", "s[t - lo] = acc;"),
    "max_not_subtracted": ("z += exp(s[t - lo] - m);", "z += exp(s[t - lo]);"),
    "prob_sign_flipped": ("double p = exp(s[t - lo] - L);", "double p = exp(L - s[t - lo]);"),
    "values_read_from_keys": ("o[d] += p * kv_value(kv, kv->v, kv->v_ss, t, d);",
                              "o[d] += p * kv_value(kv, kv->k, kv->k_ss, t, d);"),
    "value_feature_shifted": ("o[d] += p * kv_value(kv, kv->v, kv->v_ss, t, d);",
                              "o[d] += p * kv_value(kv, kv->v, kv->v_ss, t, (d + 1) % D);"),
    "empty_row_lse_zero": ("*lse = -INFINITY;\n        return;", "*lse = 0.0;\n        return;"),
    "page_row_shifted": ("int64_t row = t % kv->page_size;", "int64_t row = (t + 1) % kv->page_size;"),
    "merge_weight_sign": ("double w = exp(ls[sp] - M);", "double w = exp(M - ls[sp]);"),
    "merge_lse_dropped_max": ("lse_out[n] = M + log(wsum);", "lse_out[n] = log(wsum);"),
    "half_exponent_bias": ("v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "multi_query_position_off_by_one": ("int64_t vis_end = len - q_len + i + 1;",
                                        "int64_t vis_end = len - q_len + i;"),
    "multi_query_order_reversed": ("int64_t vis_end = len - q_len + i + 1;",
                                   "int64_t vis_end = len - i;"),
    "paged_prefill_last_page_ignored": ("kv_len = (n_pages - 1) * page_size + (kv_last_page_len ? kv_last_page_len[b] : page_size);",
                                        "kv_len = n_pages * page_size;"),
    "e4m3_exponent_bias": ("v = ldexp((double)(m | 0x8), e - 10);", "v = ldexp((double)(m | 0x8), e - 9);"),
    "e4m3_subnormal_scale": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "fp8_scale_shift_swapped": ("return x * half_bits_to_double((uint16_t)(w & 0xffff)) + half_bits_to_double((uint16_t)(w >> 16));",
                                "return x * half_bits_to_double((uint16_t)(w >> 16)) + half_bits_to_double((uint16_t)(w & 0xffff));"),
    "paged_prefill_top_left": ("int64_t vis_end = causal ? i + 1 + (kv_len - q_len) : kv_len;",
                               "int64_t vis_end = causal ? i + 1 : kv_len;"),
    "bias_dropped": ("if (bias.p) s[t - lo] += elem(bias.p, bias.off + t, bias.dt);", ";"),
    "bias_scaled_with_scores": ("if (bias.p) s[t - lo] += elem(bias.p, bias.off + t, bias.dt);",
                                "if (bias.p) s[t - lo] += scale * elem(bias.p, bias.off + t, bias.dt);"),
    "bias_query_and_head_strides_swapped": ("bias_view bv = {bias, bias_dt, b * sb + h * sh + i * sq};",
                                            "bias_view bv = {bias, bias_dt, b * sb + h * sq + i * sh};"),
    "decode_bias_query_index_dropped": ("bias_view bv = {bias, bias_dt, (int64_t)b * sb + (int64_t)h * sh + i * sq};",
                                        "bias_view bv = {bias, bias_dt, (int64_t)b * sb + (int64_t)h * sh};"),
    "bias_fully_masked_row_not_empty": ("if (m == -INFINITY) { *lse = m; return; }", ";"),
    "merge_standalone_lse_without_max": ("lse_out[n] = log(wtot) + M;", "lse_out[n] = log(wtot);"),
    "merge_backward_dot_dropped": ("d_lse_parts[ps] = w == 0.0 ? 0.0 : w * (d_lse[n] + dot);",
                                   "d_lse_parts[ps] = w == 0.0 ? 0.0 : w * d_lse[n];"),
    "merge_backward_difference_reversed": ("dot += (os[d] - orow[d]) * dorow[d];",
                                           "dot += (orow[d] - os[d]) * dorow[d];"),
    "merge_backward_weight_unnormalised": ("exp(ls - lse[n])", "exp(ls)"),
    "bias_fwd_causal_off_by_one": ("int64_t vis_end = causal ? (i + 1) + delta : (int64_t)kv_len;",
                                   "int64_t vis_end = causal ? i + delta : (int64_t)kv_len;"),
    "bias_fwd_head_map_modulo": ("const int g = h / group;  /* K/V head of query head h */",
                                 "const int g = h % Hkv;  /* K/V head of query head h */"),
    "decode_bias_position_off_by_one": ("int64_t vis_end = (len - q_len) + i + 1;",
                                        "int64_t vis_end = (len - q_len) + i;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, GQA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
