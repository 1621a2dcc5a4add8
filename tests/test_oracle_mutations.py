"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong index, sign or tie rule), builds it on the CPU, and checks that
at least one pin from ``test_oracle_pins`` fails against it.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_prefill_pins as prefill_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTATIONS = {
    "drop_scale": ("score[t] = scale * dot;", "score[t] = dot;"),
    "drop_normalisation": ("out_row[d] /= denom;", "out_row[d] /= 1.0;"),
    "wrong_gqa_head": ("int g = h / group;", "int g = h % Hkv;"),
    "wrong_slot_in_block": ("int o = (int)(t % 16);\n        double dot", "int o = (int)((t + 1) % 16);\n        double dot"),
    "wrong_value_row": ("out_row[d] += w * orc_load(v_pool, orc_v_offset(b, g, o, d,",
                        "out_row[d] += w * orc_load(v_pool, orc_v_offset(b, g, (o + 1) % 16, d,"),
    "query_index_transposed": ("int64_t qrow = (int64_t)s * Hq + h;",
                               "int64_t qrow = (int64_t)h * 1 + s;"),
    "fp8_ties_up": ("c = (lo % 2 == 0) ? lo : hi;", "c = hi;"),
    "fp8_subnormal_exponent": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "fp8_no_saturation": ("if (a >= orc_fp8_mag[126])\n        return (uint8_t)(sign | 0x7E);",
                          "if (a >= orc_fp8_mag[126])\n        return (uint8_t)(sign | 0x7F);"),
    "scatter_skips_offset": ("int t = slot % 16;", "int t = slot % 15;"),
    "prefill_excludes_own_token": ("tables + (int64_t)s * MBS, pos + 1,",
                                   "tables + (int64_t)s * MBS, pos,"),
    "prefill_not_causal": ("tables + (int64_t)s * MBS, pos + 1,",
                           "tables + (int64_t)s * MBS, (int64_t)ctx[s],"),
    "prefill_ignores_cached_prefix": ("int64_t pos = (int64_t)ctx[s] - n_new + i;",
                                      "int64_t pos = i;"),
    "prefill_query_rows_transposed": ("q, q_dt, qi * Hq + h, Hq, h,", "q, q_dt, qi + h * Hq, Hq, h,"),
    # fp8 dequantisation inside attention: V scaled by K's scale, codes read
    # without their scale, K's scale left out of the scores
    "fp8_v_uses_k_scale": ("pool_dt, v_scale);", "pool_dt, k_scale);"),
    "fp8_no_scale": ("return orc_fp8_decode(base[idx]) * fp8_scale;",
                     "return orc_fp8_decode(base[idx]);"),
    "fp8_k_scale_dropped": ("pool_dt, k_scale);", "pool_dt, 1.0);"),
    "fp8_scale_inverted": ("return orc_fp8_decode(base[idx]) * fp8_scale;",
                           "return orc_fp8_decode(base[idx]) / fp8_scale;"),
}

PIN_TESTS = [
    pins.test_worked_example_table_readback_and_waste,
    lambda: pins.test_workload_readback_through_tables("mha13b"),
    lambda: pins.test_paged_equals_dense_library_softmax("sampling_b"),
    lambda: pins.test_paged_equals_dense_library_softmax("fp8"),
    pins.test_fp8_scales_two_tokens_closed_form,
    pins.test_single_token_returns_its_value_exactly,
    pins.test_zero_query_gives_mean_of_values,
    pins.test_two_tokens_logistic_closed_form,
    pins.test_gqa_equals_mha_with_replicated_kv_heads,
    lambda: pins.test_one_hot_probe_selects_exactly_one_value(40),
    pins.test_fp8_decode_matches_torch_float8_e4m3fn,
    pins.test_fp8_encode_matches_torch_cast_below_overflow,
    pins.test_fp8_encode_saturates_and_keeps_nan,
    pins.test_fp8_scatter_encodes_scaled_values,
    lambda: prefill_pins.test_prefill_equals_dense_causal_library_softmax("chunked_gqa70b"),
    lambda: prefill_pins.test_prefill_equals_dense_causal_library_softmax("chunked_fp8"),
    lambda: prefill_pins.test_each_chunk_row_equals_decode_at_its_position("chunked_gqa70b"),
    prefill_pins.test_causality_future_tokens_do_not_matter,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must occur once: %s" % name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-std=c11", "-o", str(so), str(path), "-lm"])
    saved = oracle.lib()
    oracle._lib = oracle.bind(ctypes.CDLL(str(so)))
    failures = 0
    try:
        for t in PIN_TESTS:
            try:
                t()
            except (AssertionError, ValueError):
                failures += 1
    finally:
        oracle._lib = saved
    assert failures > 0, "no pin caught mutation %s" % name
