"""The pins are strong enough: each plausible slip in the oracle fails one.

Every mutant below is the oracle source with one deliberate mistake, compiled
to a temporary library on the CPU.  The pin suite of test_oracle_pins must
reject every one of them (and accept the unmodified source).
"""

import os
import tempfile

import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_prefill as prefill
import test_oracle_quant as quant

MUTANTS = {
    "interleaved_gqa_groups": ("int g = h / (p->Hq / p->Hkv);", "int g = h % p->Hkv;"),
    "dropped_softmax_scale": ("s[t - t0] = p->scale * dot;", "s[t - t0] = dot;"),
    "no_max_subtraction": ("double w = exp(s[t - t0] - M);", "double w = exp(s[t - t0]);"),
    "unnormalised_output": ("o[d] = acc[d] / Z;", "o[d] = acc[d];"),
    "int8_scale_ignored": ("x = (double)sc[tile] * x;", "x = 1.0 * x;"),
    "values_read_from_keys": ("const void *base = which ? p->v_pages : p->k_pages;",
                              "const void *base = p->k_pages;"),
    "pool_layout_head_major": ("size_t tile = ((size_t)row * p->Hkv + g) * p->PS + slot;",
                               "size_t tile = ((size_t)g * p->n_host_pages + row) * p->PS + slot;"),
    "key_slot_off_by_one": ("kv_elem(p, 0, row, g, t % p->PS, d)",
                            "kv_elem(p, 0, row, g, (t + 1) % p->PS, d)"),
    "query_transposed": ("size_t qoff = ((size_t)b * p->Hq + h) * p->D;",
                         "size_t qoff = ((size_t)h * p->B + b) * p->D;"),
    "f16_subnormal_exponent": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "f16_sign_lost": ("return sign ? -v : v;", "return v;"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "fp8_exponent_bias": ("v = ldexp((double)(m | 8), e - 10);", "v = ldexp((double)(m | 8), e - 11);"),
    "fp8_subnormal_as_normal": ("v = ldexp((double)m, -9);", "v = ldexp((double)(m | 8), -10);"),
    "quant_int8_range": ("const float qmax = kind == ORC_I8 ? 127.0f : 448.0f;",
                         "const float qmax = kind == ORC_I8 ? 128.0f : 448.0f;"),
    "quant_truncates": ("float r = rintf(y);", "float r = truncf(y);"),
    "fp8_encode_mantissa_floor": ("double m = rint((ldexp(a, -e) - 1.0) * 8.0);",
                                  "double m = floor((ldexp(a, -e) - 1.0) * 8.0);"),
    "fp8_encode_no_carry": ("        m = 0.0;\n        e += 1;", "        m = 7.0;"),
    "fp8_scale_ignored": ("static int scaled_kv(int dtype) { return dtype == ORC_I8 || dtype == ORC_FP8; }",
                          "static int scaled_kv(int dtype) { return dtype == ORC_I8; }"),
    "split_merge_missing_rescale": ("L += l[k] * exp(m[k] - M);", "L += l[k];"),
    "split_partition_max_wrong": ("m[k] = mk;", "m[k] = 0.0;"),
    "prefill_position_off_by_one": ("int pos = n - nq + i;", "int pos = n - nq + i - 1;"),
    "prefill_not_causal": ("double Z = weighted_v_g(&p, g, b, 0, pos + 1, s, M, acc);",
                           "double Z = weighted_v_g(&p, g, b, 0, pos + 1, s, M, acc);\n"
                           "            if (pos + 1 < n) { (void)scores_q(&p, ((size_t)row * Hq + h) * D, g, b, 0, n, s);"
                           " M = s[0]; for (int t = 1; t < n; ++t) if (s[t] > M) M = s[t];"
                           " Z = weighted_v_g(&p, g, b, 0, n, s, M, acc); }"),
    "prefill_query_row_of_wrong_sequence": ("long row = q_start[b] + i;", "long row = q_start[b] + (nq - 1 - i);"),
}

PIN_SUITE = [
    lambda: pins.test_f16_decode_matches_numpy_all_patterns(oracle.lib()),
    lambda: pins.test_bf16_decode_matches_torch_all_patterns(oracle.lib()),
    lambda: pins.test_fp8_e4m3_decode_matches_torch_all_patterns(oracle.lib()),
    *[(lambda s=s: pins.test_oracle_matches_pure_python_brute_force(s)) for s in pins.TINY_SHAPES],
    *[(lambda T=T: pins.test_split_merge_matches_unsplit(T)) for T in (16, 64)],
    pins.test_large_common_score_shift_is_harmless,
    pins.test_gqa_equals_mha_with_repeated_kv_heads_bitwise,
    pins.test_int8_with_unit_scales_equals_f16_of_same_integers,
    pins.test_fp8_with_unit_scales_equals_f16_of_same_values,
    lambda: quant.test_quantiser_matches_generator_encoders("i8"),
    lambda: quant.test_quantiser_matches_generator_encoders("fp8"),
    quant.test_int8_ties_round_to_even,
    *[(lambda s=s: prefill.test_prefill_matches_pure_python_causal_attention(s)) for s in pins.TINY_SHAPES[:3]],
    lambda: prefill.test_last_query_of_a_chunk_is_a_decode_step(pins.TINY_SHAPES[0]),
    prefill.test_causality_later_keys_do_not_matter,
    prefill.test_first_token_of_a_sequence_returns_its_value,
    prefill.test_a_query_depends_on_its_position_not_on_its_chunk,
    quant.test_fp8_encode_round_trips_every_finite_code,
    quant.test_fp8_encode_ties_and_saturation,
]


def run_suite_against(src_text):
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(src_text)
        so = oracle.build(src=src, out=os.path.join(d, "libmutant.so"))
        prev = oracle.set_lib(oracle.load(so))
        failures = 0
        try:
            for check in PIN_SUITE:
                try:
                    check()
                except (AssertionError, oracle.OracleError, ValueError):
                    failures += 1
        finally:
            oracle.set_lib(prev)
        return failures


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC_PATH) as f:
        return f.read()


def test_unmodified_source_passes_the_suite(source):
    assert run_suite_against(source) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(source, name):
    old, new = MUTANTS[name]
    assert old in source, f"mutation site of {name} not found"
    assert run_suite_against(source.replace(old, new)) > 0
