"""Every plausible single mistake in the oracle fails at least one pin.

Each case copies the oracle's C source, plants one mistake by text
substitution, builds it with gcc into a temporary directory, and runs the pins
against that build.  The real oracle is never modified.
"""

import os

import pytest

import oracle
import pins

MUTANTS = {
    "causal_top_left": ("int64_t lim = i + kv_len - qo_len + 1;", "int64_t lim = i + 1;"),
    "causal_off_by_one": ("int64_t lim = i + kv_len - qo_len + 1;",
                          "int64_t lim = i + kv_len - qo_len;"),
    "gqa_modulo_mapping": ("int hk = h / group;", "int hk = h % num_kv_heads;"),
    "dropped_scale": ("s[j - j_lo] = sm_scale * dot;", "s[j - j_lo] = dot;"),
    "lse_without_max": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "lse_log2": ("*lse_out = m + log(z);", "*lse_out = m + log2(z);"),
    "no_normalisation": ("out[d] /= z;", "out[d] /= 1.0;"),
    "values_from_keys": ("const uint16_t *vrow = vreq + j * kv_row_stride;",
                         "const uint16_t *vrow = kreq + j * kv_row_stride;"),
    "query_head_stride": ("const uint16_t *qrow = q + ((q0 + i) * num_qo_heads + h) * (int64_t)head_dim;",
                          "const uint16_t *qrow = q + ((q0 + i) + h) * (int64_t)head_dim;"),
    "exp_without_shift": ("double w = exp(s[j - j_lo] - m);", "double w = exp(s[j - j_lo]);"),
    "merge_swapped_weights": ("vo[d] = va[d] * wa + vb[d] * wb;",
                              "vo[d] = va[d] * wb + vb[d] * wa;"),
    "merge_lse_max_only": ("double lse = m + log(exp(a - m) + exp(b - m));", "double lse = m;"),
    "merge_states_unnormalised": ("const double w = exp(l[i] - merged);",
                                  "const double w = exp(l[i] - m);"),
    "merge_states_lse_no_shift": ("const double merged = m + log(total);",
                                  "const double merged = log(total);"),
    "merge_states_first_only": ("for (int i = 0; i < k; ++i)\n            total += exp(l[i] - m);",
                                "for (int i = 0; i < 1; ++i)\n            total += exp(l[i] - m);"),
    "window_low_ignored": ("int64_t j_lo = key_lo > 0 ? key_lo : 0;", "int64_t j_lo = 0;"),
    "masked_row_nan": ("        *lse_out = -INFINITY;\n        return;",
                       "        *lse_out = NAN;\n        return;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load_library(oracle.compile_source(str(mutated), str(tmp_path / "libmutant.so")))
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib=lib)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"
