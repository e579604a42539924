"""Each plausible slip in the oracle's C source must fail at least one pin.

A mutant is the oracle source with one systematic edit (every occurrence of
a fragment replaced).  It is compiled with gcc into a temporary library and
the pin checks of ``oracle_checks.py`` run against it; the test passes when
at least one check fails.  Nothing here touches the real oracle library.
"""
import os

import pytest

import oracle
import oracle_checks

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "gqa_interleaved": ("int g = n / G;", "int g = n % K;"),
    "block_index_mod": ("int64_t p = table[t / bs];", "int64_t p = table[t % bs];"),
    "offset_swapped": ("int o = t % bs;", "int o = (t / bs) % bs;"),
    "no_max_subtract": ("scores[t] = exp(scores[t] - m);", "scores[t] = exp(scores[t]);"),
    "sign_flip": ("scores[t] = exp(scores[t] - m);", "scores[t] = exp(m - scores[t]);"),
    "no_normalise": ("row[h] /= z;", "row[h] /= 1.0;"),
    "no_scale": ("scores[t] = sc * dot;", "scores[t] = dot;"),
    "value_index_transposed": ("value_index(p, g, h, o, K, bs, H)", "value_index(p, g, o % H, h % bs, K, bs, H)"),
    "key_index_transposed": ("key_index(p, g, o, h, K, bs, H)", "key_index(p, g, h % bs, o % H, K, bs, H)"),
    "ctx_off_by_one": ("for (int t = first; t < ctx; t++)", "for (int t = first; t < ctx - 1; t++)"),
    "append_v_from_k": ("value_cache[value_index(p, g, h, o, K, bs, H)] = v[src];",
                        "value_cache[value_index(p, g, h, o, K, bs, H)] = k[src];"),
    "append_negative_slot_not_skipped": ("if (s < 0)\n            continue;",
                                         "if (s < 0)\n            s = 0;"),
    "merge_unweighted_l": ("L += w * piece_l[j];", "L += piece_l[j];"),
    "merge_no_rescale": ("double w = exp(piece_m[j] - M);", "double w = 1.0;"),
    "kv_formula_no_two": ("return 2 * layers", "return layers"),
    "e4m3_bias": ("mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3_subnormal": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "e4m3_ties_odd": ("((lo + 1) & 1) == 0", "((lo + 1) & 1) == 1"),
    "e4m3_nan_not_kept": ("if (isnan(y))\n        return 0xFF;", "if (0)\n        return 0xFF;"),
    "e4m3_truncate": ("if (d_hi < d_lo ||", "if (0 &&"),
    "fp8_scale_dropped": ("return oracle_e4m3_value(((const uint8_t *)pool)[index]) * scale;",
                          "return oracle_e4m3_value(((const uint8_t *)pool)[index]);"),
    "fp8_append_v_from_k": ("oracle_e4m3_quantize(v[src], v_inv);", "oracle_e4m3_quantize(k[src], v_inv);"),
    "multi_top_left_mask": ("int v = ctx - Q + i + 1;", "int v = i + 1;"),
    "multi_mask_off_by_one": ("int v = ctx - Q + i + 1;", "int v = ctx - Q + i;"),
    "multi_query_layout": ("int b = r / (Q * N), i = (r / N) % Q, n = r % N;",
                           "int b = r / (Q * N), i = r % Q, n = (r / Q) % N;"),
    "multi_rows_query_layout": ("q + (((size_t)b * Q + i) * N + n) * H",
                                "q + (((size_t)b * N + n) * Q + i) * H"),
    "copy_value_from_key": ("value_cache[vd] = value_cache[vs];", "value_cache[vd] = key_cache[ks];"),
    "copy_one_head": ("for (int g = 0; g < K; g++)\n            for (int o = 0; o < bs; o++)",
                      "for (int g = 0; g < 1; g++)\n            for (int o = 0; o < bs; o++)"),
    "window_off_by_one": ("int first = ctx - window > 0 ? ctx - window : 0;",
                          "int first = ctx - window + 1 > 0 ? ctx - window + 1 : 0;"),
    "window_ignored": ("int first = ctx - window > 0 ? ctx - window : 0;", "int first = 0;"),
    "copy_low_bytes_only": ("for (int e = 0; e < elem_bytes; e++) {", "for (int e = 0; e < 1; e++) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found in the oracle source"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.load_library(oracle.build(force=True, src=str(mutant_src),
                                           out=str(tmp_path / "libmutant.so")))
    failures = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError) as e:
            failures.append(f"{check.__name__}: {str(e)[:80]}")
    assert failures, f"mutant {name} passed every pin"
