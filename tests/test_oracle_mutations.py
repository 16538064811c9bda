"""Plant plausible mistakes in the oracle's C source and check the pins catch them.

Each mutant is a copy of oracle/sdpa_oracle.c with one textual change (a dropped
term, a wrong sign, a wrong index or an off-by-one in a mask), compiled with gcc
into a temporary library.  The pin battery of ``pins.py`` must pass on the real
oracle and fail on every mutant.  Nothing here touches the GPU.
"""
import os

import pytest

import oracle
import pins

MUTATIONS = {
    "scale_dropped": ("s[j] = dot / root_dk;", "s[j] = dot;"),
    "scale_by_dk": ("const double root_dk = sqrt((double)d_k);",
                    "const double root_dk = (double)d_k;"),
    "scale_by_dv": ("const double root_dk = sqrt((double)d_k);",
                    "const double root_dk = sqrt((double)d_v);"),
    "causal_diagonal_excluded": ("if (causal && j > i) return 0;",
                                 "if (causal && j >= i) return 0;"),
    "causal_reversed": ("if (causal && j > i) return 0;", "if (causal && j < i) return 0;"),
    "padding_off_by_one": ("if (j >= len) return 0;", "if (j > len) return 0;"),
    "exp_sign": ("w[j] = exp(s[j] - m);", "w[j] = exp(m - s[j]);"),
    "not_normalised": ("w[j] = w[j] / Z;", "w[j] = w[j];"),
    "max_reversed": ("if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    "dot_wrong_index": ("dot += q[t] * k[t];", "dot += q[t] * k[0];"),
    "key_stride_dv": ("const double *k = K + j * d_k;", "const double *k = K + j * d_v;"),
    "value_wrong_column": ("o[t] += pj * v[t];", "o[t] += pj * v[0];"),
    "value_head_zero": ("const double *Vh = V + bh * Lk * d_v;",
                        "const double *Vh = V + b * H * Lk * d_v;"),
    "key_head_zero": ("const double *Kh = K + bh * Lk * d_k;",
                      "const double *Kh = K + b * H * Lk * d_k;"),
    "query_row_zero": ("attention_row(Q + r * d_k, Kh, Vh,", "attention_row(Q + bh * Lq * d_k, Kh, Vh,"),
    "empty_row_nan": ("for (int64_t t = 0; t < d_v; ++t) o[t] = 0.0;\n        if (p_out)",
                      "for (int64_t t = 0; t < d_v; ++t) o[t] = NAN;\n        if (p_out)"),
    "lse_without_max": ("if (lse) *lse = m + log(Z);", "if (lse) *lse = log(Z);"),
    "rows_api_causal_dropped": ("Lk, d_k, d_v, clamp_len(key_lengths, b, Lk), causal, radius, i,",
                                "Lk, d_k, d_v, clamp_len(key_lengths, b, Lk), 0, radius, i,"),
    "rows_api_radius_dropped": ("Lk, d_k, d_v, clamp_len(key_lengths, b, Lk), causal, radius, i,",
                                "Lk, d_k, d_v, clamp_len(key_lengths, b, Lk), causal, -1, i,"),
    "band_lower_off_by_one": ("j < i - radius ||", "j <= i - radius ||"),
    "band_upper_off_by_one": ("|| j > i + radius)", "|| j >= i + radius)"),
    "band_upper_dropped": ("|| j > i + radius)", ")"),
    "band_lower_dropped": ("(j < i - radius || j > i + radius)", "(j > i + radius)"),
    "band_radius_doubled": ("j < i - radius || j > i + radius", "j < i - 2 * radius || j > i + 2 * radius"),
    # multi-head projections (§3.2.2)
    "mh_wq_uses_wk": ("row_times(Xq + r * d_model, Wq, d_model, h * d_k, y);",
                      "row_times(Xq + r * d_model, Wk, d_model, h * d_k, y);"),
    "mh_wv_uses_wk": ("row_times(Xkv + r * d_model, Wv, d_model, h * d_v, y);",
                      "row_times(Xkv + r * d_model, Wk, d_model, h * d_v, y);"),
    "mh_keys_from_queries": ("row_times(Xkv + r * d_model, Wk, d_model, h * d_k, y);",
                             "row_times(Xq + (r % (B * Lq)) * d_model, Wk, d_model, h * d_k, y);"),
    "mh_projection_transposed": ("y[n] += xc * w[n];", "y[n] += xc * W[n * d_model + c];"),
    "mh_head_split_offset_dropped": ("P[((b * h + hd) * L + i) * d + t] = y[hd * d + t];",
                                     "P[((b * h + hd) * L + i) * d + t] = y[t];"),
    "mh_concat_head_dropped": ("cat[hd * d_v + t] = A[((b * h + hd) * Lq + i) * d_v + t];",
                               "cat[hd * d_v + t] = A[((b * h) * Lq + i) * d_v + t];"),
    "mh_wo_uses_wv": ("row_times(cat, Wo, h * d_v, d_model, O + r * d_model);",
                      "row_times(cat, Wv, h * d_v, d_model, O + r * d_model);"),
    "mh_causal_dropped": ("rc = oracle_attention(Qp, Kp, Vp, key_lengths, causal, -1,",
                          "rc = oracle_attention(Qp, Kp, Vp, key_lengths, 0, -1,"),
    "mh_lengths_dropped": ("rc = oracle_attention(Qp, Kp, Vp, key_lengths, causal, -1,",
                           "rc = oracle_attention(Qp, Kp, Vp, NULL, causal, -1,"),
    "mh_rows_causal_dropped": ("d_v, len, causal, -1, i, sc, w, cat + hd * d_v, NULL, NULL);",
                               "d_v, len, 0, -1, i, sc, w, cat + hd * d_v, NULL, NULL);"),
    "mh_rows_head_offset": ("attention_row(q + hd * d_k, Kp + hd * Lk * d_k,",
                            "attention_row(q, Kp + hd * Lk * d_k,"),
}


def _run_battery(orc):
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            failed.append((check.__name__, str(e)[:120]))
    return failed


def test_real_oracle_passes_battery():
    assert _run_battery(oracle.default()) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE, encoding="utf-8").read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(src.replace(old, new), encoding="utf-8")
    lib = oracle.compile_oracle(str(path), str(tmp_path / ("libmutant_%s.so" % name)))
    failed = _run_battery(oracle.Oracle(lib))
    assert failed, "mutant %s passed every pin" % name
