"""The oracle pins are strong enough to catch plausible mistakes (CPU only).

Each case copies ``oracle/oracle.c``, plants one mistake in the copy (a
dropped term, a wrong sign, a swapped operand, an off-by-one index), builds
it in a temporary directory and reruns the pins against it: at least one pin
must fail.  The real oracle library is restored afterwards.
"""
from __future__ import annotations

import os
import subprocess

import pytest

import oracle
from tests import test_oracle_backward as bwd
from tests import test_oracle_block_max as blk
from tests import test_oracle_pins as pins
from tests import test_oracle_rope_ring as rr

MUTANTS = {
    "lse drops the sink": ("*lse_out = M + log(Z + E);", "*lse_out = M + log(Z);"),
    "denominator drops the sink": ("out_row[d] /= (Z + E);", "out_row[d] /= Z;"),
    "sink not shifted by the max": ("exp(sink - M)", "exp(sink)"),
    "wrong GQA head mapping": ("const int64_t g = h / G;", "const int64_t g = h % Hkv;"),
    "missing 1/sqrt(D)": ("x[j] = scale * dot;", "x[j] = dot;"),
    "exponent sign flipped": ("const double w = exp(x[j] - M);",
                              "const double w = exp(M - x[j]);"),
    "scores use V": ("dot += qrow[d] * krows[j][d];", "dot += qrow[d] * vrows[j][d];"),
    "output uses K": ("out_row[d] += w * vrows[j][d];", "out_row[d] += w * krows[j][d];"),
    "ring slot off by one": ("const int64_t slot = P % W;",
                             "const int64_t slot = (P + 1) % W;"),
    "draft position off by one": ("const int64_t p = L - T + t;",
                                  "const int64_t p = L - T + t - 1;"),
    "ring keeps one key too few": ("const int64_t oldest = L - W > 0 ? L - W : 0;",
                                   "const int64_t oldest = L - W + 1 > 0 ? L - W + 1 : 0;"),
    "pair count misses the diagonal": ("total += i - lo + 1;", "total += i - lo;"),
    # backward
    "backward drops -Dsum": ("const double dx = P * (dp[j] - Dsum);", "const double dx = P * dp[j];"),
    "dk misses the scale": ("dk[row * D + d] += scale * dx * qi[d];",
                            "dk[row * D + d] += dx * qi[d];"),
    "sink gradient sign flipped": ("ds_part[b * Hq + h] += p_sink * (0.0 - Dsum);",
                                   "ds_part[b * Hq + h] += p_sink * Dsum;"),
    "dv weighted by dP": ("dv[row * D + d] += P * gi[d];", "dv[row * D + d] += dp[j] * gi[d];"),
    "backward lse drops the sink": ("const double lse = M + log(Z + E);",
                                    "const double lse = M + log(Z);"),
    "dq uses q": ("dqi[d] += scale * dx * kj[d];", "dqi[d] += scale * dx * qi[d];"),
    "backward misses the diagonal key": ("const int64_t n = i - lo + 1;",
                                         "const int64_t n = i - lo;"),
    # block maxima
    "block max misses the diagonal": ("for (int64_t j = 0; j <= pos; ++j) {",
                                      "for (int64_t j = 0; j < pos; ++j) {"),
    "block max unscaled": ("    x *= scale;\n                    double *slot", "    x *= 1.0;\n                    double *slot"),
    "block max row blocks of 16": ("double *slot = blk + (i / 32) * nkb + j / bk;",
                                   "double *slot = blk + (i / 16 < nqb ? i / 16 : nqb - 1) * nkb + j / bk;"),
    "rope frequency exponent sign": ("pow(theta, -2.0 * (double)i / (double)D)",
                                     "pow(theta, 2.0 * (double)i / (double)D)"),
    "rope rotation sign": ("yr[i] = xr[i] * cs - xr[i + half] * sn;",
                           "yr[i] = xr[i] * cs + xr[i + half] * sn;"),
    "ring window one key short": ("const int64_t first = p - Wnd + 1 > oldest ? p - Wnd + 1 : oldest;",
                                  "const int64_t first = p - Wnd + 2 > oldest ? p - Wnd + 2 : oldest;"),
    "block max aligned at the start": ("const int64_t pos = S_kv - S_q + i;\n                const double *qi",
                                       "const int64_t pos = i;\n                const double *qi"),
}

PINS = [
    (pins.test_prefill_equals_sdpa_with_virtual_sink_token, dict(W=5)),
    (pins.test_prefill_equals_sdpa_with_virtual_sink_token, dict(W=100)),
    (pins.test_sink_neg_inf_is_banded_softmax_attention, {}),
    (pins.test_window_ge_S_is_full_causal_attention, {}),
    (pins.test_real_token_mass_is_one_minus_sink_share, {}),
    (pins.test_single_key_is_logistic, {}),
    (pins.test_window_locality, {}),
    (pins.test_gqa_head_mapping, {}),
    (pins.test_brute_force_decimal, {}),
    (pins.test_global_bottom_right_causal, {}),
    (pins.test_ring_decode_equals_sdpa_over_sequence, dict(L=23, T=4)),
    (pins.test_ring_decode_equals_sdpa_over_sequence, dict(L=9, T=4)),
    (pins.test_ring_decode_full_ring_matches_prefill_and_is_slot_order_free, {}),
    (pins.test_ring_decode_draft_windows, {}),
    (pins.test_window_pair_count_closed_form, dict(S=5000, W=128)),
    (bwd.test_backward_equals_autograd, dict(W=9)),
    (bwd.test_backward_equals_autograd_gqa_shapes, {}),
    (bwd.test_sink_neg_inf_has_zero_gradient, {}),
    (bwd.test_backward_matches_finite_differences, {}),
    (bwd.test_gqa_is_repeated_kv_heads_summed, {}),
    (bwd.test_sink_gradient_from_forward_outputs, dict(W=3)),
    (bwd.test_dv_is_attention_weights_times_dout, {}),
    (blk.test_block_max_equals_torch, dict(Sq=70, Skv=90, bk=64)),
    (blk.test_block_max_brute_force_loops, {}),
    (blk.test_row_max_brackets_lse, {}),
    (blk.test_zero_keys_give_the_causal_block_pattern, {}),
    (blk.test_heads_of_a_group_with_equal_queries_agree, {}),
    (rr.test_rope_equals_complex_rotation, dict(theta=10000.0)),
    (rr.test_rope_invariants, {}),
    (rr.test_rollback_ring_gives_full_windows, dict(R=10, W=5, T=3)),
]


def _build_mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) >= 1, old
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(lib), str(path), "-lm"], check=True)
    return oracle.bind(str(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    monkeypatch.setattr(oracle, "_lib", _build_mutant(tmp_path, old, new))
    caught = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, "no pin caught the planted mistake: %s" % name
