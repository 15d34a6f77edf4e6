"""Planted mistakes in the oracle must each be caught by at least one pin (CPU only).

Every mutant is a copy of oracle/gdn_oracle.c with one textual change: a dropped
term, a wrong sign, a wrong or transposed index, a swapped operand, a wrong
head map. Each copy is compiled into a temporary library and run through all
pins of tests/oracle_pins.py.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = {
    "drop_decay": ("S[(int64_t)i * dk + j] = alpha * (s - beta * u[i] * kj) + beta * (double)vv[i] * kj;",
                   "S[(int64_t)i * dk + j] = (s - beta * u[i] * kj) + beta * (double)vv[i] * kj;"),
    "decay_misses_erase": ("S[(int64_t)i * dk + j] = alpha * (s - beta * u[i] * kj) + beta * (double)vv[i] * kj;",
                           "S[(int64_t)i * dk + j] = alpha * s - beta * u[i] * kj + beta * (double)vv[i] * kj;"),
    "erase_sign": ("alpha * (s - beta * u[i] * kj)", "alpha * (s + beta * u[i] * kj)"),
    "write_without_beta": ("+ beta * (double)vv[i] * kj;", "+ (double)vv[i] * kj;"),
    "erase_without_beta": ("alpha * (s - beta * u[i] * kj)", "alpha * (s - u[i] * kj)"),
    "transposed_read": ("acc += S[(int64_t)i * dk + j] * (double)kk[j];",
                        "acc += S[(int64_t)j * dk + i] * (double)kk[j];"),
    "transposed_output": ("acc += S[(int64_t)i * dk + j] * (scale * (double)qq[j]);",
                          "acc += S[(int64_t)j * dk + i] * (scale * (double)qq[j]);"),
    "no_scale": ("(scale * (double)qq[j])", "((double)qq[j])"),
    "output_reads_key": ("(scale * (double)qq[j])", "(scale * (double)kk[j])"),
    "value_index_swapped": ("+ beta * (double)vv[i] * kj;", "+ beta * (double)vv[j % dv] * kj;"),
    "tiled_map_wrong": ("if (head_map == 0) return h % Hk;", "if (head_map == 0) return h / (Hv / Hk);"),
    "grouped_map_wrong": ("return h / (Hv / Hk);", "return h % Hk;"),
    "decay_from_previous_token": ("double alpha = exp((double)g[gi]);",
                                  "double alpha = exp((double)g[t > 0 ? gi - 1 : gi]);"),
    "decay_not_exponentiated": ("double alpha = exp((double)g[gi]);", "double alpha = 1.0 + (double)g[gi];"),
    "value_reads_key_head": ("const float *vv = v + (((int64_t)b * Hv + h) * T + t) * dv;",
                             "const float *vv = v + (((int64_t)b * Hv + kh) * T + t) * dv;"),
    "initial_state_transposed": ("for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = src[e];",
                                 "for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = src[(e % dk) * dv + e / dk];"),
    "initial_state_ignored": ("for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = src[e];",
                              "for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = 0.0 * src[e];"),
    "output_before_update": [
        ("    /* S <- alpha * S (I - beta k k^T) + beta v k^T",
         "    for (int i = 0; i < dv; ++i) {\n"
         "        double acc = 0.0;\n"
         "        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (scale * (double)qq[j]);\n"
         "        out[i] = acc;\n"
         "    }\n"
         "    /* S <- alpha * S (I - beta k k^T) + beta v k^T"),
        ("        out[i] = acc;\n    }\n}", "    }\n}"),
    ],
    "rmsnorm_sum_not_mean": ("const double inv = 1.0 / sqrt(ss / n + eps);", "const double inv = 1.0 / sqrt(ss + eps);"),
    "rmsnorm_eps_outside": ("const double inv = 1.0 / sqrt(ss / n + eps);", "const double inv = 1.0 / (sqrt(ss / n) + eps);"),
    "rmsnorm_no_sqrt": ("const double inv = 1.0 / sqrt(ss / n + eps);", "const double inv = 1.0 / (ss / n + eps);"),
    "silu_is_sigmoid": ("v *= z / (1.0 + exp(-z));", "v *= 1.0 / (1.0 + exp(-z));"),
    "silu_sign": ("v *= z / (1.0 + exp(-z));", "v *= z / (1.0 + exp(z));"),
    "weight_by_row": ("double v = xr[i] * inv * (double)weight[i];", "double v = xr[i] * inv * (double)weight[r % n];"),
    "conv_taps_reversed": ("acc += win[(size_t)(t + i) * C + c] * (double)w[(size_t)c * K + i];",
                           "acc += win[(size_t)(t + i) * C + c] * (double)w[(size_t)c * K + (K - 1 - i)];"),
    "conv_window_shifted": ("acc += win[(size_t)(t + i) * C + c] * (double)w[(size_t)c * K + i];",
                            "acc += win[(size_t)(t + i + (i < K - 1)) * C + c] * (double)w[(size_t)c * K + i];"),
    "conv_state_ignored": ("win[(size_t)r * C + c] = state_in ? state_in[((size_t)b * (K - 1) + r) * C + c] : 0.0;",
                           "win[(size_t)r * C + c] = 0.0;"),
    "prologue_silu_is_sigmoid": ("y[j] = acc / (1.0 + exp(-acc));", "y[j] = 1.0 / (1.0 + exp(-acc));"),
    "prologue_v_normalised": ("if (hh < 2 * Hk) {", "if (hh < 2 * Hk + Hv) {"),
    "prologue_mean_not_sum": ("f = 1.0 / sqrt(ss + eps);", "f = 1.0 / sqrt(ss / d + eps);"),
    "prologue_k_reads_q": ("k + (((size_t)b * Hk + (hh - Hk)) * T + t) * d", "k + (((size_t)b * Hk + (hh - Hk + Hk - 1) % Hk) * T + t) * d"),
    "kda_decay_on_value_rows": ("for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= alpha[j];",
                                "for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= alpha[i % dk];"),
    "kda_no_decay": ("for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= alpha[j];",
                     "for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= 1.0;"),
    "kda_erase_sign": ("+= beta * ((double)vv[i] - u[i]) * (double)kk[j];",
                       "+= beta * ((double)vv[i] + u[i]) * (double)kk[j];"),
    "kda_write_without_beta": ("+= beta * ((double)vv[i] - u[i]) * (double)kk[j];",
                               "+= ((double)vv[i] - beta * u[i]) * (double)kk[j];"),
    "kda_channels_reversed": ("alpha[j] = exp((double)g[gi * dk + j]);", "alpha[j] = exp((double)g[gi * dk + (dk - 1 - j)]);"),
    "kda_decay_not_exponentiated": ("alpha[j] = exp((double)g[gi * dk + j]);", "alpha[j] = 1.0 + (double)g[gi * dk + j];"),
    "kda_decay_of_previous_token": ("alpha[j] = exp((double)g[gi * dk + j]);",
                                    "alpha[j] = exp((double)g[(t > 0 ? gi - 1 : gi) * dk + j]);"),
    "kda_decode_one_channel": ("alpha[j] = exp((double)g[pair * dk + j]);", "alpha[j] = exp((double)g[pair * dk]);"),
    "kda_erase_before_decay": [
        ("    /* S <- S diag(alpha) */\n    for (int i = 0; i < dv; ++i)\n"
         "        for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= alpha[j];\n", ""),
        ("    /* S <- S (I - beta k k^T) + beta v k^T = S + beta (v - S k) k^T */\n"
         "    for (int i = 0; i < dv; ++i)\n"
         "        for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] += beta * ((double)vv[i] - u[i]) * (double)kk[j];\n",
         "    for (int i = 0; i < dv; ++i)\n"
         "        for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] = alpha[j] * (S[(int64_t)i * dk + j] - beta * u[i] * (double)kk[j]) + beta * (double)vv[i] * (double)kk[j];\n"),
    ],
    "kda_output_reads_key": ("for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (scale * (double)qq[j]);\n        out[i] = acc;\n    }\n}\n\n/*\n * KDA prefill",
                             "for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (scale * (double)kk[j]);\n        out[i] = acc;\n    }\n}\n\n/*\n * KDA prefill"),
    "output_step_off_by_one": ("if (o) memcpy(o + ((int64_t)p * T + t) * dv, out,",
                               "if (o) memcpy(o + ((int64_t)p * T + (t + 1) % T) * dv, out,"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    mutated = source
    for old, new in edits:
        assert mutated.count(old) >= 1, f"mutant {name}: pattern no longer in the oracle source"
        mutated = mutated.replace(old, new, 1)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(src), lib, extra_flags=["-w"])
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:  # a failed pin, or arguments the mutant rejects
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches the planted mistake {name!r}"
    os.remove(lib)
