"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of moe_oracle.c (a swapped table entry, a wrong nibble,
index or sign, a dropped term, a transposed operand, ...), builds it, and
runs the oracle pin tests against that build in a fresh process. Every
mutant must fail at least one pin; the unmodified source is the one the
rest of the suite tests."""

import os
import subprocess
import sys
import tempfile
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "moe_oracle.c"

MX = "tests/test_oracle_mx.py"
ROUTE = "tests/test_oracle_routing.py"
LAYER = "tests/test_oracle_layer.py"
LORA = "tests/test_oracle_lora.py"
MX8 = "tests/test_oracle_mx8.py"
FP6 = "tests/test_oracle_fp6x2.py"

# name: (text in moe_oracle.c, replacement, pin files expected to catch it)
MUTANTS = {
    "e2m1_codes_5_6_swapped": ("0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,",
                               "0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 4.0f, 3.0f, 6.0f,", [MX]),
    "negative_zero_unsigned": ("    -0.0f, -0.5f,", "    0.0f, -0.5f,", [MX]),
    "nibble_order": ("int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);",
                     "int code = (i % 2 == 0) ? (byte >> 4) : (byte & 15);", [MX]),
    "scale_bias_126": ("return ldexpf(E2M1_VALUE[code], s - 127);",
                       "return ldexpf(E2M1_VALUE[code], s - 126);", [MX]),
    "scale_of_next_block": ("int s = scales[n * (K / 32) + i / 32];",
                            "int s = scales[n * (K / 32) + (i / 32 + 1) % (K / 32)];", [MX]),
    "ties_to_odd": ("(dist == best_dist && (c % 2) == 0 && (best % 2) != 0)) {\n            best = c;\n            best_dist = dist;\n        }\n    }\n    return best;\n}\n\n/* OCP-MX conversion of one 32-element block",
                    "(dist == best_dist && (c % 2) != 0 && (best % 2) == 0)) {\n            best = c;\n            best_dist = dist;\n        }\n    }\n    return best;\n}\n\n/* OCP-MX conversion of one 32-element block", [MX]),
    "scale_exponent_from_log2f": ("s = (e2 - 1) - 2 + 127;",
                                  "s = (int)floorf(log2f(amax)) - 2 + 127;", [MX]),
    "router_bias_dropped": ("if (bias) acc += bias[e];", "(void)bias;", [ROUTE]),
    "ties_to_higher_index": ("return le > lf || (le == lf && e < f);",
                             "return le > lf || (le == lf && e > f);", [ROUTE]),
    "softmax_not_normalised": ("w[t * k + j] = z[j] / sum;", "w[t * k + j] = z[j];", [ROUTE]),
    "histogram_drops_last": ("for (int64_t a = 0; a < T * k; a++) counts[idx[a]] += 1;",
                             "for (int64_t a = 0; a + 1 < T * k; a++) counts[idx[a]] += 1;",
                             [ROUTE]),
    "offsets_ignore_local_begin": ("off[i + 1] = off[i] + counts[e0 + i];",
                                   "off[i + 1] = off[i] + counts[i];", [ROUTE, LAYER]),
    "permute_descending_tokens": ("    for (int64_t t = 0; t < T; t++) {\n        for (int64_t j = 0; j < k; j++) {\n            int64_t le = (int64_t)idx[t * k + j] - e0;\n            if (le < 0 || le >= n_local) {",
                                  "    for (int64_t t = T - 1; t >= 0; t--) {\n        for (int64_t j = 0; j < k; j++) {\n            int64_t le = (int64_t)idx[t * k + j] - e0;\n            if (le < 0 || le >= n_local) {",
                                  [ROUTE]),
    "silu_on_up": ("float silu = g / (1.0f + expf(-g));\n        return silu * u;",
                   "float silu = u / (1.0f + expf(-u));\n        return silu * g;", [LAYER]),
    "gate_reads_up_weights": ("for (int64_t i = 0; i < d; i++) g += xt[i] * wg[n * d + i];",
                              "for (int64_t i = 0; i < d; i++) g += xt[i] * wu[n * d + i];",
                              [LAYER]),
    "down_weights_transposed": ("for (int64_t n = 0; n < I; n++) acc += h[n] * wd[m * I + n];\n        y[m] = acc;",
                                "for (int64_t n = 0; n < I; n++) acc += h[n] * wd[(n * d + m) % (d * I)];\n        y[m] = acc;",
                                [LAYER]),
    "combine_unweighted": ("acc += w[t * k + j] * y[(int64_t)r * d + m];",
                           "acc += y[(int64_t)r * d + m];", [LAYER, ROUTE]),
    "lora_scale_dropped": ("out[n] = base + scale * delta;", "out[n] = base + delta;", [LORA]),
    "lora_factor_transposed": ("delta += t[j] * bf16_bits_to_float(B[n * r + j]);",
                               "delta += t[j] * bf16_bits_to_float(B[(j * N + n) % (N * r)]);",
                               [LORA]),
    "e4m3_emax_7": ("s = (e2 - 1) - 8 + 127;", "s = (e2 - 1) - 7 + 127;", [MX8]),
    "e2m3_emax_3": ("s = (e2 - 1) - emax_e2m3 + 127;", "s = (e2 - 1) - 3 + 127;", [FP6]),
    "e2m3_subnormal_step": ("(float)m / 8.0f : ldexpf(1.0f + (float)m / 8.0f, e - 1);",
                            "(float)m / 4.0f : ldexpf(1.0f + (float)m / 8.0f, e - 1);", [FP6]),
    "e2m3_ties_to_odd": ("(dist == best_dist && (c % 2) == 0 && (best % 2) != 0)) {\n            best = c;\n            best_dist = dist;\n        }\n    }\n    return best;\n}\n\n/* OCP-MX conversion of [N, K] fp32 to MXFP6",
                         "(dist == best_dist && (c % 2) != 0 && (best % 2) == 0)) {\n            best = c;\n            best_dist = dist;\n        }\n    }\n    return best;\n}\n\n/* OCP-MX conversion of [N, K] fp32 to MXFP6", [FP6]),
    "e2m3_clamp_at_7": ("int mag = (a >= 7.5f) ? 31 : e2m3_round_magnitude(a);",
                        "int mag = (a >= 7.0f) ? 31 : e2m3_round_magnitude(a);", [FP6]),
    "fp6x2_plane2_of_value": ("for (int64_t i = 0; i < N * K; i++) r[i] = v[i] - d1[i];",
                              "for (int64_t i = 0; i < N * K; i++) r[i] = v[i] + 0.0f * d1[i];",
                              [FP6]),
}


def _build(src_text, out):
    with tempfile.NamedTemporaryFile("w", suffix=".c", delete=False) as f:
        f.write(src_text)
        c = f.name
    try:
        subprocess.check_call(["gcc", *oracle.CFLAGS, c, "-lm", "-o", str(out)])
    finally:
        os.unlink(c)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    text, repl, files = MUTANTS[name]
    src = SRC.read_text()
    assert src.count(text) == 1, f"{name}: the mutated text must occur exactly once"
    lib = tmp_path / "liboracle_mutant.so"
    _build(src.replace(text, repl), lib)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 1, f"{name}: no pin failed\n{r.stdout[-2000:]}"


def test_unmodified_build_passes_the_same_pins(tmp_path):
    """The control: the same build and run of the unmodified source pass, so
    a mutant's failure is the planted mistake's doing."""
    lib = tmp_path / "liboracle_control.so"
    _build(SRC.read_text(), lib)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", MX, ROUTE, LORA, MX8, FP6], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
