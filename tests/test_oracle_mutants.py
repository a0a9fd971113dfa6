"""Sensitivity of the oracle's pins: each case plants one plausible mistake in a temporary copy of
oracle.c (on the CPU), builds it, and runs the pin suite against it, which must fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "decode_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "subnormal_quantum": ("v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),
    "rounding_truncates": ("nearbyint(ldexp(ax, -unit_exp))", "trunc(ldexp(ax, -unit_exp))"),
    "bf16_no_subnormal_range": ("if (e2 - 1 < -126) unit_exp = -126 - 7;", ""),
    "block_sum_drops_last_term": ("k1 = k0 + 128 < K ? k0 + 128 : K;", "k1 = (k0 + 128 < K ? k0 + 128 : K) - 1;"),
    "sa_index_fixed_block": ("double s = (double)sa_row[kb] * (double)sb_row[kb];",
                             "double s = (double)sa_row[0] * (double)sb_row[kb];"),
    "sb_block_from_k_not_n": ("sb + (n / 128) * nkb, K);", "sb + 0 * nkb, K);"),
    "fp32_accumulation": ("acc = fma(s, block, acc);", "acc = (float)(acc + (float)(s * block));"),
    "encode_ties_away": ("double q = nearbyint(ldexp(ax, 3 - E));", "double q = round(ldexp(ax, 3 - E));"),
    "encode_subnormal_quantum": ("double f = nearbyint(ldexp(ax, 9));", "double f = nearbyint(ldexp(ax, 10));"),
    "encode_zero_sign_lost": ("uint8_t sign = signbit(x) ? 0x80 : 0;", "uint8_t sign = x < 0 ? 0x80 : 0;"),
    "encode_binade_carry_lost": ("if (q == 16.0) { q = 8.0; ++E; }", ""),
    "quant_floor_dropped": ("if (amax < floor_amax) amax = floor_amax;", ""),
    "quant_scale_divisor": ("float s = (float)((double)amax / 448.0);", "float s = (float)((double)amax / 240.0);"),
    "quant_sa_transposed": ("sa[m * nkb + kb] = s;", "sa[kb * M + m] = s;"),
    "quant_multiplies_by_reciprocal": ("float v = (float)((double)xs[k] / (double)s);",
                                       "float v = xs[k] * (1.0f / s);"),
    "quant_amax_skips_last": ("if (a > amax) amax = a;", "if (a > amax && k + 1 < n) amax = a;"),
    "swiglu_halves_swapped": ("const uint16_t* up = gate + I;\n", "const uint16_t* up = gate; gate += I;\n"),
    "swiglu_sigmoid_not_silu": ("double silu = (double)g / (1.0 + exp(-(double)g));",
                                "double silu = 1.0 / (1.0 + exp(-(double)g));"),
    "swiglu_sign_of_exponent": ("double silu = (double)g / (1.0 + exp(-(double)g));",
                                "double silu = (double)g / (1.0 + exp((double)g));"),
    "fp4_nibble_order_swapped": ("Bd[i] = e2m1[(i & 1) ? (byte >> 4) : (byte & 0xF)];",
                                 "Bd[i] = e2m1[(i & 1) ? (byte & 0xF) : (byte >> 4)];"),
    "fp4_scale_per_64_values": ("block += oracle_e8m0_value(srow[k0 / 32]) * sub;",
                                "block += oracle_e8m0_value(srow[k0 / 64]) * sub;"),
    "e2m1_subnormal_quantum": ("double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);",
                               "double v = (e == 0) ? 0.25 * m : ldexp(1.0 + 0.5 * m, e - 1);"),
    "e8m0_bias": ("ldexp(1.0, (int)s - 127)", "ldexp(1.0, (int)s - 128)"),
    "swiglu_activation_perturbed": ("xs[k - k0] = (float)v;", "xs[k - k0] = (float)v * 1.0000001f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new)
    c = tmp_path / "oracle_mutant.c"
    so = tmp_path / "liboracle_mutant.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %s was not caught:\n%s" % (name, r.stdout[-2000:])
