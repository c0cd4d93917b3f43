"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies oracle/paro_ref.c, plants one plausible mistake (a dropped
term, a wrong sign, index, operand or order), compiles the copy with gcc and
runs the pin suite (tests/test_oracle_pins.py) against it in a subprocess.
The suite must fail for every mutant: that is what makes the pins a check of
the oracle rather than of themselves.
"""
import os
import subprocess
import sys

import pytest

from oracle import ref

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "b_prime_sign": ("row[j] = -a * s + b * c;", "row[j] = a * s + b * c;"),
    "a_prime_sign": ("row[i] = a * c + b * s;", "row[i] = a * c - b * s;"),
    "aliased_update": ("row[j] = -a * s + b * c;", "row[j] = -row[i] * s + b * c;"),
    "theta_group_offset": ("g * (G / 2) + p;", "p;"),
    "pair_members_swapped": (
        "const int64_t i = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p];\n"
        "        const int64_t j = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p + 1];",
        "const int64_t i = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p + 1];\n"
        "        const int64_t j = g * G + L->pairs[(int64_t)t * I + g * G + 2 * p];"),
    "stage_order_reversed": ("for (int t = 0; t < L->krot; ++t) {\n    for (int64_t g = 0; g < ngroups",
                             "for (int t = L->krot - 1; t >= 0; --t) {\n    for (int64_t g = 0; g < ngroups"),
    "channel_scale_divides": ("row[k] = load_elem(x, x_dt, m * I + k) * (double)L->channel_scales[k];",
                              "row[k] = load_elem(x, x_dt, m * I + k) / (double)L->channel_scales[k];"),
    "awq_order_sequential": ("{0, 4, 1, 5, 2, 6, 3, 7}", "{0, 1, 2, 3, 4, 5, 6, 7}"),
    "zero_not_subtracted": ("(double)(q - z) * s;", "(double)(q) * s;"),
    "bias_dropped": ("y_out[m * O + n0 + n] = acc[n] + b;", "y_out[m * O + n0 + n] = acc[n];"),
    "group_index_transposed": ("const int64_t g = k / G;", "const int64_t g = k % (I / G);"),
    "f16_exponent_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "rounding_ties_away": ("return rint(a / quantum) * quantum;", "return round(a / quantum) * quantum;"),
    "bf16_fraction_bits": ("ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    "quant_zero_outside_range": ("double xmin = 0.0, xmax = 0.0;", "double xmin = x[0], xmax = x[0];"),
    "quant_ties_away": ("double q = rint(x[e] / scale) + zero;", "double q = round(x[e] / scale) + zero;"),
    "quant_sym_zero": ("(maxq + 1.0) / 2.0", "maxq / 2.0"),
    "quant_steps_16": ("double scale = (xmax - xmin) / maxq;", "double scale = (xmax - xmin) / (maxq + 1.0);"),
    "quant_affine_zero_sign": ("rint(-xmin / scale)", "rint(xmin / scale)"),
    "quant_sym_one_sided": ("if (xmin < 0.0) xmin = -xmax;", ""),
    "quant_no_sentinel": ("xmin = -1.0;\n        xmax = 1.0;", "xmin = 0.0;\n        xmax = 0.0;"),
    "quant_no_lower_bound": ("if (scale < 1e-5) scale = 1e-5;", ""),
    "transform_multiplies": ("/ (double)L->channel_scales[k];", "* (double)L->channel_scales[k];"),
    "pack_sequential_slots": ("<< (4 * SLOT_OF_COL[j]);\n      qweight", "<< (4 * j);\n      qweight"),
    "bwd_theta_sign": ("gth[ang] += ga * out[j] - gb * out[i];", "gth[ang] += ga * out[j] + gb * out[i];"),
    "bwd_theta_pre_stage": ("gth[ang] += ga * out[j] - gb * out[i];",
                            "gth[ang] += ga * states[(size_t)t * I + j] - gb * states[(size_t)t * I + i];"),
    "bwd_grad_sign": ("grad[i] = ga * c - gb * sn;", "grad[i] = ga * c + gb * sn;"),
    "bwd_stage_order": ("for (int t = krot - 1; t >= 0; --t) {", "for (int t = 0; t < krot; ++t) {"),
    "bwd_cs_uses_scaled": ("gc[k] += grad[k] * xk;", "gc[k] += grad[k] * xk * (double)L->channel_scales[k];"),
    "pack_zeros_sequential": ("<< (4 * SLOT_OF_COL[j]);\n      qzeros", "<< (4 * j);\n      qzeros"),
    "mx_exponent_off_by_one": ("biased = (ex - 1) - 2 + 127;", "biased = (ex - 1) - 1 + 127;"),
    "mx_ties_to_odd": ("(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    "mx_nibble_order": ("(uint8_t)(c[0] | (c[1] << 4));", "(uint8_t)(c[1] | (c[0] << 4));"),
    "mx_sign_dropped": ("c[h] = (q < 0.0 && m != 0) ? (m | 8) : m;", "c[h] = m;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    with open(ref.SRC_PATH) as f:
        src = f.read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique/present"
    mutant_src = tmp_path / "paro_ref_mutant.c"
    assert find in src, f"mutant {name}: its target text is not in the oracle"
    mutant_src.write_text(src.replace(find, repl))
    lib = tmp_path / "libparo_ref_mutant.so"
    ref.build(str(lib), str(mutant_src))
    env = dict(os.environ, PARO_REF_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    # exit code 1 = some pin failed (not a crash or a collection error)
    assert r.returncode == 1, f"mutant {name}: pytest exit {r.returncode}:\n{r.stdout[-2000:]}"
