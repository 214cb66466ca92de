"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.

Each mutant is the oracle source with one edit; it is compiled to a temporary
library and the whole pin module is run against it in a subprocess.  A mutant
that survives means a pin is missing.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

FMA = "acc = fmaf(elem_f32(x, x_dt, (size_t)t * H + h), elem_f32(w, w_dt, (size_t)e * H + h), acc);"
MUTANTS = {
    "router_drops_last_term": ("for (int h = 0; h < H; h++)\n                " + FMA,
                               "for (int h = 0; h < H - 1; h++)\n                " + FMA),
    "router_mul_then_add": (FMA, "acc = elem_f32(x, x_dt, (size_t)t * H + h) * elem_f32(w, w_dt, (size_t)e * H + h) + acc;"),
    "router_descending_order": ("for (int h = 0; h < H; h++)\n                " + FMA,
                                "for (int h = H - 1; h >= 0; h--)\n                " + FMA),
    "router_ignores_bias": ("acc = acc + bias[e];", "acc = acc + 0.0f;"),
    "topk_ties_to_higher_index": ("l[e] > l[best]", "l[e] >= l[best]"),
    "gates_not_renormalised": ("gates[j] = (float)(u[j] / sum);", "gates[j] = (float)(u[j] / (sum + 1e-3));"),
    "silu_sign": ("exp(-G)", "exp(G)"),
    "gate_up_swapped": ("size_t rg = (le * 2 * I + i) * (size_t)H, ru = (le * 2 * I + I + i) * (size_t)H;",
                        "size_t ru = (le * 2 * I + i) * (size_t)H, rg = (le * 2 * I + I + i) * (size_t)H;"),
    "h_not_rounded": ("hb[i] = round_h ? (double)bf16_bits_to_float(oracle_bf16_round(hf)) : (double)hf;",
                      "hb[i] = (double)hf;"),
    "permute_tokens_descending": ("for (int t = 0; t < T; t++) {\n        for (int j = 0; j < k; j++) {\n            size_t a",
                                  "for (int t = T - 1; t >= 0; t--) {\n        for (int j = 0; j < k; j++) {\n            size_t a"),
    "fp8_down_scale_dropped": ("o *= (double)s_down[le * H + n];", "o *= 1.0;"),
    "fp8_gate_scale_wrong_channel": ("G *= (double)s_gate_up[le * 2 * I + i];", "G *= (double)s_gate_up[le * 2 * I + I + i];"),
    "e4m3_subnormal_exponent": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "down_weight_transposed": ("o += hb[i] * elem(w_down, w_dt, rd + i);",
                               "o += hb[i] * elem(w_down, w_dt, le * (size_t)H * I + (size_t)i * H + n);"),
    "bf16_round_truncates": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)((u + 0u * lsb) >> 16);"),
    "combine_ignores_gate": ("acc += (double)topk_w[(size_t)t * k + j] * (double)y_perm[(size_t)r * H + n];",
                             "acc += (double)y_perm[(size_t)r * H + n];"),
    "mx_emax_7": ("int s = ex - 1 - 8 + 127;", "int s = ex - 1 - 7 + 127;"),
    "e4m3_ties_away_from_zero": ("(lo & 1) ? hi : lo", "hi"),
    "e4m3_overflow_to_nan": ("        return sign | 126;\n    int lo", "        return sign | 127;\n    int lo"),
    "mx_x_not_quantised": ("xq[32 * b + i] = ldexp(oracle_e4m3_value(codes[i]), (int)sb - 127);",
                           "xq[32 * b + i] = xv[32 * b + i];"),
    "mx_h_not_quantised": ("hq[32 * b + i] = ldexp(oracle_e4m3_value(codes[i]), (int)sb - 127);",
                           "hq[32 * b + i] = hv[32 * b + i];"),
    "mx_weight_scale_wrong_block": ("const double f = ldexp(1.0, (int)sc[b] - 127);",
                                    "const double f = ldexp(1.0, (int)sc[(b + 1) % (K / 32)] - 127);"),
    "mx_weight_scale_bias_126": ("const double f = ldexp(1.0, (int)sc[b] - 127);",
                                 "const double f = ldexp(1.0, (int)sc[b] - 126);"),
    "mx_table_drops_subnormals": ("e4m3_tab[c] = oracle_e4m3_value((uint8_t)c);",
                                  "e4m3_tab[c] = (c & 0x78) ? oracle_e4m3_value((uint8_t)c) : 0.0;"),
    "mx_weight_row_misread": ("const uint8_t *q = codes + row * (size_t)K;",
                              "const uint8_t *q = codes + (row ^ 1) * (size_t)K;"),
    "shared_up_rows_misplaced": ("size_t rg = (size_t)i * H, ru = (size_t)(I_s + i) * H;",
                                 "size_t rg = (size_t)i * H, ru = (size_t)(I_s / 2 + i) * H;"),
    "shared_silu_dropped": ("float hf = (float)(G / (1.0 + exp(-G)) * U);", "float hf = (float)(G * U);"),
    "shared_fp8_down_scale_dropped": ("o *= (double)s_down[n];", "o *= 1.0;"),
    "shared_down_row_stride": ("o += hb[i] * elem(w_down, w_dt, (size_t)n * I_s + i);",
                               "o += hb[i] * elem(w_down, w_dt, (size_t)i * H + n);"),
    "combine_gate_added_not_multiplied": ("acc += (double)topk_w[(size_t)t * k + j] * (double)y_perm[(size_t)r * H + n];",
                                          "acc += (double)topk_w[(size_t)t * k + j] + (double)y_perm[(size_t)r * H + n];"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path_c = os.path.join(tmp, name + ".c")
    path_so = os.path.join(tmp, name + ".so")
    open(path_c, "w").write(src.replace(old, new, 1))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           "-o", path_so, path_c, "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIBRARY=path_so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-400:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            res = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp), MUTANTS)))
    survivors = {n: out for n, (rc, out) in res.items() if rc == 0}
    assert not survivors, f"mutants not caught by any pin: {list(survivors)}"
    # a failure must be a test failure (pytest exit code 1), not a crash or collection error
    odd = {n: (rc, out) for n, (rc, out) in res.items() if rc != 1}
    assert not odd, odd
