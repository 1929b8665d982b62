"""Mutation check of the oracle's pins (CPU only).

Plants one plausible slip at a time into a copy of oracle/nvfp4_oracle.c,
builds it into a temporary library, and runs the pin tests against it: every
planted slip must make at least one pin fail.  The oracle source itself is
never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "nvfp4_oracle.c")

# (name, text to find, replacement) -- each find string must occur in the source
PLANTS = [
    ("nibble order swapped", "return (k & 1) ? (b >> 4) : (b & 0xF);",
     "return (k & 1) ? (b & 0xF) : (b >> 4);"),
    ("block index k/32", "return ws[n * (K / 16) + k / 16];", "return ws[n * (K / 16) + k / 32];"),
    ("E4M3 exponent bias 8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("E4M3 subnormal exponent", "ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    ("E2M1 subnormal 1.0", "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);",
     "double mag = (e == 0) ? 1.0 * m : ldexp(1.0 + 0.5 * m, e - 1);"),
    ("E2M1 sign dropped", "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);\n  return s ? -mag : mag;",
     "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);\n  return mag;"),
    ("global scale multiplied", "nvfp4_oracle_e4m3(scale_at(ws, K, n, k)) / g;",
     "nvfp4_oracle_e4m3(scale_at(ws, K, n, k)) * g;"),
    ("row stride K/4", "uint8_t b = wq[n * (K / 2) + k / 2];", "uint8_t b = wq[n * (K / 4) + k / 2];"),
    ("abs sum drops fabs", "mag += fabs(t);", "mag += t;"),
    ("x row index", "double t = bf16_to_double(x[m * K + k]) * weight_at(wq, ws, gd, K, n, k);\n        acc += t;\n        mag += fabs(t);\n      }\n      y[m * N + n] = acc;",
     "double t = bf16_to_double(x[k]) * weight_at(wq, ws, gd, K, n, k);\n        acc += t;\n        mag += fabs(t);\n      }\n      y[m * N + n] = acc;"),
]

PLANTS += [
    ("bf16 rounding truncates", "const double r = nearbyint(ldexp(a, -qe));",
     "const double r = floor(ldexp(a, -qe));"),
    ("bf16 keeps 9 bits", "const int qe = (e - 1 >= -126) ? e - 8 : -133;",
     "const int qe = (e - 1 >= -126) ? e - 9 : -133;"),
]

PIN_TESTS = [
    pins.test_e2m1_matches_ocp_table,
    pins.test_e4m3_matches_torch_all_codes,
    pins.test_dequant_layout_positions,
    pins.test_gemm_hand_example,
    lambda: pins.test_gemm_bruteforce_exact(2, 3, 32, 1),
    lambda: pins.test_gemm_bruteforce_exact(3, 4, 64, 2),
    pins.test_bf16_rne_matches_torch_cast,
    pins.test_mlp_bruteforce,
]


@pytest.mark.parametrize("name,find,repl", PLANTS, ids=[p[0] for p in PLANTS])
def test_planted_slip_is_caught(tmp_path, name, find, repl):
    src = open(SRC).read()
    assert src.count(find) >= 1, f"plant site for '{name}' not found"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(find, repl, 1))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(mutant), "-lm"], check=True)
    caught = []
    with oracle.use_library(str(lib)):
        for t in PIN_TESTS:
            try:
                t()
            except AssertionError:
                caught.append(t)
    assert caught, f"no pin caught the planted slip '{name}'"
