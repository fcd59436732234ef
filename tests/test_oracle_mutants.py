"""Planted mistakes in the GEMM oracle each fail at least one of its pins.

Each case compiles a copy of oracle.c with one plausible mistake, swaps it in
for the oracle library, and runs the pins of tests/test_oracle.py (closed
forms, torch's casts, hand-worked cases, exact integer sums, the dequantised
matmul, the per-tensor special case, routing signatures) against it. A pin
set that lets a mutant through would not be fixing that part of the oracle.
The real library is restored afterwards.
"""
import ctypes
import subprocess

import pytest

import oracle
from tests import hand_cases
from tests import test_oracle as pins
from tests.test_oracle_quant import ORACLE_SRC

PIN_CALLS = [
    pins.test_e4m3_spot_values,
    pins.test_e4m3_all_codes_match_torch_cast,
    pins.test_bf16_hand_ties,
    pins.test_block_partial_exact_int64,
    pins.test_single_block_gemm_equals_int64_matmul,
    lambda: pins.test_gemm_matches_dequantised_matmul(64, 256, 512, 1),
    lambda: pins.test_gemm_matches_dequantised_matmul(7, 384, 1024, 2),
    pins.test_per_tensor_special_case_exact,
    pins.test_identity_rhs,
    pins.test_contiguous_routing_signature,
    pins.test_contiguous_matches_dense_per_row,
    pins.test_masked_routing_signature,
    pins.test_masked_matches_dense_per_group,
] + [(lambda c=c: pins.test_hand_cases(c)) for c in hand_cases.load()]

# (first occurrence of `old`) -> `new`
MUTANTS = {
    "sB dropped": ("double scale = (double)sa[kb * sa_kb] * (double)sb[kb * sb_kb];",
                   "double scale = (double)sa[kb * sa_kb];"),
    "sB indexed by n % 128": ("B + n * ldb, sB + (n / BLK) * sb_nb, sb_kb, K);",
                              "B + n * ldb, sB + (n % BLK) * sb_nb, sb_kb, K);"),
    "sA indexed by kb + 1": ("double scale = (double)sa[kb * sa_kb] * (double)sb[kb * sb_kb];",
                             "double scale = (double)sa[((kb + 1) % (K / BLK)) * sa_kb] * (double)sb[kb * sb_kb];"),
    "e4m3 exponent bias 8": ("mag = ldexp((double)(8 + f), e - 10);", "mag = ldexp((double)(8 + f), e - 11);"),
    "e4m3 subnormals as normals": ("mag = ldexp((double)f, -9);", "mag = ldexp((double)(8 + f), -10);"),
    "bf16 truncation": ("double r = rint(a / quantum) * quantum;", "double r = floor(a / quantum) * quantum;"),
    "bf16 ties away": ("double r = rint(a / quantum) * quantum;", "double r = round(a / quantum) * quantum;"),
    "fp32 accumulator": ("double acc = 0.0;\n    for (int64_t kb = 0; kb < K / BLK; ++kb) {\n        double partial = 0.0;",
                         "float acc = 0.0f;\n    for (int64_t kb = 0; kb < K / BLK; ++kb) {\n        double partial = 0.0;"),
    "scale applied once after the loop": ("        acc += partial * scale;\n    }\n    return acc;\n}\n\nstatic void set_threads",
                                          "        acc += partial * (double)sa[0] * (double)sb[0];\n    }\n    return acc;\n}\n\nstatic void set_threads"),
    "contiguous ids off by one": ("            if (e < 0 || e >= G)\n                continue;",
                                  "            if (e < 0 || e > G)\n                continue;"),
    "masked: one row past the count": ("                if (m >= valid_rows(masked_m, g, M_max))\n                    continue;",
                                       "                if (m > valid_rows(masked_m, g, M_max))\n                    continue;"),
    "masked rows from the wrong group": ("double v = element(A + g * a_stride_g + m * lda, sA + g * sa_g + m * sa_m, sa_kb,\n                                   B + g * b_stride_g",
                                         "double v = element(A + g * a_stride_g + m * lda, sA + g * sa_g + m * sa_m, sa_kb,\n                                   B + ((g + 1) % G) * b_stride_g"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert old in src, name
    (tmp_path / "m.c").write_text(src.replace(old, new, 1))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           str(tmp_path / "m.c"), "-o", str(tmp_path / "m.so"), "-lm"])
    mutant = oracle.configure(ctypes.CDLL(str(tmp_path / "m.so")))
    real = oracle.lib()
    failed = []
    oracle._lib = mutant
    try:
        for i, pin in enumerate(PIN_CALLS):
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(i)
    finally:
        oracle._lib = real
    assert failed, "no pin caught: %s" % name


def test_real_oracle_passes_every_pin():
    for pin in PIN_CALLS:
        pin()
