"""Pins of the oracle's 1x128 activation quantiser.

The quantiser turns fp32 (or bf16) activations into the GEMM's LHS: per row
and 128-wide K block, s = amax / 448 in fp32 (rkmt.cn walkthrough, §5.2) and
codes = e4m3 round-to-nearest-even of x / s (lpnh.cn article, §6.3), one scale
per 1x128 tile (hotdry.top, "fine-grained scaling core design").

What fixes it, other than itself:
  * the e4m3 grid: every midpoint between adjacent codes, and its fp32
    neighbours on either side, against the decode table of torch's
    float8_e4m3fn cast (a library routine);
  * torch's own fp32 -> float8_e4m3fn cast through the generator (whose
    encoder is itself pinned against an independent numpy encoder);
  * invariants: a code of magnitude 448 in every non-zero block, s equal to
    the fp32 quotient amax / 448, reconstruction within half a code step;
  * bf16 inputs equal the fp32 path on the widened values;
  * brute force on a single block equals the block inside a larger array;
  * planted mistakes in copies of the oracle source each fail a check above.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from synth import gen

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


def e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def with_unit_scale(values: np.ndarray, amax: float = 448.0) -> np.ndarray:
    """Rows of 128 whose first entry is amax (448 gives s = 1 exactly, so
    x / s = x), followed by the values under test."""
    n = len(values)
    per = 127
    rows = -(-n // per)
    x = np.zeros((rows, 128), np.float32)
    x[:, 0] = amax
    flat = np.zeros(rows * per, np.float32)
    flat[:n] = values
    x[:, 1:] = flat.reshape(rows, per)
    return x


def codes_of(values, quantize=oracle.quantize_1x128):
    x = with_unit_scale(np.asarray(values, np.float32))
    q, s = quantize(x)
    assert np.all(s == 1.0)
    return q[:, 1:].reshape(-1)[:len(values)]


def grid_cases():
    """Midpoints of adjacent finite e4m3 values and the fp32 values just
    below and above them, for both signs, with the expected codes."""
    tab = e4m3_table()
    vals, want = [], []
    for c in range(0x7E):
        lo, hi = tab[c], tab[c + 1]
        mid = np.float32((lo + hi) / 2)            # exact: at most 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(-np.inf), dtype=np.float32)
        above = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
        for v, code in ((mid, even), (below, c), (above, c + 1), (np.float32(lo), c)):
            vals += [v, -v]
            want += [code, code | 0x80]
    vals += [np.float32(448.0), np.float32(-448.0), np.float32(0.0), np.float32(-0.0)]
    want += [0x7E, 0xFE, 0x00, 0x80]
    return np.array(vals, np.float32), np.array(want, np.uint8)


DIVISION_AMAX = np.float32(3.3)


def division_cases(amax=DIVISION_AMAX):
    """Inputs x whose fp32 quotient x / s lands exactly on a midpoint between
    two e4m3 values while x times the fp32 reciprocal of s does not: the
    quantiser must divide (s = amax / 448 is not a power of two here).
    Returns the inputs and the expected (even) codes."""
    tab = e4m3_table()
    s = np.float32(amax) / np.float32(448.0)
    r = np.float32(1.0) / s
    vals, want = [], []
    for c in range(1, 0x7D):
        mid = np.float32((tab[c] + tab[c + 1]) / 2)
        x = np.float32(mid * s)
        for _ in range(4):
            x = np.nextafter(x, np.float32(-np.inf), dtype=np.float32)
        for _ in range(9):
            if np.float32(x / s) == mid and np.float32(x * r) != mid:
                vals.append(x)
                want.append(c if c % 2 == 0 else c + 1)
            x = np.nextafter(x, np.float32(np.inf), dtype=np.float32)
    return np.array(vals, np.float32), np.array(want, np.uint8)


def test_encode_hand_values():
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie between 1 and 1.125 -> even (1.0)
    assert oracle.e4m3_encode(1.1875) == 0x3A          # tie between 1.125 and 1.25 -> even (1.25)
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # half the smallest subnormal -> 0
    assert oracle.e4m3_encode(3 * 2.0 ** -11) == 0x01  # 1.5 x 2^-10 -> 2^-9
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(-448.0) == 0xFE
    assert oracle.e4m3_encode(-1e-9) == 0x80           # sign kept on a value that rounds to zero
    assert oracle.e4m3_encode(460.0) == 0x7E           # beyond 448: clamped


def test_quantiser_on_the_e4m3_grid():
    vals, want = grid_cases()
    got = codes_of(vals)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_quantiser_divides_by_the_scale():
    vals, want = division_cases()
    assert len(vals) >= 20
    x = with_unit_scale(vals, DIVISION_AMAX)
    q, s = oracle.quantize_1x128(x)
    assert np.all(s == np.float32(DIVISION_AMAX) / np.float32(448.0))
    got = q[:, 1:].reshape(-1)[:len(vals)]
    assert np.array_equal(got, want)


def test_quantiser_matches_torch_cast_generator():
    rng = np.random.Generator(np.random.PCG64(7))
    x = gen.normal_with_outliers(rng, (96, 1152))
    x[5, 256:384] = 0.0                               # all-zero block
    x[6, 0:128] = -0.0                                 # all negative zeros
    x[7, 128:256] *= np.float32(1e-30)                 # tiny block: tiny scale
    x[8, 512:640] *= np.float32(1e30)                  # huge block
    q, s = oracle.quantize_1x128(x)
    q2, s2 = gen.quantize_lhs(x)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(q, q2)
    assert s[5, 2] == 1.0 and np.all(q[5, 256:384] == 0)
    assert s[6, 0] == 1.0 and np.all(q[6, 0:128] == 0x80)


def test_quantiser_invariants():
    rng = np.random.Generator(np.random.PCG64(8))
    x = gen.normal_with_outliers(rng, (40, 768))
    q, s = oracle.quantize_1x128(x)
    tab = e4m3_table()
    blocks_x = x.reshape(40, 6, 128).astype(np.float64)
    blocks_q = q.reshape(40, 6, 128)
    amax = np.abs(x.reshape(40, 6, 128)).max(axis=2)
    assert np.array_equal(s, amax / np.float32(448.0))        # fp32 quotient
    assert np.all((blocks_q & 0x7F).max(axis=2) == 0x7E)     # the amax element maps to 448
    rec = tab[blocks_q] * s[:, :, None].astype(np.float64)
    # half the spacing of the code's binade (subnormals share 2^-9's step), times s
    mag = np.abs(tab[blocks_q])
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
    half_step = np.ldexp(1.0, (e - 4).astype(int)) * s[:, :, None]
    assert np.all(np.abs(blocks_x - rec) <= half_step * (1 + 1e-6))


def test_bf16_input_equals_fp32_path():
    rng = np.random.Generator(np.random.PCG64(9))
    xb = torch.from_numpy(gen.normal_with_outliers(rng, (24, 640))).to(torch.bfloat16)
    q1, s1 = oracle.quantize_1x128(xb)
    q2, s2 = oracle.quantize_1x128(xb.to(torch.float32).numpy())
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_blocks_are_independent():
    rng = np.random.Generator(np.random.PCG64(10))
    x = gen.normal_with_outliers(rng, (5, 512))
    q, s = oracle.quantize_1x128(x)
    for m in range(5):
        for kb in range(4):
            qb, sb = oracle.quantize_1x128(x[m:m + 1, 128 * kb:128 * kb + 128])
            assert np.array_equal(qb[0], q[m, 128 * kb:128 * kb + 128]) and sb[0, 0] == s[m, kb]


# ---------------------------------------------------------------- planted mistakes

def load_mutant(tmp_path, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           str(path), "-o", str(so), "-lm"])
    return ctypes.CDLL(str(so))


def mutant_quantize(lib):
    def quantize(x):
        x = np.ascontiguousarray(x, np.float32)
        M, K = x.shape
        q = np.zeros((M, K), np.uint8)
        s = np.zeros((M, K // 128), np.float32)
        i64 = ctypes.c_int64
        lib.dgo_quantize_1x128(ctypes.c_void_p(x.ctypes.data), ctypes.c_int(0), i64(K), i64(M), i64(K),
                               ctypes.c_void_p(q.ctypes.data), i64(K), ctypes.c_void_p(s.ctypes.data),
                               i64(K // 128), i64(1), ctypes.c_int(1))
        return q, s
    return quantize


MUTANTS = {
    "ties away from zero": ("(err == best_err && (c & 1) == 0 && (best & 1) == 1)", "(err == best_err)"),
    "truncation": ("double err = fabs(dec_table[c] - a);",
                   "double err = dec_table[c] <= a ? a - dec_table[c] : 1e300;"),
    "scale inverted": ("amax / 448.0f;", "448.0f / amax;"),
    "sign dropped": ("(signbit(v) ? (0x80 | best) : best)", "(v < 0 ? (0x80 | best) : best)"),
    "multiply by reciprocal": ("load_x(X, is_bf16, m * ldx + k) / s;",
                               "load_x(X, is_bf16, m * ldx + k) * (1.0f / s);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(tmp_path, name):
    lib = load_mutant(tmp_path, *MUTANTS[name])
    quantize = mutant_quantize(lib)
    failures = 0
    vals, want = grid_cases()
    failures += int(not np.array_equal(codes_of(vals, quantize), want))
    dvals, dwant = division_cases()
    dq, _ = quantize(with_unit_scale(dvals, DIVISION_AMAX))
    failures += int(not np.array_equal(dq[:, 1:].reshape(-1)[:len(dvals)], dwant))
    rng = np.random.Generator(np.random.PCG64(7))
    x = gen.normal_with_outliers(rng, (64, 1024))
    x[6, 0:128] = -0.0
    q, s = quantize(x)
    q2, s2 = gen.quantize_lhs(x)
    failures += int(not (np.array_equal(q, q2) and np.array_equal(s, s2)))
    assert failures > 0, name
