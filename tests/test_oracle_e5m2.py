"""Pins of the oracle's e5m2 operand path (e4m3 x e5m2, e5m2 x e4m3, e5m2 x e5m2).

e5m2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, largest finite
57344, infinities and NaNs (rkmt.cn walkthrough §2.1; mixing e4m3 A with
e5m2 B: lpnh.cn article §2.1). Fixed by: torch's float8_e5m2 cast (decode of
all 256 codes), exact Python integer sums of every block, the e4m3-only
oracle (which the format path must reproduce bit for bit), a brute-force
fp64 matmul of the dequantised operands, hand-worked cases, an independent
numpy encoder for the generator, and planted mistakes.
"""
import ctypes
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.test_oracle_quant import ORACLE_SRC

FMT_CASES = [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


def torch_table(fmt):
    dtype = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dtype).to(torch.float64).numpy()


def test_e5m2_spot_values():
    assert oracle.e5m2_decode(0x3C) == 1.0
    assert oracle.e5m2_decode(0x3E) == 1.5
    assert oracle.e5m2_decode(0x7B) == 57344.0
    assert oracle.e5m2_decode(0xFB) == -57344.0
    assert oracle.e5m2_decode(0x01) == 2.0 ** -16
    assert oracle.e5m2_decode(0x04) == 2.0 ** -14
    assert oracle.e5m2_decode(0x7C) == np.inf and oracle.e5m2_decode(0xFC) == -np.inf
    assert np.isnan(oracle.e5m2_decode(0x7D)) and np.isnan(oracle.e5m2_decode(0xFF))


def test_e5m2_all_codes_match_torch_cast():
    ref = torch_table("e5m2")
    ours = np.array([oracle.e5m2_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def exact_block(a, fa, b, fb):
    """Python-integer block sum, rounded once to binary64 (float() of a Fraction rounds to nearest)."""
    ta, tb = torch_table(fa), torch_table(fb)
    sa, sb = (9 if fa == "e4m3" else 16), (9 if fb == "e4m3" else 16)
    total = sum(int(ta[x] * 2 ** sa) * int(tb[y] * 2 ** sb) for x, y in zip(a, b))
    return float(Fraction(total, 2 ** (sa + sb)))


def finite_codes(fmt):
    t = torch_table(fmt)
    return np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)


@pytest.mark.parametrize("fa,fb", FMT_CASES + [("e4m3", "e4m3")])
def test_block_partial_is_the_exact_sum_rounded_once(fa, fb):
    rng = np.random.default_rng(3)
    ca, cb = finite_codes(fa), finite_codes(fb)
    for _ in range(40):
        a, b = rng.choice(ca, 128), rng.choice(cb, 128)
        assert oracle.block_partial_fmt(a, fa, b, fb) == exact_block(a, fa, b, fb)
    big_a = np.full(128, 0x7B if fa == "e5m2" else 0x7E, np.uint8)
    big_b = np.full(128, 0x7B if fb == "e5m2" else 0x7E, np.uint8)
    assert oracle.block_partial_fmt(big_a, fa, big_b, fb) == exact_block(big_a, fa, big_b, fb)
    # cancellation: a huge product and its negative leave the small ones behind
    a = rng.choice(ca, 128)
    a[0], a[1] = big_a[0], big_a[0] | 0x80
    b = rng.choice(cb, 128)
    b[1] = b[0] = big_b[0]
    assert oracle.block_partial_fmt(a, fa, b, fb) == exact_block(a, fa, b, fb)


def test_format_path_reproduces_the_e4m3_oracle():
    p = gen.make_dense(33, 256, 640, 41, 42)
    assert np.array_equal(oracle.gemm_nt_fmt(p.a, "e4m3", p.sa_t.T, p.b, "e4m3", p.sb),
                          oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb))


@pytest.mark.parametrize("fa,fb", FMT_CASES)
def test_gemm_matches_dequantised_matmul(fa, fb):
    p = gen.make_dense(24, 256, 512, 51, 52, fa, fb)
    d, acc = oracle.gemm_nt_fmt(p.a, fa, p.sa_t.T, p.b, fb, p.sb, want_acc=True)
    ta, tb = torch_table(fa), torch_table(fb)
    A = ta[p.a] * np.repeat(p.sa_t.T.astype(np.float64), 128, axis=1)
    B = tb[p.b] * np.repeat(np.repeat(p.sb.astype(np.float64), 128, axis=0), 128, axis=1)
    ref = A @ B.T
    bound = 1e-12 * (np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(acc - ref) <= bound)
    pts, pacc = oracle.gemm_nt_fmt_points(p.a, fa, p.sa_t.T, p.b, fb, p.sb, [0, 5, 23], [0, 130, 255])
    assert np.array_equal(pts, d[[0, 5, 23], [0, 130, 255]])


def test_hand_cases():
    # 57344^2 * 2^-30 * 2^-2 = 49 * 2^-6 = 0.765625 -> bf16 0x3F44
    a = np.zeros((1, 128), np.uint8)
    b = np.zeros((128, 128), np.uint8)
    a[0, 0], b[0, 0] = 0x7B, 0x7B
    sa = np.full((1, 1), 2.0 ** -30, np.float32)
    sb = np.full((1, 1), 2.0 ** -2, np.float32)
    d = oracle.gemm_nt_fmt(a, "e5m2", sa, b, "e5m2", sb)
    assert d[0, 0] == 0x3F44 and np.all(d[0, 1:] == 0)
    # smallest subnormals: e5m2 2^-16 times e4m3 2^-9 = 2^-25 -> bf16 0x3300
    a[0, 0], b[0, 0] = 0x01, 0x01
    d = oracle.gemm_nt_fmt(a, "e5m2", np.ones((1, 1), np.float32), b, "e4m3", np.ones((1, 1), np.float32))
    assert d[0, 0] == 0x3300


def encode_reference(v, ebits, mbits, bias):
    """Independent minifloat encoder: round to nearest, ties to even, |v| <= largest finite."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    emin = 1 - bias
    E = np.maximum(ex - 1, emin)
    quantum = np.ldexp(1.0, E - mbits)
    r = np.rint(a / quantum) * quantum
    _, ex2 = np.frexp(r)
    E2 = np.maximum(ex2 - 1, emin)
    normal = r >= 2.0 ** emin
    mant = np.where(normal, r / np.ldexp(1.0, E2 - mbits) - 2 ** mbits, r / 2.0 ** (emin - mbits))
    code = np.where(normal, ((E2 + bias) << mbits) + mant.astype(np.int64), mant.astype(np.int64))
    code = np.where(r == 0, 0, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_generator_e5m2_encoder_matches_reference():
    rng = np.random.default_rng(4)
    x = (rng.random(1_000_000, dtype=np.float32) * 2 - 1) * np.float32(57344)
    x[:2000] *= np.float32(1e-9)                      # subnormal range
    ours = gen._encode(torch.from_numpy(x.copy()), "e5m2").numpy()
    assert np.array_equal(ours, encode_reference(x, 5, 2, 15))
    fin = finite_codes("e5m2")
    assert np.array_equal(encode_reference(torch_table("e5m2")[fin], 5, 2, 15), fin)


def test_generator_e5m2_blocks_reach_the_format_maximum():
    codes, s = gen.quantize_rhs(gen.normal_with_outliers(np.random.default_rng(5), (256, 512)), "e5m2")
    blocks = codes.reshape(2, 128, 4, 128).transpose(0, 2, 1, 3).reshape(8, -1)
    assert np.all((blocks & 0x7F).max(axis=1) == 0x7B)


MUTANTS = {
    "e5m2 bias 16": ("mag = ldexp((double)(4 + f), e - 17);", "mag = ldexp((double)(4 + f), e - 18);"),
    "e5m2 treated as e4m3": ("double v = fmt ? dgo_e5m2_decode(code) : dgo_e4m3_decode(code);",
                             "double v = dgo_e4m3_decode(code);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, name
    (tmp_path / "m.c").write_text(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(tmp_path / "m.c"),
                           "-o", str(tmp_path / "m.so"), "-lm"])
    lib = ctypes.CDLL(str(tmp_path / "m.so"))
    lib.dgo_block_partial_fmt.restype = ctypes.c_double
    lib.dgo_block_partial_fmt.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    rng = np.random.default_rng(6)
    bad = 0
    for fa, fb in FMT_CASES:
        a, b = rng.choice(finite_codes(fa), 128), rng.choice(finite_codes(fb), 128)
        got = lib.dgo_block_partial_fmt(ctypes.c_void_p(a.ctypes.data), oracle.FMTS[fa],
                                        ctypes.c_void_p(b.ctypes.data), oracle.FMTS[fb])
        bad += got != exact_block(a, fa, b, fb)
    assert bad > 0, name
