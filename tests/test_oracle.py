"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle with an independent source: the e4m3 and
bf16 bit layouts (closed forms and torch's CPU casts, a library routine),
hand-worked cases, an exact int64 matmul of the integer codes, a brute-force
fp64 matmul of the dequantised inputs (numpy), the per-tensor special case,
and routing signatures for the grouped layouts.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests import hand_cases


def torch_decode_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- e4m3 decode

def test_e4m3_spot_values():
    # Closed form of the e4m3 layout; 448 is the largest finite value.
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x3C) == 1.5
    assert oracle.e4m3_decode(0x40) == 2.0
    assert oracle.e4m3_decode(0x18) == 2.0 ** -4
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0xFE) == -448.0
    v = oracle.e4m3_decode(0x80)
    assert v == 0.0 and np.signbit(v)
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))


def test_e4m3_all_codes_match_torch_cast():
    ref = torch_decode_table()
    ours = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_monotone_and_symmetric():
    pos = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    assert np.all(np.diff(pos) > 0)
    neg = np.array([oracle.e4m3_decode(0x80 | c) for c in range(0x7F)])
    assert np.array_equal(neg, -pos)
    assert pos.max() == 448.0


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_hand_ties():
    assert oracle.bf16_rne(1.0) == 0x3F80
    assert oracle.bf16_rne(1 + 2.0 ** -8) == 0x3F80            # tie -> even (down)
    assert oracle.bf16_rne(1 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert oracle.bf16_rne(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # single rounding
    assert oracle.bf16_rne(-0.390625) == 0xBEC8
    assert oracle.bf16_rne(2.0 ** -18) == 0x3680
    assert oracle.bf16_rne(-0.0) == 0x8000
    assert oracle.bf16_rne(0.0) == 0x0000
    assert oracle.bf16_rne(2.0 ** -133) == 0x0001               # smallest subnormal
    assert oracle.bf16_rne(2.0 ** -134) == 0x0000               # tie to even zero
    assert oracle.bf16_rne(3 * 2.0 ** -134) == 0x0002
    assert oracle.bf16_rne(1e39) == 0x7F80
    assert oracle.bf16_rne(-1e39) == 0xFF80
    b = oracle.bf16_rne(float("nan"))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_bf16_matches_torch_on_fp32_values():
    # fp32 -> bf16 in torch is a single RNE rounding, so on values exactly
    # representable in fp32 it must agree bit for bit.
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_rne(float(x)) for x in f[:40_000]], dtype=np.uint16)
    assert np.array_equal(ours, ref[:40_000])
    # plus values near every bf16 tie
    base = rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint32) << 16
    tie = (base | 0x8000).astype(np.uint32).view(np.float32)
    tie = tie[np.isfinite(tie)]
    ref = torch.from_numpy(tie.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_rne(float(x)) for x in tie], dtype=np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- block partial

def int_codes(codes):
    """e4m3 codes -> exact integers 2^9 * value, through torch's cast."""
    t = torch_decode_table()
    return (t[codes] * 512).astype(np.int64)


def test_block_partial_exact_int64():
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for _ in range(300):
        a = rng.choice(finite, 128)
        b = rng.choice(finite, 128)
        exact = int(np.dot(int_codes(a), int_codes(b)))
        assert oracle.block_partial(a, b) == exact / 2.0 ** 18


def test_block_partial_extremes_exact():
    a = np.full(128, 0x7E, dtype=np.uint8)
    b = np.full(128, 0x7E, dtype=np.uint8)
    assert oracle.block_partial(a, b) == 128 * 448.0 * 448.0
    b2 = b.copy()
    b2[::2] = 0x01
    exact = int(np.dot(int_codes(a), int_codes(b2)))
    assert oracle.block_partial(a, b2) == exact / 2.0 ** 18


def test_single_block_gemm_equals_int64_matmul():
    # K = 128 and unit scales: the output before rounding is exactly the
    # integer dot product / 2^18.
    rng = np.random.default_rng(3)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a = rng.choice(finite, (5, 128))
    b = rng.choice(finite, (128, 128))
    ones_a = np.ones((5, 1), np.float32)
    ones_b = np.ones((1, 1), np.float32)
    d, acc = oracle.gemm_nt(a, ones_a, b, ones_b, want_acc=True)
    exact = int_codes(a) @ int_codes(b).T
    assert np.array_equal(acc, exact / 2.0 ** 18)


# ---------------------------------------------------------------- whole GEMM

def dequant_matmul(a, sa, b, sb):
    """Brute force: fp64 matmul of the dequantised operands, all K at once."""
    t = torch_decode_table()
    K = a.shape[1]
    at = t[a] * np.repeat(np.asarray(sa, np.float64), 128, axis=1)
    bt = t[b] * np.repeat(np.repeat(np.asarray(sb, np.float64), 128, axis=0), 128, axis=1)
    assert at.shape[1] == K and bt.shape[1] == K
    return at @ bt.T, np.abs(at) @ np.abs(bt).T


@pytest.mark.parametrize("M,N,K,seed", [(64, 256, 512, 1), (7, 384, 1024, 2), (33, 128, 128, 3)])
def test_gemm_matches_dequantised_matmul(M, N, K, seed):
    p = gen.make_dense(M, N, K, seed, seed + 100)
    sa = p.sa_t.T
    d, acc = oracle.gemm_nt(p.a, sa, p.b, p.sb, want_acc=True)
    ref, mag = dequant_matmul(p.a, sa, p.b, p.sb)
    assert np.all(np.abs(acc - ref) <= 1e-12 * mag + 1e-300)
    # bf16 bits agree except where ref sits within 1e-12 of a rounding boundary
    ref_bits = np.array([oracle.bf16_rne(float(x)) for x in ref.ravel()], np.uint16).reshape(ref.shape)
    mism = d != ref_bits
    if mism.any():
        lo = bf16_to_f64(d[mism])
        hi = bf16_to_f64(ref_bits[mism])
        mid = (lo + hi) / 2
        assert np.all(np.abs(ref[mism] - mid) <= 1e-12 * mag[mism])


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_per_tensor_special_case_exact():
    # Per-tensor scaling is the special case sA = alpha, sB = beta everywhere
    # (rkmt.cn walkthrough §2.2; lpnh.cn §2.2): the result is
    # alpha*beta*int64_matmul/2^18, exactly, when alpha and beta are powers of two.
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    M, N, K = 9, 256, 512
    a = rng.choice(finite, (M, K))
    b = rng.choice(finite, (N, K))
    alpha, beta = 2.0 ** -7, 2.0 ** 3
    sa = np.full((M, K // 128), alpha, np.float32)
    sb = np.full((N // 128, K // 128), beta, np.float32)
    d, acc = oracle.gemm_nt(a, sa, b, sb, want_acc=True)
    exact = (int_codes(a) @ int_codes(b).T).astype(np.float64) * (alpha * beta / 2.0 ** 18)
    assert np.array_equal(acc, exact)


def test_scale_stride_layouts_agree():
    p = gen.make_dense(16, 256, 384, 21, 22)
    sa_mmajor = p.sa_t.T                    # strides (1, M)
    sa_rowmajor = np.ascontiguousarray(sa_mmajor)  # strides (K/128, 1)
    d1 = oracle.gemm_nt(p.a, sa_mmajor, p.b, p.sb)
    d2 = oracle.gemm_nt(p.a, sa_rowmajor, p.b, p.sb)
    assert np.array_equal(d1, d2)


def test_points_match_full():
    p = gen.make_dense(40, 384, 512, 31, 32)
    d = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 40, 500)
    ns = rng.integers(0, 384, 500)
    dp, _ = oracle.gemm_nt_points(p.a, p.sa_t.T, p.b, p.sb, ms, ns)
    assert np.array_equal(dp, d[ms, ns])


@pytest.mark.parametrize("case", hand_cases.load(), ids=lambda c: c["name"])
def test_hand_cases(case):
    d = oracle.gemm_nt(case["a"], case["sa"], case["b"], case["sb"])
    assert np.array_equal(d, case["expect"])


def test_identity_rhs():
    # B = I (code 0x38 on the diagonal), sB = 1: D[m,n] = bf16(dec(A[m,n]) * sA[m, n/128]).
    p = gen.make_dense(8, 256, 256, 41, 42)
    b = np.zeros((256, 256), np.uint8)
    np.fill_diagonal(b, 0x38)
    sb = np.ones((2, 2), np.float32)
    d = oracle.gemm_nt(p.a, p.sa_t.T, b, sb)
    t = torch_decode_table()
    expect_f64 = t[p.a] * np.repeat(p.sa_t.T.astype(np.float64), 128, axis=1)
    # dec(A) * sA is exact in fp64; bf16_rne is pinned on its own above
    exp_bits = np.array([oracle.bf16_rne(float(x)) for x in expect_f64.ravel()],
                        np.uint16).reshape(expect_f64.shape)
    assert np.array_equal(d, exp_bits)


# ---------------------------------------------------------------- grouped routing

SENTINEL = 0x7FA5


def test_contiguous_routing_signature():
    # Expert e's B scale is e+1, A = B = 1.0, so D[r, n] = K*(e+1) names the expert.
    G, N, K = 5, 256, 256
    expert_of_token = np.array([3, 0, 3, 4, 0, 0, 3, 1] * 3)
    ids, tok, counts = gen.route_contiguous(expert_of_token, G)
    M_total = ids.shape[0]
    a = np.full((M_total, K), 0x38, np.uint8)
    sa = np.ones((M_total, K // 128), np.float32)
    b = np.full((G, N, K), 0x38, np.uint8)
    sb = np.stack([np.full((N // 128, K // 128), e + 1, np.float32) for e in range(G)])
    d0 = np.full((M_total, N), SENTINEL, np.uint16)
    d = oracle.grouped_contiguous(a, sa, b, sb, ids, d0)
    for r in range(M_total):
        if ids[r] < 0:
            assert np.all(d[r] == SENTINEL)
        else:
            assert np.all(d[r] == oracle.bf16_rne(K * (ids[r] + 1)))
    # expert 2 has no tokens: no rows at all
    assert counts[2] == 0 and not np.any(ids == 2)
    # out-of-range ids are not produced either
    ids_bad = ids.copy()
    ids_bad[0] = G
    ids_bad[1] = -7
    d = oracle.grouped_contiguous(a, sa, b, sb, ids_bad, d0)
    assert np.all(d[0] == SENTINEL) and np.all(d[1] == SENTINEL)


def test_contiguous_matches_dense_per_row():
    c = gen.make_contiguous(3, 200, 256, 384, 51, 52, 53)
    d0 = np.full((c.M_total, c.N), SENTINEL, np.uint16)
    d = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, d0)
    for e in range(c.G):
        rows = np.nonzero(c.ids == e)[0]
        de = oracle.gemm_nt(c.a[rows], c.sa_t.T[rows], c.b[e], c.sb[e])
        assert np.array_equal(d[rows], de)
    assert np.all(d[c.ids < 0] == SENTINEL)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, c.M_total, 300)
    ns = rng.integers(0, c.N, 300)
    dp, _, prod = oracle.grouped_contiguous_points(c.a, c.sa_t.T, c.b, c.sb, c.ids, rows, ns)
    assert np.array_equal(prod, c.ids[rows] >= 0)
    assert np.array_equal(dp[prod], d[rows, ns][prod])


def test_masked_routing_signature():
    G, M_max, N, K = 6, 40, 128, 256
    mm = np.array([0, 1, 39, 40, 17, 99], np.int32)   # 99 is clamped to M_max
    a = np.full((G, M_max, K), 0x38, np.uint8)
    sa_t = np.ones((G, K // 128, M_max), np.float32)
    b = np.full((G, N, K), 0x38, np.uint8)
    sb = np.stack([np.full((N // 128, K // 128), g + 1, np.float32) for g in range(G)])
    d0 = np.full((G, M_max, N), SENTINEL, np.uint16)
    d = oracle.grouped_masked(a, sa_t, b, sb, mm, d0)
    for g in range(G):
        c = min(max(int(mm[g]), 0), M_max)
        assert np.all(d[g, :c] == oracle.bf16_rne(K * (g + 1)))
        assert np.all(d[g, c:] == SENTINEL)
    mm_neg = mm.copy()
    mm_neg[2] = -5
    d = oracle.grouped_masked(a, sa_t, b, sb, mm_neg, d0)
    assert np.all(d[2] == SENTINEL)


def test_masked_matches_dense_per_group():
    m = gen.make_masked(4, 48, 256, 256, 61, 62, 63)
    d0 = np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16)
    d = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m, d0)
    for g in range(m.G):
        c = int(m.masked_m[g])
        if c:
            de = oracle.gemm_nt(m.a[g, :c], m.sa_t[g].T[:c], m.b[g], m.sb[g])
            assert np.array_equal(d[g, :c], de)
        assert np.all(d[g, c:] == SENTINEL)
    rng = np.random.default_rng(2)
    gs = rng.integers(0, m.G, 200)
    ms = rng.integers(0, m.M_max, 200)
    ns = rng.integers(0, m.N, 200)
    dp, _, prod = oracle.grouped_masked_points(m.a, m.sa_t, m.b, m.sb, m.masked_m, gs, ms, ns)
    assert np.array_equal(prod, ms < m.masked_m[gs])
    assert np.array_equal(dp[prod], d[gs, ms, ns][prod])


def test_two_experts_eight_tokens_fixed_grouping():
    # The minimal MoE bring-up case of the rkmt.cn walkthrough §5.3: two
    # experts, eight tokens each, a fixed grouping.
    c = gen.make_contiguous(2, 16, 128, 256, 71, 72, 73,
                            expert_of_token=np.array([0] * 8 + [1] * 8))
    assert c.M_total == 256
    assert np.array_equal(c.ids[:8], [0] * 8) and np.all(c.ids[8:128] == -1)
    assert np.array_equal(c.ids[128:136], [1] * 8) and np.all(c.ids[136:] == -1)
    d0 = np.full((c.M_total, c.N), SENTINEL, np.uint16)
    d = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, d0)
    t = torch_decode_table()
    for r in list(range(8)) + list(range(128, 136)):
        e = c.ids[r]
        ref, _ = dequant_matmul(c.a[r:r + 1], c.sa_t.T[r:r + 1], c.b[e], c.sb[e])
        got = np.array([oracle.bf16_rne(x) for x in ref[0]], np.uint16)
        # brute-force fp64 and the oracle agree to within 1e-12 relative,
        # which decides the bf16 bits except at a rounding boundary
        assert np.mean(got == d[r]) > 0.99
