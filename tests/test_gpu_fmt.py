"""GPU dense GEMM with e5m2 operands (e4m3 x e5m2, e5m2 x e4m3, e5m2 x e5m2)
vs the oracle's format path, through the C ABI (dg_fp8_gemm_nt_fmt)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests.check import SENTINEL, assert_close
from tests.gpu_util import bits, dev, run_dense, sentinel_bf16

pytestmark = pytest.mark.gpu

FMT_CASES = [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


def run_fmt(p, fa, fb):
    d = sentinel_bf16((p.M, p.N))
    ops.dg_fp8_gemm_nt_fmt(dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb), fa, fb, d=d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("fa,fb", FMT_CASES)
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (8, 256, 512), (64, 256, 1024), (200, 384, 1024),
                                   (777, 1152, 1280), (300, 512, 7168)])
def test_fmt_full_parity(gpu_device, fa, fb, M, N, K):
    p = gen.make_dense(M, N, K, 1100 + M, 1200 + N, fa, fb)
    ref = oracle.gemm_nt_fmt(p.a, fa, p.sa_t.T, p.b, fb, p.sb)
    assert_close(run_fmt(p, fa, fb), ref, "%s x %s %dx%dx%d" % (fa, fb, M, N, K))


def test_fmt_hand_case_exact(gpu_device):
    """57344^2 * 2^-30 * 2^-2 = 0.765625 (bf16 0x3F44): exact in fp32 and bf16."""
    a = np.zeros((1, 128), np.uint8)
    b = np.zeros((128, 128), np.uint8)
    a[0, 0] = b[0, 0] = 0x7B
    d = sentinel_bf16((1, 128))
    ops.dg_fp8_gemm_nt_fmt(dev(a), dev(np.full((1, 1), 2.0 ** -30, np.float32)), dev(b),
                           dev(np.full((1, 1), 2.0 ** -2, np.float32)), "e5m2", "e5m2", d=d)
    torch.cuda.synchronize()
    got = bits(d)
    assert got[0, 0] == 0x3F44 and np.all(got[0, 1:] == 0)


def test_e4m3_pair_through_the_format_entry_is_the_dense_call(gpu_device):
    p = gen.make_dense(96, 512, 2048, 1301, 1302)
    assert np.array_equal(run_fmt(p, "e4m3", "e4m3"), run_dense(p.a, p.sa_t.T, p.b, p.sb))


def test_fmt_square_4096_sampled(gpu_device):
    p = gen.make_config("square_4096_e4m3xe5m2")
    got = run_fmt(p, "e4m3", "e5m2")
    rng = np.random.default_rng(11)
    ms = np.concatenate([rng.integers(0, 4096, 512), np.full(64, 4095)])
    ns = np.concatenate([rng.integers(0, 4096, 512), np.arange(64) * 64])
    ref, _ = oracle.gemm_nt_fmt_points(p.a, "e4m3", p.sa_t.T, p.b, "e5m2", p.sb, ms, ns)
    assert_close(got[ms, ns], ref, "4096^3 e4m3 x e5m2")
    assert not np.any(got == 0x7FA5)      # every output written


@pytest.mark.parametrize("side", ["A", "B"])
def test_mfma_decodes_every_e5m2_code(gpu_device, side):
    """Every finite e5m2 code through the MFMA, in either operand position:
    the code row times an identity (1.0 on the diagonal, the other format) with
    unit scales gives the decoded value, exact in bf16 (3 significant bits,
    exponents 2^-16 .. 2^15)."""
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)    # 248 finite codes
    K = 256
    vals = np.zeros((2, K), np.uint8)
    vals.ravel()[:len(codes)] = codes                    # two rows of up to 256 codes (K positions)
    ident_e4m3 = np.zeros((K, K), np.uint8)
    np.fill_diagonal(ident_e4m3, 0x38)
    ones = lambda r, c: np.ones((r, c), np.float32)      # noqa: E731
    d = sentinel_bf16((2, K))
    if side == "A":    # A holds e5m2 codes, B = I in e4m3: D = dec_e5m2(A)
        ops.dg_fp8_gemm_nt_fmt(dev(vals), dev(ones(2, 2)), dev(ident_e4m3), dev(ones(2, 2)), "e5m2", "e4m3", d=d)
    else:              # B holds e5m2 codes, A = I in e4m3: D[m, n] = dec_e5m2(B[n, m]) -> the codes come out on a row
        b = np.zeros((K, K), np.uint8)
        b[:, :2] = vals.T                                # B[n, m] = vals[m, n]
        ident_rows = np.zeros((2, K), np.uint8)
        ident_rows[0, 0] = ident_rows[1, 1] = 0x38
        ops.dg_fp8_gemm_nt_fmt(dev(ident_rows), dev(ones(2, 2)), dev(b), dev(ones(2, 2)), "e4m3", "e5m2", d=d)
    torch.cuda.synchronize()
    got = bits(d).ravel()[:len(codes)]
    want = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float32).to(torch.bfloat16)
    want = want.view(torch.int16).numpy().view(np.uint16)
    nz = (codes & 0x7F) != 0          # -0 sums with +0 products to +0: zeros compare by value
    assert np.array_equal(got[nz], want[nz])
    assert np.all((got[~nz] & 0x7FFF) == 0)


@pytest.mark.parametrize("fa,fb", FMT_CASES)
def test_contiguous_fmt_matches_per_expert_dense_oracle(gpu_device, fa, fb):
    """Contiguous layout with e5m2 operands: every routed row equals the
    format oracle's dense GEMM of that row against its expert's B; padding rows
    stay untouched."""
    G, T, N, K = 5, 600, 384, 768
    rng = np.random.default_rng(41)
    e = rng.choice(G, T, p=rng.dirichlet(np.ones(G))).astype(np.int32)
    ids, tok, _ = gen.route_contiguous(e, G)
    xa, sa_tok = gen.make_lhs(T, K, 42, fa)
    a = np.zeros((len(ids), K), np.uint8)
    sa = np.ones((len(ids), K // 128), np.float32)
    real = tok >= 0
    a[real], sa[real] = xa[tok[real]], sa_tok.T[tok[real]]
    b = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        b[g], sb[g] = gen.make_rhs(N, K, 43 + g, fb)
    d = sentinel_bf16((len(ids), N))
    ops.dg_fp8_grouped_gemm_contiguous_fmt(dev(a), dev(sa), dev(b), dev(sb), dev(ids), fa, fb, d=d)
    torch.cuda.synchronize()
    got = bits(d)
    assert np.all(got[~real] == SENTINEL)
    for g in range(G):
        rows = np.nonzero(ids == g)[0]
        if len(rows):
            ref = oracle.gemm_nt_fmt(a[rows], fa, sa[rows], b[g], fb, sb[g])
            assert_close(got[rows], ref, "%s x %s expert %d" % (fa, fb, g))


@pytest.mark.parametrize("fa,fb", FMT_CASES)
def test_masked_fmt_matches_per_group_dense_oracle(gpu_device, fa, fb):
    G, M_max, N, K = 4, 200, 512, 640
    mm = np.array([0, 200, 73, 129], np.int32)
    a = np.empty((G, M_max, K), np.uint8)
    sa = np.empty((G, M_max, K // 128), np.float32)
    b = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        a[g], sat = gen.make_lhs(M_max, K, 52 + g, fa)
        sa[g] = sat.T
        b[g], sb[g] = gen.make_rhs(N, K, 62 + g, fb)
    d = sentinel_bf16((G, M_max, N))
    ops.dg_fp8_grouped_gemm_masked_fmt(dev(a), dev(sa), dev(b), dev(sb), dev(mm), fa, fb, d=d)
    torch.cuda.synchronize()
    got = bits(d)
    for g in range(G):
        c = int(mm[g])
        assert np.all(got[g, c:] == SENTINEL)
        if c:
            ref = oracle.gemm_nt_fmt(a[g, :c], fa, sa[g, :c], b[g], fb, sb[g])
            assert_close(got[g, :c], ref, "%s x %s group %d" % (fa, fb, g))
