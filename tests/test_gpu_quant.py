"""GPU 1x128 activation quantiser vs the oracle, through the C ABI.

The codes and scales are integer/bit results of a fixed fp32 recipe, so the
bar is bit-exact agreement: codes byte for byte, scales bit for bit, and
every byte/slot outside the output left untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests.gpu_util import bits, dev, run_dense
from tests.test_oracle_quant import DIVISION_AMAX, division_cases, grid_cases, with_unit_scale

pytestmark = pytest.mark.gpu

Q_GUARD = 0xA5


def run_quant(x_np, bf16=False, ldx_pad=0, ldq_pad=0, m_major=True):
    """Quantise x [M, K] on the GPU with padded row strides; returns codes,
    scales (logical [M, K/128]) and the guard regions for inspection."""
    M, K = x_np.shape
    xt = torch.from_numpy(np.ascontiguousarray(x_np))
    if bf16:
        xt = xt.to(torch.bfloat16)
    xbuf = torch.zeros((M, K + ldx_pad), dtype=xt.dtype, device="cuda")
    xbuf[:, :K] = xt.cuda()
    x = xbuf[:, :K]
    qbuf = torch.full((M, K + ldq_pad), Q_GUARD, dtype=torch.uint8, device="cuda")
    q = qbuf[:, :K]
    nkb = K // 128
    if m_major:
        sbuf = torch.full((nkb, M + 3), float("nan"), dtype=torch.float32, device="cuda")
        s = sbuf[:, :M].t()
    else:
        sbuf = torch.full((M, nkb + 2), float("nan"), dtype=torch.float32, device="cuda")
        s = sbuf[:, :nkb]
    ops.dg_fp8_quantize_1x128(x, q=q, s=s)
    torch.cuda.synchronize()
    qb = qbuf.cpu().numpy()
    sb = sbuf.cpu().numpy()
    codes = qb[:, :K]
    scales = sb[:, :M].T if m_major else sb[:, :nkb]
    assert np.all(qb[:, K:] == Q_GUARD), "bytes past K in a code row were written"
    assert np.all(np.isnan(sb[:, M:] if m_major else sb[:, nkb:])), "scale padding was written"
    return codes, np.ascontiguousarray(scales), xt


def assert_same(x_np, bf16=False, **kw):
    codes, scales, xt = run_quant(x_np, bf16=bf16, **kw)
    ref_q, ref_s = oracle.quantize_1x128(xt)
    assert np.array_equal(scales.view(np.uint32), ref_s.view(np.uint32)), "scales differ"
    bad = np.argwhere(codes != ref_q)
    assert bad.size == 0, "codes differ at %s" % bad[:5].tolist()
    return codes, scales


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,K,ldx_pad,ldq_pad,m_major", [
    (1, 128, 0, 0, True),
    (3, 1152, 0, 16, True),      # 9 blocks: one full span and a one-block tail
    (64, 512, 8, 0, False),      # half a span, row-major scales
    (17, 2944, 16, 32, True),    # 23 blocks: ragged last span
    (200, 7168, 0, 0, True),     # the GEMM's K
    (130, 1024, 8, 16, False),   # exactly one span
])
def test_quant_parity(gpu_device, bf16, M, K, ldx_pad, ldq_pad, m_major):
    rng = np.random.Generator(np.random.PCG64(600 + M))
    x = gen.normal_with_outliers(rng, (M, K))
    assert_same(x, bf16=bf16, ldx_pad=ldx_pad, ldq_pad=ldq_pad, m_major=m_major)


def test_quant_e4m3_grid_midpoints(gpu_device):
    vals, want = grid_cases()
    codes, scales = assert_same(with_unit_scale(vals))
    assert np.all(scales == 1.0)
    assert np.array_equal(codes[:, 1:].reshape(-1)[:len(vals)], want)


def test_quant_divides_by_the_scale(gpu_device):
    vals, want = division_cases()
    codes, _ = assert_same(with_unit_scale(vals, DIVISION_AMAX))
    assert np.array_equal(codes[:, 1:].reshape(-1)[:len(vals)], want)


@pytest.mark.parametrize("bf16", [False, True])
def test_quant_special_blocks(gpu_device, bf16):
    rng = np.random.Generator(np.random.PCG64(611))
    x = gen.normal_with_outliers(rng, (10, 1280))
    x[0, 0:128] = 0.0                          # all zero: s = 1, codes 0
    x[1, 128:256] = -0.0                       # negative zeros: codes 0x80
    x[2, 256:384] *= np.float32(1e-30)         # tiny values, normal scale
    x[3, 384:512] *= np.float32(1e30)          # huge values
    x[4, 512:640] = np.float32(3e-39) * np.sign(x[4, 512:640])   # subnormal inputs: subnormal scale
    x[5, 640:768] = np.float32(-7.0)           # constant block: every code -448
    x[6, 768:896] = 0.0
    x[6, 800] = np.float32(-1e-20)             # a lone negative value sets amax
    x[7, 896:1024] *= np.float32(2e-17)        # scale just above 2^-64: the reciprocal path
    x[7, 0:128:3] = np.float32(1e-40)          # subnormal inputs in a normal block
    x[7, 1:128:3] = np.float32(-1e-40)
    x[8, 1024:1152] = np.float32(-1e-38)       # quotients that underflow: signed zero codes
    x[8, 1030] = np.float32(1e30)
    x[9, 128:256] = np.float32(-0.0)           # negative zeros beside a normal value
    x[9, 200] = np.float32(2.5)
    codes, scales = assert_same(x, bf16=bf16)
    assert scales[0, 0] == 1.0 and np.all(codes[0, :128] == 0)
    assert np.all(codes[5, 640:768] == 0xFE)
    assert np.all(codes[8, 1024:1152][np.arange(128) != 6] == 0x80)
    assert np.all(codes[9, 128:256][np.arange(128) != 72] == 0x80)


def test_quant_then_gemm_equals_gemm_on_generator_codes(gpu_device):
    """The quantiser's output fed to the dense GEMM gives the same bits as the
    GEMM on the generator's codes (which equal the oracle's quantisation)."""
    M, N, K = 96, 512, 2048
    xa = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(621)), (M, K))
    b, sb = gen.make_rhs(N, K, 622)
    q, s = ops.dg_fp8_quantize_1x128(dev(xa))
    d = ops.dg_fp8_gemm_nt(q, s, dev(b), dev(sb))
    torch.cuda.synchronize()
    ca, sa = gen.quantize_lhs(xa)
    ref = run_dense(ca, sa, b, sb)
    assert np.array_equal(bits(d), ref)


def test_quant_full_size_sampled_rows(gpu_device):
    """Token activations of the MoE workloads, 8192 x 7168 fp32: the whole
    output is checked for structure, and 48 rows against the oracle."""
    M, K = 8192, 7168
    x = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(631)), (M, K))
    xd = dev(x)
    q, s = ops.dg_fp8_quantize_1x128(xd)
    torch.cuda.synchronize()
    codes = q.cpu().numpy()
    scales = s.cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(0).choice(M, 45, replace=False)]))
    ref_q, ref_s = oracle.quantize_1x128(x[rows])
    assert np.array_equal(codes[rows], ref_q)
    assert np.array_equal(scales[rows].view(np.uint32), ref_s.view(np.uint32))
    # every block's largest element maps to 448 and every scale is amax / 448
    assert np.all((codes.reshape(M, K // 128, 128) & 0x7F).max(axis=2) == 0x7E)
    amax = torch.amax(xd.view(M, K // 128, 128).abs(), dim=2).cpu().numpy()
    assert np.array_equal(scales, amax / np.float32(448.0))


def test_quant_bf16_full_size_sampled_rows(gpu_device):
    M, K = 4096, 7168
    x = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(632)), (M, K))
    xb = torch.from_numpy(x).to(torch.bfloat16)
    q, s = ops.dg_fp8_quantize_1x128(xb.cuda())
    torch.cuda.synchronize()
    rows = np.random.default_rng(1).choice(M, 32, replace=False)
    ref_q, ref_s = oracle.quantize_1x128(xb[torch.from_numpy(rows)])
    assert np.array_equal(q.cpu().numpy()[rows], ref_q)
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), ref_s.view(np.uint32))


def test_quant_empty(gpu_device):
    x = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    q, s = ops.dg_fp8_quantize_1x128(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)
