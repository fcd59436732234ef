"""GPU dense GEMM with e5m2 operands (e4m3 x e5m2, e5m2 x e4m3, e5m2 x e5m2)
vs the oracle's format path, through the C ABI (dg_fp8_gemm_nt_fmt)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests.check import assert_close
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
