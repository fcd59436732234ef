"""The allocation-free dense entry point (dg_fp8_gemm_nt_noalloc), called
through the C ABI: its split-K partial sums live in the library's static
scratch array. Each call must equal dg_fp8_gemm_nt_ws (caller workspace) bit
for bit, and the oracle within tolerance, on two calls in a row, the second
with a smaller problem (the array keeps the first call's partial sums, which
the second must not pick up)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import _lib, ops
from synth import gen
from tests.check import assert_close
from tests.gpu_util import bits, dev, sentinel_bf16

pytestmark = pytest.mark.gpu


def noalloc_abi(a, sa, b, sb, d):
    """dg_fp8_gemm_nt_noalloc through ctypes (the raw C ABI), on torch's current stream."""
    M, K = a.shape
    N = b.shape[0]
    lib = _lib.load()
    fn = lib.dg_fp8_gemm_nt_noalloc
    return fn(a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1),
              b.data_ptr(), b.stride(0), sb.data_ptr(), sb.stride(0), sb.stride(1),
              d.data_ptr(), d.stride(0), M, N, K, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("first,second", [
    ((200, 1024, 2048), (96, 512, 1024)),     # 256x128 tiles, 8 slices; then 128x128 tiles, 8 slices
    ((256, 4096, 7168), (40, 256, 8192)),     # 32 MiB of partial sums (the array's size); then split 24 < M <= 64
])
def test_noalloc_equals_workspace_call(gpu_device, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        need = ops.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
        assert 0 < need <= 32 << 20, (M, N, K, need)
        p = gen.make_dense(M, N, K, 9100 + M + i, 9200 + N + i)
        a, sa, b, sb = dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)
        d_ws = sentinel_bf16((M, N))
        ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, ops.workspace(need), d=d_ws)
        d_na = sentinel_bf16((M, N))
        st = noalloc_abi(a, sa, b, sb, d_na)
        assert st == 0, ops.DGError(st, "dg_fp8_gemm_nt_noalloc")
        torch.cuda.synchronize()
        got = bits(d_na)
        assert np.array_equal(got, bits(d_ws)), "call %d (%dx%dx%d): differs from the workspace call" % (i, M, N, K)
        ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
        assert_close(got, ref, "noalloc call %d" % i)


def test_noalloc_without_split_and_empty(gpu_device):
    # decode and 256x256 shapes take no scratch at all; M = 0 launches nothing
    for M, N, K in ((8, 4096, 7168), (4096, 4096, 256)):
        p = gen.make_dense(M, N, K, 9301, 9302)
        a, sa, b, sb = dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)
        d = sentinel_bf16((M, N))
        assert noalloc_abi(a, sa, b, sb, d) == 0
        torch.cuda.synchronize()
        assert_close(bits(d), oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb), "noalloc %dx%dx%d" % (M, N, K))
    e = torch.zeros((0, 256), dtype=torch.uint8, device="cuda")
    assert noalloc_abi(e, torch.zeros((0, 2), device="cuda"), torch.zeros((128, 256), dtype=torch.uint8,
                       device="cuda"), torch.zeros((1, 2), device="cuda"),
                       torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")) == 0
