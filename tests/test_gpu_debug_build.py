"""The release library against its -O1 -g build (libdg_fp8_O1.so), bit for
bit, on every dispatch path: a different instruction schedule, register
allocation and scratch spills between the LDS copies must not change a
single output bit (a race on the LDS stages, or a wait that only holds for
one schedule, would). The release result is also held to the oracle."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import _lib, build, ops
from synth import gen
from tests.check import SENTINEL, assert_close
from tests.gpu_util import bits, dev, sentinel_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def debug_lib():
    if not os.path.exists(build.DEBUG_LIBRARY):
        raise ImportError("libdg_fp8_O1.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(build.DEBUG_LIBRARY)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def both(debug_lib, fn):
    """fn() through the release library, then through the -O1 build."""
    _lib.load()
    rel = fn()
    saved = _lib._lib
    _lib._lib = debug_lib
    try:
        dbg = fn()
    finally:
        _lib._lib = saved
    return rel, dbg


@pytest.mark.parametrize("M,N,K,ws", [
    (8, 4096, 7168, False),       # decode kernel
    (40, 512, 2048, False),       # decode kernel, 3 passes of 16 rows
    (96, 4096, 7168, True),       # 128x128 tiles split over K + reduction
    (512, 4096, 2048, True),      # 256x128 tiles split over K
    (4096, 4096, 512, False),     # 256x256 tiles, one round
    (4096, 4352, 512, True),      # 256x256 whole rounds + a strip split over K
])
def test_dense_release_equals_O1(gpu_device, debug_lib, M, N, K, ws):
    p = gen.make_dense(M, N, K, 8100 + M, 8200 + N)
    a, sa, b, sb = dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)

    def run():
        w = ops.workspace(ops.dg_fp8_gemm_nt_workspace_bytes(M, N, K)) if ws else None
        d = sentinel_bf16((M, N))
        ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, w, d=d)
        torch.cuda.synchronize()
        return bits(d)
    rel, dbg = both(debug_lib, run)
    assert np.array_equal(rel, dbg), "-O1 build differs from the release build"
    assert_close(rel, oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb), "dense %dx%dx%d" % (M, N, K))


def test_fmt_release_equals_O1(gpu_device, debug_lib):
    p = gen.make_dense(300, 512, 1024, 8301, 8302, "e4m3", "e5m2")
    args = (dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb))

    def run():
        d = sentinel_bf16((300, 512))
        ops.dg_fp8_gemm_nt_fmt(*args, "e4m3", "e5m2", d=d)
        torch.cuda.synchronize()
        return bits(d)
    rel, dbg = both(debug_lib, run)
    assert np.array_equal(rel, dbg)


@pytest.mark.parametrize("call", ["plain", "derived_ws", "layout_ws", "to_tokens_ws"])
def test_contiguous_release_equals_O1(gpu_device, debug_lib, call):
    G, T, N, K = 8, 3000, 512, 2048
    e = np.random.Generator(np.random.PCG64(8401)).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 8402, 8403, 0, expert_of_token=e)
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    layout = dev(gen.segment_layout(c.counts).astype(np.int32))
    tok = dev(c.token_of_row.astype(np.int32))

    def run():
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, N, K, G))
        if call == "to_tokens_ws":
            d = sentinel_bf16((T, N))
            ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, token_of_row=tok, T=T, layout=layout, d=d)
        else:
            d = sentinel_bf16((c.M_total, N))
            if call == "plain":
                ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
            else:
                ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, layout=layout if call == "layout_ws" else None, d=d)
        torch.cuda.synchronize()
        return bits(d)
    rel, dbg = both(debug_lib, run)
    assert np.array_equal(rel, dbg), "-O1 build differs from the release build (%s)" % call
    if call != "to_tokens_ws":
        ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
        valid = c.ids >= 0
        assert np.all(rel[~valid] == SENTINEL)
        assert_close(rel[valid], ref[valid], call)


def test_masked_release_equals_O1(gpu_device, debug_lib):
    m = gen.make_masked(8, 256, 1024, 2048, 8501, 8502, 8503)
    args = (dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb), dev(m.masked_m.astype(np.int32)))

    def run():
        d = sentinel_bf16((m.G, m.M_max, m.N))
        ops.dg_fp8_grouped_gemm_masked(*args, d=d)
        torch.cuda.synchronize()
        return bits(d)
    rel, dbg = both(debug_lib, run)
    assert np.array_equal(rel, dbg)
    ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m, np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16))
    ok = ref != SENTINEL
    assert np.array_equal(rel == SENTINEL, ~ok)
    assert_close(rel[ok], ref[ok], "masked")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantizer_and_routing_release_equals_O1(gpu_device, debug_lib, dtype):
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(8601)), (700, 2048)))
    x = x.to(dtype).cuda()
    e = torch.from_numpy(np.random.Generator(np.random.PCG64(8602)).choice(6, 700).astype(np.int32)).cuda()

    def run():
        q, s = ops.dg_fp8_quantize_1x128(x)
        row, ids, tok, layout = ops.dg_moe_route_contiguous(e, 6)
        torch.cuda.synchronize()
        return [np.ascontiguousarray(t.cpu().numpy()) for t in (q, s, row, ids, tok, layout)]
    rel, dbg = both(debug_lib, run)
    for r, d in zip(rel, dbg):
        assert np.array_equal(r.view(np.uint8), d.view(np.uint8))
