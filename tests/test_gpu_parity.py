"""GPU vs oracle parity on seeded inputs, through the C ABI.

Every output element is compared with the oracle, at every size: the small
and ragged shapes, and the full-size workloads (4096^3, the 8192x7168x2048
prefill, the 8-expert contiguous MoE through each of its calls, the 32-expert
masked MoE). Every output buffer sits between 4 KB sentinel guard bands that
must stay untouched, rows the layouts leave out must keep the sentinel, and
each full-size test reports the share of elements within one bf16 ulp of the
oracle (the tolerance is the looser bound; the ulp share shows how close the
fp32 accumulation comes to the exact sum).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests.check import SENTINEL, assert_close
from tests.gpu_util import bits, dev, run_contiguous, run_dense, run_masked, sentinel_bf16

pytestmark = pytest.mark.gpu


def report(rep, what):
    share = rep["le1ulp"] / max(rep["n"], 1)
    print("%s: %d elements, %.5f within 1 ulp, %.5f exact, max err/tol %.3f"
          % (what, rep["n"], share, rep["exact"] / max(rep["n"], 1), rep["max_err_over_tol"]))
    assert share >= 0.99, "%s: only %.4f of the elements within one bf16 ulp" % (what, share)


@pytest.mark.parametrize("M,N,K", [
    (64, 256, 512),       # the small dense workload's shape
    (1, 128, 128), (8, 512, 1024), (17, 384, 896), (33, 256, 256), (63, 384, 640),
    (65, 256, 256), (129, 384, 1024), (200, 512, 384), (300, 128, 128), (1000, 256, 512),
    (777, 1152, 1280),
    (9, 256, 2048), (12, 384, 7168), (16, 512, 1024), (16, 128, 7168),   # 16-row LHS staging
    (17, 256, 1024), (24, 512, 1024), (32, 256, 7168), (48, 384, 2048), (64, 128, 4096),  # 2-4 passes
    (8, 256, 14336), (5, 128, 12288), (16, 256, 9216),   # long K: 12-14 blocks per wave; M=16 falls back
    (8, 512, 4096), (5, 384, 8192), (16, 256, 4096), (40, 256, 8192),  # 4 KB row strides: rotated block order
])
def test_dense_full_parity(gpu_device, M, N, K):
    p = gen.make_dense(M, N, K, 1000 + M, 2000 + N)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    assert_close(got, ref, "dense %dx%dx%d" % (M, N, K))


def test_small_dense_workload(gpu_device):
    """The small dense workload with its own seeds (101 / 102)."""
    p = gen.make_config("dense_64x256x512")
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    rep = assert_close(run_dense(p.a, p.sa_t.T, p.b, p.sb), ref, "dense_64x256x512")
    report(rep, "dense_64x256x512")


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("M", [40, 96, 256])   # with a workspace: split over K on 128x128 / 256x128 tiles
def test_medium_m_full_parity(gpu_device, M, ws):
    p = gen.make_dense(M, 4096, 7168, 3000 + M, 4000 + M)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb, ws=ws)
    assert_close(got, ref, "dense %dx4096x7168 ws=%s" % (M, ws))


def test_decode_full_parity(gpu_device):
    p = gen.make_config("decode_8x4096x7168")
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    report(assert_close(got, ref, "decode 8x4096x7168"), "decode_8x4096x7168")


@pytest.mark.parametrize("name", ["square_4096", "prefill_8192x7168x2048", "square_4096_e4m3xe5m2"])
def test_large_dense_full_parity(gpu_device, name):
    """The 256x256-tile path on the full-size dense workloads, every element."""
    p = gen.make_config(name)
    fa, fb = gen.CONFIGS[name].get("fmt", ("e4m3", "e4m3"))
    d = sentinel_bf16((p.M, p.N))
    if (fa, fb) == ("e4m3", "e4m3"):
        ops.dg_fp8_gemm_nt(dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb), d=d)
        ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    else:
        ops.dg_fp8_gemm_nt_fmt(dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb), fa, fb, d=d)
        ref = oracle.gemm_nt_fmt(p.a, fa, p.sa_t.T, p.b, fb, p.sb)
    torch.cuda.synchronize()
    got = bits(d)
    report(assert_close(got, ref, name), name)


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("M,N", [(4096, 4352), (4352, 4096)])
def test_round_cut_full_parity(gpu_device, M, N, ws):
    """272 tiles of 256x256 leave a last round of 16 on 256 CUs: the first
    4096 columns (rows) run as whole rounds on 256x256 tiles and the
    remaining strip as a second launch on smaller tiles (split over K with a
    workspace). Every element of both parts against the oracle."""
    p = gen.make_dense(M, N, 512, 5000 + M, 6000 + N)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb, ws=ws)
    report(assert_close(got, ref, "round cut %dx%d" % (M, N)), "round cut %dx%dx512 ws=%s" % (M, N, ws))


@pytest.mark.parametrize("N", [384, 512])   # 256x128 and 256x256 tiles
@pytest.mark.parametrize("ws", [False, True])
def test_small_contiguous_full_parity(gpu_device, N, ws):
    # Segments of 1, 3, 1, 2 and 1 128-row blocks: without a workspace three
    # of the four 256-row tiles hold two experts (a pass per expert); with one
    # (N 512) the tiles follow the derived segments.
    counts = [100, 300, 50, 129, 121]
    tokens = np.repeat(np.arange(5), counts)
    np.random.default_rng(14).shuffle(tokens)
    c = gen.make_contiguous(5, len(tokens), N, 640, 11, 12, 13, expert_of_token=tokens)
    assert c.M_total == 8 * 128
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids,
                                    np.full((c.M_total, c.N), SENTINEL, np.uint16))
    got = run_contiguous(c, ws=ws)
    pad = c.ids < 0
    assert np.all(got[pad] == SENTINEL)
    assert_close(got[~pad], ref[~pad], "contiguous small")


@pytest.fixture(scope="module")
def moe_contiguous():
    c = gen.make_config("moe_contiguous_g8_t8192")
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids,
                                    np.full((c.M_total, c.N), SENTINEL, np.uint16))
    return c, ref


@pytest.mark.parametrize("call", ["plain", "ws", "layout", "layout_ws", "to_tokens_ws"])
def test_moe_contiguous_full_size(gpu_device, moe_contiguous, call):
    """The 8-expert, 8192-token contiguous workload, every element, through
    each call: the uniform grid (no workspace), offsets derived on the device
    with split tails (workspace), segment tiles from the given offsets with
    and without a workspace, and the same written straight to token order."""
    c, ref = moe_contiguous
    pad = c.ids < 0
    layout = gen.segment_layout(c.counts).astype(np.int32)
    if call == "to_tokens_ws":
        T = len(c.token_of_row[c.token_of_row >= 0])
        tok = c.token_of_row.astype(np.int32)
        out = sentinel_bf16((T, c.N))
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, c.N, c.K, c.G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids), w,
                                              token_of_row=dev(tok), T=T, layout=dev(layout), d=out)
        torch.cuda.synchronize()
        got_tok = bits(out)
        assert not np.any(got_tok == SENTINEL), "every token's row written"
        got = np.full_like(ref, SENTINEL)
        got[~pad] = got_tok[tok[~pad]]
    else:
        got = run_contiguous(c, ws=call in ("ws", "layout_ws"),
                             layout=layout if call in ("layout", "layout_ws") else None)
    assert np.all(got[pad] == SENTINEL), "padding rows untouched"
    report(assert_close(got[~pad], ref[~pad], "moe contiguous (%s)" % call), "moe_contiguous_g8_t8192 %s" % call)


def test_small_masked_full_parity(gpu_device):
    for N in (256, 384):   # 256x256 and 256x128 tiles
        m = gen.make_masked(6, 200, N, 512, 21, 22, 23, masked_m=np.array([0, 1, 200, 77, 128, 129]))
        ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m,
                                    np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16))
        got = run_masked(m)
        assert np.array_equal(got == SENTINEL, ref == SENTINEL), "rows written = rows the oracle produces"
        for g in range(m.G):
            c = int(m.masked_m[g])
            assert np.all(got[g, c:] == SENTINEL)
            if c:
                assert_close(got[g, :c], ref[g, :c], "masked small g%d" % g)


def test_moe_masked_full_size(gpu_device):
    """The 32-expert masked workload: every valid element against the oracle,
    every row past a group's count untouched."""
    m = gen.make_config("moe_masked_g32_m256")
    ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m,
                                np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16))
    got = run_masked(m)
    valid = np.zeros((m.G, m.M_max), bool)
    for g in range(m.G):
        valid[g, :int(m.masked_m[g])] = True
    assert np.all(got[~valid] == SENTINEL), "rows past the count untouched"
    report(assert_close(got[valid], ref[valid], "moe masked"), "moe_masked_g32_m256")
