"""Seeded random shapes across the whole kernel-dispatch space vs the oracle.

Each case draws M, N, K (and strides, scale layout, operand formats, MoE
routing) from a fixed seed, so a failure names a reproducible case. Sizes are
capped so the oracle finishes each case in well under a second; together the
cases reach every dispatch branch: the small-M kernels (with and without the
LHS staging, K a multiple of 1024 or not), split-K, 128x128 / 256x128 /
256x256 tiles, ragged M, N an odd multiple of 128, padded row strides and both
scale layouts.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests.check import SENTINEL, assert_close
from tests.gpu_util import bits, dev, sentinel_bf16

pytestmark = pytest.mark.gpu

MAX_MACS = 60_000_000


def dense_case(seed):
    rng = np.random.default_rng(seed)
    while True:
        M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 400)]))
        N = 128 * int(rng.integers(1, 13))
        K = 128 * int(rng.choice([rng.integers(1, 9) * 8, rng.integers(1, 40)]))
        if M * N * K <= MAX_MACS:
            return rng, M, N, K


def padded(t, extra):
    """A view of t with `extra` unused elements after each row (row stride grows)."""
    rows, cols = t.shape
    buf = torch.zeros((rows, cols + extra), dtype=t.dtype, device=t.device)
    buf[:, :cols] = t
    return buf[:, :cols]


@pytest.mark.parametrize("seed", range(100))
def test_dense_fuzz(gpu_device, seed):
    rng, M, N, K = dense_case(1000 + seed)
    fa, fb = ("e4m3", "e4m3") if seed % 4 else [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")][seed // 4 % 3]
    p = gen.make_dense(M, N, K, 5000 + seed, 6000 + seed, fa, fb)
    a = padded(dev(p.a), 16 * int(rng.integers(0, 3)))
    b = padded(dev(p.b), 16 * int(rng.integers(0, 3)))
    m_major = bool(rng.integers(0, 2))
    sa = dev(p.sa_t).t() if m_major else dev(np.ascontiguousarray(p.sa_t.T))
    d = padded(sentinel_bf16((M, N)), 8 * int(rng.integers(0, 3)))
    if (fa, fb) == ("e4m3", "e4m3") and seed % 2:   # odd seeds: with a workspace (split-K)
        ops.dg_fp8_gemm_nt_ws(a, sa, b, dev(p.sb), ops.workspace(ops.dg_fp8_gemm_nt_workspace_bytes(M, N, K)), d=d)
    elif (fa, fb) == ("e4m3", "e4m3"):
        ops.dg_fp8_gemm_nt(a, sa, b, dev(p.sb), d=d)
    else:
        ops.dg_fp8_gemm_nt_fmt(a, sa, b, dev(p.sb), fa, fb, d=d)
    torch.cuda.synchronize()
    got = bits(d)
    ref = oracle.gemm_nt_fmt(p.a, fa, p.sa_t.T, p.b, fb, p.sb)
    assert_close(got, ref, "seed %d: %s x %s M=%d N=%d K=%d" % (seed, fa, fb, M, N, K))


@pytest.mark.parametrize("seed", range(30))
def test_contiguous_fuzz(gpu_device, seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.integers(1, 9))
    T = int(rng.integers(1, 700))
    N = 128 * int(rng.integers(1, 5))
    K = 128 * int(rng.integers(1, 9))
    probs = rng.dirichlet(np.ones(G) * 0.5)
    e = rng.choice(G, T, p=probs).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 2100 + seed, 2200 + seed, 0, expert_of_token=e)
    got = bits(_run_contiguous(c, ws=seed % 2 == 1))
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    valid = c.ids >= 0
    assert np.all(got[~valid] == SENTINEL), "seed %d: padding rows written" % seed
    if valid.any():
        assert_close(got[valid], ref[valid], "seed %d: G=%d T=%d N=%d K=%d" % (seed, G, T, N, K))


def _run_contiguous(c, ws=False):
    """The plain call, or (ws) the call with the workspace its query asks for."""
    d = sentinel_bf16((c.M_total, c.N))
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, c.N, c.K, c.G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, d=d)
    else:
        ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("seed", range(30))
def test_masked_fuzz(gpu_device, seed):
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.integers(1, 7))
    M_max = int(rng.choice([16, 64, 128, 200, 256]))
    N = 128 * int(rng.integers(1, 5))
    K = 128 * int(rng.integers(1, 9))
    mm = rng.integers(-2, M_max + 3, G).astype(np.int32)
    m = gen.make_masked(G, M_max, N, K, 3100 + seed, 3200 + seed, 0, masked_m=mm)
    d = sentinel_bf16((G, M_max, N))
    ops.dg_fp8_grouped_gemm_masked(dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb), dev(mm), d=d)
    torch.cuda.synchronize()
    got = bits(d)
    ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, mm, np.full((G, M_max, N), SENTINEL, np.uint16))
    for g in range(G):
        cnt = int(np.clip(mm[g], 0, M_max))
        assert np.all(got[g, cnt:] == SENTINEL), "seed %d group %d: rows past the count written" % (seed, g)
        if cnt:
            assert_close(got[g, :cnt], ref[g, :cnt], "seed %d group %d" % (seed, g))


MAX_LAYOUT_MACS = 1_500_000_000


@pytest.mark.parametrize("seed", range(30))
def test_contiguous_layout_fuzz(gpu_device, seed):
    """Segment-tiled contiguous GEMM (segment offsets given) on seeded shapes:
    skewed expert loads, K up to 4096 so the segments' last 128 rows are
    split over K with the slice count the device picks from the number of
    such segments; every fourth case writes to token order."""
    rng = np.random.default_rng(4000 + seed)
    while True:
        G = int(rng.integers(1, 17))
        T = int(rng.integers(1, 2500))
        N = 256 * int(rng.integers(1, 5))
        K = 128 * int(rng.choice([rng.integers(1, 9), rng.integers(8, 33)]))
        if T * N * K <= MAX_LAYOUT_MACS:
            break
    e = rng.choice(G, T, p=rng.dirichlet(np.ones(G) * 0.6)).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 4100 + seed, 4200 + seed, 0, expert_of_token=e)
    layout = gen.segment_layout(c.counts).astype(np.int32)
    assert layout[-1] == c.M_total
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    valid = c.ids >= 0
    what = "seed %d: G=%d T=%d N=%d K=%d" % (seed, G, T, N, K)
    # odd seeds give the call a workspace (tails split over K), even seeds none
    w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, N, K, G)) if seed % 2 else None
    if seed % 4 == 3:
        tok = c.token_of_row.astype(np.int32)
        out = sentinel_bf16((T, N))
        ops.dg_fp8_grouped_gemm_contiguous_ws(args[0], args[1], args[2], args[3], args[4], w,
                                              token_of_row=dev(tok), T=T, layout=dev(layout), d=out)
        torch.cuda.synchronize()
        got = bits(out)
        assert_close(got[tok[valid]], ref[valid], what)
        routed = np.zeros(T, bool)
        routed[tok[valid]] = True
        assert np.all(got[~routed] == SENTINEL), what
        return
    d = sentinel_bf16((c.M_total, N))
    if w is not None:
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, layout=dev(layout), d=d)
    else:
        ops.dg_fp8_grouped_gemm_contiguous_layout(*args, dev(layout), d=d)
    torch.cuda.synchronize()
    got = bits(d)
    assert np.all(got[~valid] == SENTINEL), "%s: padding rows written" % what
    assert_close(got[valid], ref[valid], what)
