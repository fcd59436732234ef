"""Bitwise determinism: 100 repeats of each dispatch path give the same bits.

The kernels add their fp32 partial sums in a fixed order (no atomics, split-K
slices reduced in slice order), so a repeat may differ from the first result
only through a race. Each path runs 100 times on the same inputs into the
same output buffer (cleared to the sentinel in between) and every repeat is
compared with the first on the device; the first is checked against the
oracle so that the repeats compare a correct result.
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

REPEATS = 100


def repeat_equal(fn, d):
    """Run fn() REPEATS times into d; every result equals the first bit for bit."""
    d.view(torch.int16).fill_(SENTINEL)
    fn()
    first = d.clone()
    for r in range(REPEATS - 1):
        d.view(torch.int16).fill_(SENTINEL)
        fn()
        assert torch.equal(d.view(torch.int16), first.view(torch.int16)), "repeat %d differs" % (r + 1)
    torch.cuda.synchronize()
    return bits(d)


def dense_args(p):
    return dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)


@pytest.mark.parametrize("path,M,N,K,ws", [
    ("decode", 8, 4096, 7168, False),            # small-M kernel, LHS staged per wave
    ("split_k", 96, 4096, 7168, True),           # 128x128 tiles split over K + ordered reduction
    ("split_k_256x128", 512, 4096, 2048, True),  # 256x128 tiles split over K
    ("tiles_256", 4096, 4096, 1024, False),      # 256x256 tiles, one round of 256
    ("round_cut", 4096, 4352, 512, True),        # 256x256 whole rounds + a strip split over K
])
def test_dense_paths_deterministic(gpu_device, path, M, N, K, ws):
    p = gen.make_dense(M, N, K, 7100 + M, 7200 + N)
    a, sa, b, sb = dense_args(p)
    d = sentinel_bf16((M, N))
    w = ops.workspace(ops.dg_fp8_gemm_nt_workspace_bytes(M, N, K)) if ws else None
    if ws:
        assert w.numel() > 0, "%s: this shape should take the split-K path" % path
    got = repeat_equal(lambda: ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, w, d=d), d)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    assert_close(got, ref, path)


@pytest.mark.parametrize("path", ["uniform_grid", "derived_segments_split_tails", "layout_split_tails",
                                  "to_tokens_split_tails"])
def test_contiguous_paths_deterministic(gpu_device, path):
    G, T, N, K = 8, 3000, 512, 2048
    e = np.random.Generator(np.random.PCG64(7301)).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 7302, 7303, 0, expert_of_token=e)
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, N, K, G))
    layout = dev(gen.segment_layout(c.counts).astype(np.int32))
    tok = dev(c.token_of_row.astype(np.int32))
    if path == "to_tokens_split_tails":
        d = sentinel_bf16((T, N))
        got = repeat_equal(lambda: ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, token_of_row=tok, T=T,
                                                                         layout=layout, d=d), d)
        valid = c.ids >= 0
        rows = np.full((c.M_total, N), SENTINEL, np.uint16)
        rows[valid] = got[c.token_of_row[valid]]
        got = rows
    else:
        d = sentinel_bf16((c.M_total, N))
        if path == "uniform_grid":
            fn = lambda: ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)  # noqa: E731
        elif path == "derived_segments_split_tails":
            fn = lambda: ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, d=d)  # noqa: E731
        else:
            fn = lambda: ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, layout=layout, d=d)  # noqa: E731
        got = repeat_equal(fn, d)
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    valid = c.ids >= 0
    assert np.all(got[~valid] == SENTINEL)
    assert_close(got[valid], ref[valid], path)


def test_masked_deterministic(gpu_device):
    m = gen.make_masked(8, 256, 1024, 2048, 7401, 7402, 7403)
    d = sentinel_bf16((m.G, m.M_max, m.N))
    args = (dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb), dev(m.masked_m.astype(np.int32)))
    got = repeat_equal(lambda: ops.dg_fp8_grouped_gemm_masked(*args, d=d), d)
    ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m, np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16))
    assert np.array_equal(got == SENTINEL, ref == SENTINEL)
    ok = ref != SENTINEL
    assert_close(got[ok], ref[ok], "masked")
