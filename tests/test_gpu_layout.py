"""Contiguous grouped GEMM tiled along the experts' segments (layout given,
or derived on the device into the caller's workspace).

Rows in a segment's whole 256-row tiles go through the same per-element
arithmetic as on the uniform grid, so they must equal the uniform-grid result
bit for bit. With a workspace, a segment's last 128 rows (where its size is
an odd multiple of 128) may be split over K and summed slice by slice, which
only regroups the fp32 additions: those rows are held to the oracle's
tolerance; without one they run unsplit and equal the grid too. Every valid row
is held against the oracle, padding rows must stay untouched, and a layout
that does not fit the rows must write nothing (and not fault).
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


def layout_of(counts):
    padded = (np.asarray(counts) + 127) // 128 * 128
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)


def tail_rows(layout, M):
    """Rows in a segment's last 128 rows when its size is an odd multiple of 128."""
    mask = np.zeros(M, bool)
    for lo, hi in zip(layout[:-1], layout[1:]):
        if hi - lo > 0 and ((hi - lo) >> 7) & 1:
            mask[lo + ((hi - lo) & ~255):hi] = True
    return mask


def run_both(c, layout, ws=True):
    """(uniform grid, segment tiles): the plain call, and the call given the
    layout, with the workspace its query asks for (ws) or none."""
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    d_grid = sentinel_bf16((c.M_total, c.N))
    ops.dg_fp8_grouped_gemm_contiguous(*args, d=d_grid)
    d_seg = sentinel_bf16((c.M_total, c.N))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, c.N, c.K, c.G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, layout=dev(layout), d=d_seg)
    else:
        ops.dg_fp8_grouped_gemm_contiguous_layout(*args, dev(layout), d=d_seg)
    torch.cuda.synchronize()
    return bits(d_grid), bits(d_seg)


@pytest.mark.parametrize("G,T,N,K,seed", [
    (4, 700, 256, 512, 1),      # 256x256 tiles
    (5, 900, 384, 640, 2),      # 256x128 tiles
    (8, 1500, 512, 256, 3),
    (3, 130, 256, 128, 4),      # one 256-row tile and a 128-row tail
    (6, 400, 256, 384, 5),      # empty experts
    (4, 700, 256, 1152, 6),     # tails split over K: 2 slices of 4 and 5 blocks
    (7, 1300, 384, 2048, 7),    # 4 slices
    (3, 900, 512, 4096, 8),     # 8 slices
])
@pytest.mark.parametrize("ws", [True, False])
def test_segment_tiles_equal_grid_tiles_and_oracle(gpu_device, G, T, N, K, seed, ws):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(G) * 0.7)
    if seed == 5:
        p[1] = p[4] = 0
        p /= p.sum()
    e = rng.choice(G, T, p=p).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 700 + seed, 800 + seed, 0, expert_of_token=e)
    layout = layout_of(c.counts)
    assert layout[-1] == c.M_total
    grid, seg = run_both(c, layout, ws)
    whole = ~tail_rows(layout, c.M_total) if ws else np.ones(c.M_total, bool)
    assert np.array_equal(seg[whole], grid[whole])
    valid = c.ids >= 0
    assert np.all(seg[~valid] == SENTINEL)
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    assert_close(seg[valid], ref[valid], "segment tiles G=%d T=%d" % (G, T))


def test_segment_tiles_full_size(gpu_device):
    """The contiguous MoE workload (8 experts, 8192 tokens, N 4096, K 7168):
    whole-tile rows equal the uniform grid bit for bit; sampled outputs of the
    tails (split over K) match the oracle; padding rows stay untouched."""
    c = gen.make_config("moe_contiguous_g8_t8192")
    layout = layout_of(c.counts)
    grid, seg = run_both(c, layout)
    tails = tail_rows(layout, c.M_total)
    assert tails.any()
    valid = c.ids >= 0
    assert np.array_equal(seg[~tails], grid[~tails])
    assert not np.any(seg[valid] == SENTINEL)
    assert np.all(seg[~valid] == SENTINEL)
    rng = np.random.default_rng(9)
    cand = np.nonzero(tails & valid)[0]
    rows = rng.choice(cand, 512)
    ns = rng.integers(0, c.N, 512)
    ref, _, produced = oracle.grouped_contiguous_points(c.a, c.sa_t.T, c.b, c.sb, c.ids, rows, ns)
    assert produced.all()
    assert_close(seg[rows, ns], ref, "full-size segment tails")


def test_to_tokens_with_layout(gpu_device):
    """Route, quantise into the layout, then the GEMM to token order with and
    without the layout: rows of whole tiles agree bit for bit, and every kept
    token matches the oracle (K 1024: the tails are split over K)."""
    T, G, N, K = 700, 5, 384, 1024
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(941)), (T, K)))
    e = np.random.Generator(np.random.PCG64(942)).choice(G, T).astype(np.int32)
    e[::13] = -1
    b, sb = gen.make_grouped_rhs(G, N, K, 943)
    bd, sbd = dev(b), dev(sb)
    row, ids, tok, layout = ops.dg_moe_route_contiguous(dev(e), G)
    q, s = ops.dg_fp8_quantize_1x128_gather(x.cuda(), tok)
    out0 = sentinel_bf16((T, N))
    ops.dg_fp8_grouped_gemm_contiguous_to_tokens(q, s, bd, sbd, ids, tok, T, out=out0)
    out1 = sentinel_bf16((T, N))
    w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(ids.shape[0], N, K, G))
    ops.dg_fp8_grouped_gemm_contiguous_ws(q, s, bd, sbd, ids, w, token_of_row=tok, T=T, layout=layout, d=out1)
    torch.cuda.synchronize()
    lay, tk = layout.cpu().numpy(), tok.cpu().numpy()
    tails = tail_rows(lay, len(tk))
    whole_tokens = tk[(~tails) & (tk >= 0)]
    assert np.array_equal(bits(out0)[whole_tokens], bits(out1)[whole_tokens])
    kept = e >= 0
    assert np.all(bits(out1)[~kept] == SENTINEL)
    rq, rs = oracle.quantize_1x128(x.numpy()[kept])
    ref = oracle.grouped_contiguous(rq, rs, b, sb, e[kept], np.zeros((int(kept.sum()), N), np.uint16))
    assert_close(bits(out1)[kept], ref, "to tokens with layout")


@pytest.mark.parametrize("G,T", [(200, 12000), (1024, 12000)])
@pytest.mark.parametrize("ws", [True, False])
def test_layout_many_experts(gpu_device, G, T, ws):
    """The layout given for hundreds of experts (several rounds of 64 experts
    in the tiles' segment search, many empty and one-block segments, tails
    split over K with a workspace): rows of whole tiles equal the uniform grid
    bit for bit, every valid row matches the oracle, padding stays untouched."""
    N, K = 256, 640
    rng = np.random.default_rng(G)
    # skewed routing: a few large experts among many small or empty ones
    w = rng.pareto(1.2, G) + 0.05
    e = rng.choice(G, T, p=w / w.sum()).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 961, 962, 0, expert_of_token=e)
    layout = layout_of(c.counts)
    assert layout[-1] == c.M_total
    grid, seg = run_both(c, layout, ws)
    valid = c.ids >= 0
    assert np.all(seg[~valid] == SENTINEL), "padding rows untouched"
    whole = valid & ~tail_rows(layout, c.M_total)
    assert np.array_equal(seg[whole], grid[whole]), "whole-tile rows equal the uniform grid"
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    assert_close(seg[valid], ref[valid], "layout with G=%d" % G)


@pytest.mark.parametrize("kind", ["zeros", "past_the_rows", "negative"])
@pytest.mark.parametrize("ws", [True, False])
def test_layout_that_does_not_fit_writes_nothing(gpu_device, kind, ws):
    G, T, N, K = 4, 300, 256, 256
    e = np.random.default_rng(6).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 951, 952, 0, expert_of_token=e)
    if kind == "zeros":
        layout = np.zeros(G + 1, np.int32)
    elif kind == "past_the_rows":
        layout = (c.M_total + 128 * np.arange(G + 1)).astype(np.int32)
    else:
        layout = (-4096 + 256 * np.arange(G + 1)).astype(np.int32)
    _, seg = run_both(c, layout, ws)
    assert np.all(seg == SENTINEL)


def blocks_reordered(c, order_blocks):
    """The contiguous problem c with its 128-row blocks taken in the order given
    (a list of block indexes, -1 for an extra block of padding)."""
    a = np.zeros((128 * len(order_blocks), c.K), np.uint8)
    sa_t = np.zeros((c.K // 128, 128 * len(order_blocks)), np.float32)
    ids = np.full(128 * len(order_blocks), -1, np.int32)
    tok = np.full(128 * len(order_blocks), -1, np.int32)
    for i, b in enumerate(order_blocks):
        if b >= 0:
            a[128 * i:128 * i + 128] = c.a[128 * b:128 * b + 128]
            sa_t[:, 128 * i:128 * i + 128] = c.sa_t[:, 128 * b:128 * b + 128]
            ids[128 * i:128 * i + 128] = c.ids[128 * b:128 * b + 128]
            tok[128 * i:128 * i + 128] = c.token_of_row[128 * b:128 * b + 128]
        else:
            sa_t[:, 128 * i:128 * i + 128] = 1.0
    return a, sa_t, ids, tok


@pytest.mark.parametrize("case", ["descending", "interleaved", "padding_blocks"])
@pytest.mark.parametrize("ws", [True, False])
def test_plain_call_any_block_order(gpu_device, case, ws):
    """The call given only the ids (and a workspace) derives the segment
    offsets on the device when the experts ascend (padding blocks anywhere
    allowed) and falls back to the uniform grid otherwise; without a
    workspace it tiles the rows uniformly. Either way every valid row matches
    the oracle and padding rows stay untouched."""
    G, T, N, K = 5, 900, 256, 1024
    e = np.random.default_rng(21).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 961, 962, 0, expert_of_token=e)
    layout = layout_of(c.counts)
    seg_blocks = [list(range(layout[g] // 128, layout[g + 1] // 128)) for g in range(G)]
    if case == "descending":
        order = [b for g in reversed(range(G)) for b in seg_blocks[g]]
    elif case == "interleaved":
        order = [b for g in (1, 0, 2, 4, 3) for b in seg_blocks[g]]
    else:
        order = [-1, -1] + [b for g in range(G) for b in seg_blocks[g] + ([-1] if g % 2 else [])] + [-1, -1, -1]
    a, sa_t, ids, tok = blocks_reordered(c, order)
    M = len(ids)
    args = (dev(a), dev(sa_t).t(), dev(c.b), dev(c.sb), dev(ids))
    d = sentinel_bf16((M, N))
    out = sentinel_bf16((T, N))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(M, N, K, G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, d=d)
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, token_of_row=dev(tok), T=T, d=out)
    else:
        ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
        ops.dg_fp8_grouped_gemm_contiguous_to_tokens(*args, dev(tok), T, out=out)
    torch.cuda.synchronize()
    got = bits(d)
    ref = oracle.grouped_contiguous(a, sa_t.T, c.b, c.sb, ids, np.full((M, N), SENTINEL, np.uint16))
    valid = ids >= 0
    assert np.all(got[~valid] == SENTINEL), case
    assert_close(got[valid], ref[valid], "plain call, blocks %s" % case)
    # the token-order call takes the same path: its rows equal the plain call's
    assert np.array_equal(bits(out)[tok[valid]], got[valid]), case


def plain_ids_case(kind):
    """(ids, G, K) for the plain-call edge cases."""
    rng = np.random.default_rng(31)
    if kind == "all_padding":
        return np.full(512, -1, np.int32), 4, 256
    if kind == "one_expert":
        ids = np.full(640, 0, np.int32)
        ids[600:] = -1
        return ids, 1, 1024
    if kind == "last_expert_only":
        ids = np.full(768, -1, np.int32)
        ids[256:700] = 5
        return ids, 6, 1024
    if kind == "ids_out_of_range":
        ids = np.repeat(np.arange(4, dtype=np.int32), 256)
        ids[rng.choice(len(ids), 40, replace=False)] = rng.choice([-3, 4, 7, 1000], 40)
        return ids, 4, 512
    if kind == "many_blocks":
        counts = rng.multinomial(120000, np.ones(16) / 16)
        ids = np.concatenate([np.r_[np.full(c, g), np.full((-c) % 128, -1)] for g, c in enumerate(counts)])
        return ids.astype(np.int32), 16, 256
    if kind == "no_split_k128":
        ids = np.repeat(np.arange(3, dtype=np.int32), 384)
        return ids, 3, 128
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["all_padding", "one_expert", "last_expert_only", "ids_out_of_range",
                                  "many_blocks", "no_split_k128"])
@pytest.mark.parametrize("ws", [True, False])
def test_plain_call_edge_ids(gpu_device, kind, ws):
    ids, G, K = plain_ids_case(kind)
    M, N = len(ids), 256
    rng = np.random.Generator(np.random.PCG64(32))
    a, sa_t = gen.quantize_lhs(gen.normal_with_outliers(rng, (M, K)))
    sa_t = np.ascontiguousarray(sa_t.T)
    b, sb = gen.make_grouped_rhs(G, N, K, 33)
    d = sentinel_bf16((M, N))
    args = (dev(a), dev(sa_t).t(), dev(b), dev(sb), dev(ids))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(M, N, K, G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, d=d)
    else:
        ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
    torch.cuda.synchronize()
    got = bits(d)
    # a block's expert is its largest id in [0, G); only rows with that id are written
    blk = np.where((ids >= 0) & (ids < G), ids, -1).reshape(-1, 128).max(axis=1)
    written = ids == np.repeat(blk, 128)
    written &= ids >= 0
    assert np.all(got[~written] == SENTINEL), kind
    if not written.any():
        return
    rows = np.nonzero(written)[0]
    if len(rows) > 4096:
        rows = np.sort(rng.choice(rows, 4096, replace=False))
    ns = np.tile(np.arange(0, N, 17), len(rows))
    rr = np.repeat(rows, len(np.arange(0, N, 17)))
    ref, _, produced = oracle.grouped_contiguous_points(a, sa_t.T, b, sb, ids, rr, ns)
    assert produced.all()
    assert_close(got[rr, ns], ref, "plain call edge case %s" % kind)


@pytest.mark.parametrize("G,N", [(64, 4096), (128, 4096), (64, 256), (128, 256)])
@pytest.mark.parametrize("ws", [True, False])
def test_plain_call_many_experts(gpu_device, G, N, ws):
    """8192 tokens over 64 or 128 experts, the plain call and the token-order
    call. With a workspace the offsets are derived on the device; at N 4096
    the experts' tails fill two rounds on their own, so they are not split
    over K (many 128-row tails on 256-row tiles), at N 256 they are split.
    Every routed row against the oracle, padding rows untouched."""
    T, K = 8192, 512
    e = np.random.Generator(np.random.PCG64(980 + G)).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 981, 982, 0, expert_of_token=e)
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(c.ids))
    tok = c.token_of_row.astype(np.int32)
    d = sentinel_bf16((c.M_total, N))
    out = sentinel_bf16((T, N))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, N, K, G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, d=d)
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, token_of_row=dev(tok), T=T, d=out)
    else:
        ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
        ops.dg_fp8_grouped_gemm_contiguous_to_tokens(*args, dev(tok), T, out=out)
    torch.cuda.synchronize()
    got, got_tok = bits(d), bits(out)
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    valid = c.ids >= 0
    assert np.all(got[~valid] == SENTINEL)
    assert_close(got[valid], ref[valid], "G=%d N=%d ws=%s" % (G, N, ws))
    assert np.array_equal(got_tok[tok[valid]], got[valid]), "token order equals the plain call's rows"


def test_ids_only_4_byte_aligned(gpu_device):
    """expert_ids need only 4-byte alignment: ids starting 4 bytes into an
    allocation (so not 16-byte aligned) give the same rows, bit for bit, as
    the same ids 16-byte aligned, through the call that derives the segment
    offsets from them on the device."""
    G, T, N, K = 6, 1500, 256, 512
    e = np.random.Generator(np.random.PCG64(990)).choice(G, T).astype(np.int32)
    c = gen.make_contiguous(G, T, N, K, 991, 992, 0, expert_of_token=e)
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb))
    buf = torch.zeros(c.M_total + 1, dtype=torch.int32, device="cuda")
    buf[1:] = dev(c.ids)
    ids_off = buf[1:]
    assert ids_off.data_ptr() % 16 == 4
    w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, N, K, G))
    d0, d1 = sentinel_bf16((c.M_total, N)), sentinel_bf16((c.M_total, N))
    ops.dg_fp8_grouped_gemm_contiguous_ws(*args, dev(c.ids), w, d=d0)
    ops.dg_fp8_grouped_gemm_contiguous_ws(*args, ids_off, w, d=d1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d0), bits(d1))
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids, np.full((c.M_total, N), SENTINEL, np.uint16))
    valid = c.ids >= 0
    assert_close(bits(d0)[valid], ref[valid], "aligned ids")
