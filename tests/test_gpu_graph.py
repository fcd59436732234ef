"""HIP-graph capture and replay through the C ABI.

The masked layout reads its per-group valid-row counts from device memory, and
the MoE routing step keeps its sizes on the device as well, so
one captured launch serves any counts (bhfrc.com DeepGEMM article, §4.3: shape
data kept in device memory avoids rebuilding the launch). Each test captures
once, then changes the inputs between replays, with eager work and
synchronisations in between, and checks every replay against an eager call on
the same inputs (bit for bit) and against the oracle.
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

COUNT_SETS = [
    [0, 17, 128, 64, 1, 127, 129, 255],
    [256] * 8,
    [0] * 8,
    [-5, 300, 3, 0, 256, 40, 2, 99],      # out-of-range counts are clamped to [0, M_max]
    [200, 0, 0, 0, 0, 0, 0, 1],
]


def masked_eager(a, sa, b, sb, mm, shape):
    d = sentinel_bf16(shape)
    ops.dg_fp8_grouped_gemm_masked(a, sa, b, sb, mm, d=d)
    torch.cuda.synchronize()
    return bits(d)


def check_masked(got, m, counts, ref_full):
    for g, c in enumerate(np.clip(counts, 0, m.M_max)):
        assert np.all(got[g, c:] == SENTINEL), "group %d: rows past the count were written" % g
        if c:
            assert_close(got[g, :c], ref_full[g, :c], "group %d" % g)


def test_masked_graph_replay_with_changing_counts(gpu_device):
    m = gen.make_masked(8, 256, 256, 512, 801, 802, 803, masked_m=np.full(8, 256))
    a, sa, b, sb = dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb)
    ref_full = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, np.full(8, 256, np.int32),
                                     np.zeros((8, 256, 256), np.uint16))
    mm = torch.zeros(8, dtype=torch.int32, device="cuda")
    d = sentinel_bf16((8, 256, 256))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        ops.dg_fp8_grouped_gemm_masked(a, sa, b, sb, mm, d=d)
    torch.cuda.synchronize()
    for counts in COUNT_SETS:
        mm.copy_(torch.tensor(counts, dtype=torch.int32))
        d.view(torch.int16).fill_(SENTINEL)           # eager fill kernel, not recorded in the graph
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(d)
        eager = masked_eager(a, sa, b, sb, mm, (8, 256, 256))
        assert np.array_equal(got, eager), "replay differs from the eager call for counts %s" % counts
        check_masked(got, m, np.array(counts), ref_full)


def test_quantize_then_gemm_graph_replay(gpu_device):
    """Activation quantiser and dense GEMM captured together; new activations
    are copied into the captured input buffer between replays."""
    M, N, K = 64, 384, 1024
    b, sb = gen.make_rhs(N, K, 811)
    bd, sbd = dev(b), dev(sb)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        ops.dg_fp8_quantize_1x128(x, q=q, s=s)
        ops.dg_fp8_gemm_nt(q, s, bd, sbd, d=d)
    torch.cuda.synchronize()
    for seed in (812, 813, 814):
        xh = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(seed)), (M, K)))
        xb = xh.to(torch.bfloat16)
        x.copy_(xb)
        d.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(d)
        q2, s2 = ops.dg_fp8_quantize_1x128(x)
        d2 = ops.dg_fp8_gemm_nt(q2, s2, bd, sbd)
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(d2)), "replay differs from the eager chain"
        ca, sa = oracle.quantize_1x128(xb)
        assert np.array_equal(q.cpu().numpy(), ca)
        ref = oracle.gemm_nt(ca, sa, b, sb)
        assert_close(got, ref, "quantise + GEMM replay, seed %d" % seed)


def test_masked_full_size_graph_replay(gpu_device):
    """The masked workload at its real shape (32 experts, M_max 256, N 4096,
    K 7168): replays with two count vectors equal the eager calls bit for bit,
    and sampled outputs match the oracle."""
    p = gen.make_config("moe_masked_g32_m256")
    a, sa, b, sb = dev(p.a), dev(p.sa_t).transpose(1, 2), dev(p.b), dev(p.sb)
    mm = dev(p.masked_m.astype(np.int32))
    shape = (p.G, p.M_max, p.N)
    d = sentinel_bf16(shape)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        ops.dg_fp8_grouped_gemm_masked(a, sa, b, sb, mm, d=d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for counts in (p.masked_m.astype(np.int32), rng.integers(0, 257, p.G).astype(np.int32)):
        mm.copy_(torch.from_numpy(counts))
        d.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(d)
        eager = masked_eager(a, sa, b, sb, mm, shape)
        assert np.array_equal(got, eager)
        for g in range(p.G):
            assert np.all(got[g, counts[g]:] == SENTINEL)
        gs = rng.integers(0, p.G, 256)
        ms = np.array([rng.integers(0, max(1, counts[g])) for g in gs])
        ns = rng.integers(0, p.N, 256)
        ref, _, produced = oracle.grouped_masked_points(p.a, p.sa_t, p.b, p.sb, counts, gs, ms, ns)
        sel = produced
        assert_close(got[gs[sel], ms[sel], ns[sel]], ref[sel], "full-size replay")


@pytest.mark.parametrize("K,use_layout,use_ws", [(512, False, False), (2048, True, True), (1024, False, True),
                                                (1024, True, False)])
def test_moe_step_graph_replay_with_changing_routing(gpu_device, K, use_layout, use_ws):
    """Routing, quantisation into the layout and the grouped GEMM to token
    order captured once; new routings and activations are copied into the
    captured buffers between replays. Nothing in the step reads sizes on the
    host, so every replay must equal the eager chain bit for bit. With a
    caller workspace the segments' last 128 rows are split over K (K 1024 and
    2048), and without the layout the segment offsets are derived into the
    workspace on the device; the slice count chosen on the device follows
    each routing."""
    T, G, N = 500, 6, 256
    b, sb = gen.make_grouped_rhs(G, N, K, 821)
    bd, sbd = dev(b), dev(sb)
    M_cap = ops.dg_moe_contiguous_max_rows(T, G)
    e_buf = torch.zeros(T, dtype=torch.int32, device="cuda")
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    row = torch.empty(T, dtype=torch.int32, device="cuda")
    ids = torch.empty(M_cap, dtype=torch.int32, device="cuda")
    tok = torch.empty(M_cap, dtype=torch.int32, device="cuda")
    layout = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    q = torch.empty((M_cap, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((K // 128, M_cap), dtype=torch.float32, device="cuda").t()
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(M_cap, N, K, G)) if use_ws else None
    lib = ops._lib.load()

    def step():
        st = lib.dg_moe_route_contiguous(e_buf.data_ptr(), T, G, row.data_ptr(), ids.data_ptr(), tok.data_ptr(),
                                         layout.data_ptr(), M_cap, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        ops.dg_fp8_quantize_1x128_gather(x, tok, q=q, s=s)
        if use_ws:
            ops.dg_fp8_grouped_gemm_contiguous_ws(q, s, bd, sbd, ids, w, token_of_row=tok, T=T,
                                                  layout=layout if use_layout else None, d=out)
        else:
            ops.dg_fp8_grouped_gemm_contiguous_to_tokens(q, s, bd, sbd, ids, tok, T,
                                                         layout=layout if use_layout else None, out=out)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    for seed in (822, 823, 824):
        rng = np.random.Generator(np.random.PCG64(seed))
        e = rng.choice(G, T).astype(np.int32)
        e[rng.random(T) < 0.05] = -1                      # a few dropped tokens
        if seed == 823:
            e[:] = 2                                      # everything to one expert
        xb = torch.from_numpy(gen.normal_with_outliers(rng, (T, K))).to(torch.bfloat16)
        e_buf.copy_(torch.from_numpy(e))
        x.copy_(xb)
        out.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out)
        r_row, r_ids, r_tok, r_layout = oracle.moe_route_contiguous(e, G, M_cap=M_cap)
        assert np.array_equal(row.cpu().numpy(), r_row) and np.array_equal(ids.cpu().numpy(), r_ids)
        assert np.array_equal(layout.cpu().numpy(), r_layout)
        out.view(torch.int16).fill_(SENTINEL)
        step()                                            # the same step, eager
        torch.cuda.synchronize()
        assert np.array_equal(got, bits(out)), "replay differs from the eager step (seed %d)" % seed
        kept = e >= 0
        assert np.all(got[~kept] == SENTINEL)
        xh = xb.view(torch.int16).numpy().view(np.uint16)
        rq, rs = oracle.quantize_1x128(xh[kept])
        ns = np.tile(np.arange(0, N, 37), kept.sum())
        rows = np.repeat(np.arange(kept.sum()), len(np.arange(0, N, 37)))
        ref, _, produced = oracle.grouped_contiguous_points(rq, rs, b, sb, e[kept], rows, ns)
        assert produced.all()
        assert_close(got[np.nonzero(kept)[0][rows], ns], ref, "MoE step replay, seed %d" % seed)
