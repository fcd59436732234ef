"""GPU MoE routing, gather-quantisation and un-permute vs the oracle, and the
whole contiguous MoE step (route -> quantise into the layout -> grouped GEMM
-> back to token order), through the C ABI.

Routing, codes, scales and the row copy are integer/bit results and must
agree exactly; the GEMM output is held to the bf16 tolerance.
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


def route_both(e, G, M_cap=None):
    got = [t.cpu().numpy() for t in ops.dg_moe_route_contiguous(dev(e.astype(np.int32)), G, M_cap=M_cap)]
    ref = oracle.moe_route_contiguous(e, G, M_cap=M_cap if M_cap is not None else oracle.moe_max_rows(len(e), G))
    return got, ref


@pytest.mark.parametrize("T,G,seed", [
    (8192, 8, 403),      # the contiguous MoE workload's routing
    (1000, 32, 1), (64, 256, 2), (5, 3, 3), (300, 1, 4), (4096, 1024, 5), (777, 7, 6), (65, 64, 7),
    (20000, 100, 8), (8192, 2, 9), (3000, 65, 10), (10000, 1000, 11),
])
def test_route_matches_oracle(gpu_device, T, G, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    # seeds from 8 on: skewed expert loads (Dirichlet weights), some ids dropped
    p = rng.dirichlet(np.full(G, 0.3)) if seed >= 8 else None
    e = rng.choice(G, T, p=p).astype(np.int32)
    if seed >= 8:
        e[rng.random(T) < 0.02] = -1
    got, ref = route_both(e, G)
    for name, g, r in zip(("row_of_token", "expert_ids", "token_of_row", "layout"), got, ref):
        assert np.array_equal(g, r), name


def test_route_edge_cases(gpu_device):
    e = np.array([5, -1, 2, 6, 2, 100, 5, 0] * 40, np.int32)     # ids outside [0, 6) dropped
    got, ref = route_both(e, 6)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    e = np.zeros(129, np.int32)                                   # one expert, two blocks
    got, ref = route_both(e, 4, M_cap=1024)                       # capacity above the minimum
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    e = np.full(2000, 3, np.int32)                                # skewed: all to the last expert
    got, ref = route_both(e, 4)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_route_empty(gpu_device):
    row, ids, tok, layout = ops.dg_moe_route_contiguous(torch.zeros(0, dtype=torch.int32, device="cuda"), 4,
                                                        M_cap=128)
    torch.cuda.synchronize()
    assert layout.cpu().tolist() == [0] * 5
    assert np.all(ids.cpu().numpy() == -1) and np.all(tok.cpu().numpy() == -1)


def gathered(x, src):
    """Host-side gather for the oracle: rows x[src], zeros where src is out of range."""
    out = np.zeros((len(src), x.shape[1]), x.dtype)
    ok = (src >= 0) & (src < x.shape[0])
    out[ok] = x[src[ok]]
    return out


@pytest.mark.parametrize("bf16", [False, True])
def test_gather_quantize_matches_oracle(gpu_device, bf16):
    T, K = 300, 1152
    x = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(901)), (T, K))
    src = np.random.default_rng(0).integers(-2, T + 2, size=520).astype(np.int32)
    xt = torch.from_numpy(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
    q, s = ops.dg_fp8_quantize_1x128_gather(xt.cuda(), dev(src))
    torch.cuda.synchronize()
    xh = xt.contiguous().view(torch.int16).numpy().view(np.uint16) if bf16 else x
    ref_q, ref_s = oracle.quantize_1x128(gathered(xh, src))
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    pad = (src < 0) | (src >= T)
    assert np.all(q.cpu().numpy()[pad] == 0) and np.all(s.cpu().numpy()[pad] == 1.0)


def test_unpermute_matches_oracle(gpu_device):
    rng = np.random.default_rng(8)
    d = rng.integers(0, 65536, size=(640, 384), dtype=np.uint16)
    r = rng.integers(-3, 643, size=1000).astype(np.int32)
    out = ops.dg_moe_unpermute(dev(d.view(np.int16)).view(torch.bfloat16), dev(r))
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.moe_unpermute(d, r))


def moe_step_gpu(x, e, b, sb, G):
    """route -> quantise into the layout -> contiguous grouped GEMM over M_cap rows -> token order."""
    xd, ed = x.cuda(), dev(e)
    row, ids, tok, layout = ops.dg_moe_route_contiguous(ed, G)
    q, s = ops.dg_fp8_quantize_1x128_gather(xd, tok)
    d = ops.dg_fp8_grouped_gemm_contiguous(q, s, dev(b), dev(sb), ids)
    out = ops.dg_moe_unpermute(d, row)
    fused = torch.zeros_like(out)                  # dropped tokens: zeros, as the un-permute writes
    ops.dg_fp8_grouped_gemm_contiguous_to_tokens(q, s, dev(b), dev(sb), ids, tok, x.shape[0], out=fused)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), out.view(torch.int16)), "fused epilogue differs from GEMM + un-permute"
    return out, row.cpu().numpy(), ids.cpu().numpy(), tok.cpu().numpy(), q.cpu().numpy(), s.cpu().numpy()


def test_to_tokens_equals_gemm_then_unpermute(gpu_device):
    """The GEMM written straight to token order equals the GEMM followed by
    the un-permute bit for bit; rows of dropped tokens stay untouched."""
    T, G, N, K = 700, 5, 384, 1024
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(931)), (T, K)))
    e = np.random.Generator(np.random.PCG64(932)).choice(G, T).astype(np.int32)
    e[::11] = -1
    b, sb = gen.make_grouped_rhs(G, N, K, 933)
    bd, sbd = dev(b), dev(sb)
    row, ids, tok, _ = ops.dg_moe_route_contiguous(dev(e), G)
    q, s = ops.dg_fp8_quantize_1x128_gather(x.cuda(), tok)
    d = ops.dg_fp8_grouped_gemm_contiguous(q, s, bd, sbd, ids)
    ref = ops.dg_moe_unpermute(d, row)
    out = sentinel_bf16((T, N))
    ops.dg_fp8_grouped_gemm_contiguous_to_tokens(q, s, bd, sbd, ids, tok, T, out=out)
    torch.cuda.synchronize()
    got, want = bits(out), bits(ref)
    kept = e >= 0
    assert np.array_equal(got[kept], want[kept])
    assert np.all(got[~kept] == SENTINEL)


def test_moe_step_small_full_parity(gpu_device):
    T, G, N, K = 300, 4, 256, 512
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(911)), (T, K)))
    x = x.to(torch.bfloat16)
    e = np.random.Generator(np.random.PCG64(912)).choice(G, T).astype(np.int32)
    e[::37] = -1                                                  # some tokens dropped
    b, sb = gen.make_grouped_rhs(G, N, K, 913)
    out, row, ids, tok, q, s = moe_step_gpu(x, e, b, sb, G)
    # the oracle pipeline, step by step
    r_row, r_ids, r_tok, _ = oracle.moe_route_contiguous(e, G)
    assert np.array_equal(row, r_row) and np.array_equal(ids, r_ids) and np.array_equal(tok, r_tok)
    xh = x.view(torch.int16).numpy().view(np.uint16)
    rq, rs = oracle.quantize_1x128(gathered(xh, r_tok))
    assert np.array_equal(q, rq) and np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    d = oracle.grouped_contiguous(rq, rs, b, sb, r_ids, np.zeros((len(r_ids), N), np.uint16))
    ref = oracle.moe_unpermute(d, r_row)
    got = bits(out)
    kept = r_row >= 0
    assert np.all(got[~kept] == 0)
    assert_close(got[kept], ref[kept], "MoE step %d tokens" % T)


def test_moe_step_full_size_sampled(gpu_device):
    """8 experts, 8192 tokens (the contiguous MoE workload's routing seed),
    K 7168, N 4096, bf16 activations: exact routing and codes, sampled
    outputs against the oracle."""
    c = gen.CONFIGS["moe_contiguous_g8_t8192"]
    G, T, N, K = c["G"], c["tokens"], c["N"], c["K"]
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(921)), (T, K)))
    x = x.to(torch.bfloat16)
    e = np.random.Generator(np.random.PCG64(c["seeds"][2])).choice(G, T).astype(np.int32)
    b, sb = gen.make_grouped_rhs(G, N, K, c["seeds"][1])
    out, row, ids, tok, q, s = moe_step_gpu(x, e, b, sb, G)
    r_row, r_ids, r_tok, _ = oracle.moe_route_contiguous(e, G)
    assert np.array_equal(row, r_row) and np.array_equal(ids, r_ids) and np.array_equal(tok, r_tok)
    rng = np.random.default_rng(9)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
    xh = x.view(torch.int16).numpy().view(np.uint16)
    rq, rs = oracle.quantize_1x128(xh[toks])
    assert np.array_equal(q[row[toks]], rq)
    assert np.array_equal(s[row[toks]].view(np.uint32), rs.view(np.uint32))
    pad = ids < 0
    assert np.all(q[pad] == 0) and np.all(s[pad] == 1.0)
    ns = rng.integers(0, N, size=(len(toks), 8))
    rows = np.repeat(np.arange(len(toks)), 8)
    ref, _, produced = oracle.grouped_contiguous_points(rq, rs, b, sb, e[toks], rows, ns.ravel())
    assert produced.all()
    got = bits(out)[np.repeat(toks, 8), ns.ravel()]
    assert_close(got, ref, "MoE step, sampled tokens")
