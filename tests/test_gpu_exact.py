"""GPU tests where the answer is exact: hand-worked cases, the MFMA's e4m3
decoding and operand layout, routing of the grouped layouts, determinism and
argument handling. All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_sa_amd import ops
from synth import gen
from tests import hand_cases
from tests.check import SENTINEL, assert_close
from tests.gpu_util import bits, dev, run_contiguous, run_dense, run_masked, sentinel_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", hand_cases.load(), ids=lambda c: c["name"])
def test_hand_cases_bit_exact(gpu_device, case):
    got = run_dense(case["a"], case["sa"], case["b"], case["sb"])
    if case["gpu_exact"]:
        assert np.array_equal(got, case["expect"]), case["name"]
    else:
        ok = (got == case["expect"]) | (got == case["gpu_alt"])
        assert ok.all(), case["name"]


def test_mfma_decodes_ocp_e4m3_and_layout(gpu_device):
    # Magnitudes in [1, 2) (codes 0x38..0x3F, either sign): every product is a
    # multiple of 2^-6 below 4 and every 128-term sum stays below 2^9, so the
    # fp32 MFMA result is exact and the bf16 output must equal the oracle's
    # single rounding bit for bit. A FNUZ decode (bias 8) would be off by 2x,
    # a wrong lane layout would mix rows/columns.
    rng = np.random.default_rng(123)
    M, N, K = 80, 256, 128
    pool = np.concatenate([np.arange(0x38, 0x40), np.arange(0xB8, 0xC0)]).astype(np.uint8)
    a = rng.choice(pool, (M, K))
    b = rng.choice(pool, (N, K))
    sa = np.ones((M, 1), np.float32)
    sb = np.ones((N // 128, 1), np.float32)
    ref = oracle.gemm_nt(a, sa, b, sb)
    for m_rows in (80, 8):   # tile kernel and small-M kernel
        got = run_dense(a[:m_rows], sa[:m_rows], b, sb)
        assert np.array_equal(got, ref[:m_rows])


def test_mfma_full_code_range(gpu_device):
    # All finite codes, including 448 and subnormals: within tolerance.
    rng = np.random.default_rng(7)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, N, K = 96, 128, 384
    a = rng.choice(finite, (M, K))
    b = rng.choice(finite, (N, K))
    sa = rng.uniform(0.5, 2, (M, 3)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (1, 3)).astype(np.float32)
    ref = oracle.gemm_nt(a, sa, b, sb)
    for m_rows in (96, 16):
        assert_close(run_dense(a[:m_rows], sa[:m_rows], b, sb), ref[:m_rows], "full code range")


def test_mfma_partial_against_exact_int64(gpu_device):
    """One K block through one FP8 MFMA against its exact value. A 128x128
    output split over its 8 K blocks (the split-K path, one block per slice)
    with unit scales leaves each block's fp32 MFMA partial in the caller's
    workspace ([slice][M][N] fp32, the promotion multiplying by 1). Each is
    compared with the exact sum, an int64 dot product of the codes' integer
    values (2^9 dec(code)) over 2^18. The error is measured against the sum of
    the terms' magnitudes, the scale an accumulation error has, and printed
    with the effective bits it leaves: the instruction does not accumulate
    its 128 products exactly (a few 1e-4 of the terms' magnitude), which is
    why each 128-wide block's partial is promoted into the fp32 accumulator
    on its own instead of being accumulated further inside the MFMA."""
    rng = np.random.default_rng(77)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M = N = 128
    K = 1024
    a = rng.choice(finite, (M, K))
    b = rng.choice(finite, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    nbytes = ops.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    ks = nbytes // (M * N * 4)
    assert ks == K // 128, "expected one K block per slice (%d slices)" % ks
    w = ops.workspace(nbytes)
    d = sentinel_bf16((M, N))
    ops.dg_fp8_gemm_nt_ws(dev(a), dev(np.ascontiguousarray(sa.T)).t(), dev(b), dev(sb), w, d=d)
    torch.cuda.synchronize()
    part = w[:ks * M * N * 4].view(torch.float32).cpu().numpy().reshape(ks, M, N).astype(np.float64)
    dec = np.array([oracle.e4m3_decode(c) if c not in (0x7F, 0xFF) else 0.0 for c in range(256)])
    ia = np.rint(dec[a] * 512).astype(np.int64)
    ib = np.rint(dec[b] * 512).astype(np.int64)
    worst = 0.0
    for s in range(ks):
        blk = slice(128 * s, 128 * s + 128)
        ex = (ia[:, blk] @ ib[:, blk].T).astype(np.float64) / 2.0 ** 18
        mag = (np.abs(ia[:, blk]) @ np.abs(ib[:, blk]).T).astype(np.float64) / 2.0 ** 18
        worst = max(worst, float((np.abs(part[s] - ex) / mag).max()))
    print("MFMA fp32 partial vs exact: max error %.3g of the terms' magnitude (%.1f bits)"
          % (worst, -np.log2(worst) if worst > 0 else float("inf")))
    assert worst <= 2.0 ** -10
    assert_close(bits(d), oracle.gemm_nt(a, sa, b, sb), "split-K partial test output")


def test_identity_rhs(gpu_device):
    p = gen.make_dense(100, 256, 256, 41, 42)
    b = np.zeros((256, 256), np.uint8)
    np.fill_diagonal(b, 0x38)
    sb = np.ones((2, 2), np.float32)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, b, sb)
    rep = assert_close(run_dense(p.a, p.sa_t.T, b, sb), ref, "identity")
    assert rep["le1ulp"] == rep["n"]


def test_all_ones_large_k(gpu_device):
    K = 7168
    a = np.full((70, K), 0x38, np.uint8)
    b = np.full((256, K), 0x38, np.uint8)
    sa = np.ones((70, K // 128), np.float32)
    sb = np.ones((2, K // 128), np.float32)
    want = oracle.bf16_rne(float(K))
    for m_rows in (70, 5):
        assert np.all(run_dense(a[:m_rows], sa[:m_rows], b, sb) == want)


# ---------------------------------------------------------------- routing

def signature_contiguous(G, expert_of_token, N=256, K=256):
    ids, tok, counts = gen.route_contiguous(np.asarray(expert_of_token), G)
    M_total = ids.shape[0]
    c = gen.Contiguous(G, N, K, M_total,
                       np.full((M_total, K), 0x38, np.uint8),
                       np.ones((K // 128, M_total), np.float32),
                       np.full((G, N, K), 0x38, np.uint8),
                       np.stack([np.full((N // 128, K // 128), e + 1, np.float32) for e in range(G)]),
                       ids, tok, counts)
    return c


def check_contiguous_signature(c, got, ids=None):
    ids = c.ids if ids is None else ids
    for r in range(c.M_total):
        e = ids[r]
        if 0 <= e < c.G:
            assert np.all(got[r] == oracle.bf16_rne(float(c.K * (e + 1)))), r
        else:
            assert np.all(got[r] == SENTINEL), r


@pytest.mark.parametrize("counts", [
    [1, 127, 128, 129, 256, 0, 3, 2],
    [8, 8],                                     # two experts x 8 tokens (fixed grouping)
    [0, 0, 0, 300],
    [255, 0, 1],
])
def test_contiguous_routing_signature(gpu_device, counts):
    G = len(counts)
    tokens = np.concatenate([np.full(n, e) for e, n in enumerate(counts)]).astype(np.int64)
    np.random.default_rng(0).shuffle(tokens)
    c = signature_contiguous(G, tokens)
    check_contiguous_signature(c, run_contiguous(c))


def test_contiguous_shuffled_segments_and_bad_ids(gpu_device):
    c = signature_contiguous(6, np.repeat(np.arange(6), [5, 130, 0, 128, 77, 1]))
    # permute whole 128-row blocks: segments in any order
    nblk = c.M_total // 128
    perm = np.random.default_rng(1).permutation(nblk)
    rows = (perm[:, None] * 128 + np.arange(128)[None, :]).ravel()
    ids = c.ids[rows].copy()
    c.ids = ids
    check_contiguous_signature(c, run_contiguous(c))
    # ids outside [0, G) are padding
    bad = ids.copy()
    pad_rows = np.nonzero(bad < 0)[0]
    bad[pad_rows[: len(pad_rows) // 2]] = 6      # == G
    bad[pad_rows[len(pad_rows) // 2:]] = -9
    check_contiguous_signature(c, run_contiguous(c, bad), bad)


@pytest.mark.parametrize("mm", [
    [0, 1, 127, 128, 129, 256, 200, 64],
    [-5, 1000, 0, 255],                         # clamped to [0, M_max]
])
def test_masked_routing_signature(gpu_device, mm):
    G, M_max, N, K = len(mm), 256, 256, 256
    m = gen.Masked(G, M_max, N, K,
                   np.full((G, M_max, K), 0x38, np.uint8),
                   np.ones((G, K // 128, M_max), np.float32),
                   np.full((G, N, K), 0x38, np.uint8),
                   np.stack([np.full((N // 128, K // 128), g + 1, np.float32) for g in range(G)]),
                   np.asarray(mm, np.int32))
    got = run_masked(m)
    for g in range(G):
        c = min(max(mm[g], 0), M_max)
        assert np.all(got[g, :c] == oracle.bf16_rne(float(K * (g + 1))))
        assert np.all(got[g, c:] == SENTINEL)


# ---------------------------------------------------------------- behaviour

def test_deterministic(gpu_device):
    p = gen.make_dense(300, 512, 1024, 5, 6)
    first = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    for _ in range(10):
        assert np.array_equal(run_dense(p.a, p.sa_t.T, p.b, p.sb), first)
    q = gen.make_dense(8, 1024, 2048, 7, 8)
    first = run_dense(q.a, q.sa_t.T, q.b, q.sb)
    for _ in range(10):
        assert np.array_equal(run_dense(q.a, q.sa_t.T, q.b, q.sb), first)


def test_strides_streams_and_broadcast_scales(gpu_device):
    p = gen.make_dense(130, 256, 512, 9, 10)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    # row-major sA
    assert np.array_equal(run_dense(p.a, np.ascontiguousarray(p.sa_t.T), p.b, p.sb),
                          run_dense(p.a, p.sa_t.T, p.b, p.sb))
    # padded leading dimensions for A, B and D
    a_pad = torch.zeros((130, 640), dtype=torch.uint8, device="cuda")
    a_pad[:, :512] = dev(p.a)
    b_pad = torch.zeros((256, 768), dtype=torch.uint8, device="cuda")
    b_pad[:, :512] = dev(p.b)
    d_pad = sentinel_bf16((130, 264))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.dg_fp8_gemm_nt(a_pad[:, :512], dev(p.sa_t).t(), b_pad[:, :512], dev(p.sb), d=d_pad[:, :256])
    s.synchronize()
    got = bits(d_pad)
    assert_close(got[:, :256], ref, "padded")
    assert np.all(got[:, 256:] == SENTINEL)
    # per-tensor scales through zero strides
    sa0 = torch.full((1, 1), 0.25, device="cuda").expand(130, 4)
    sb0 = torch.full((1, 1), 2.0, device="cuda").expand(2, 4)
    d = ops.dg_fp8_gemm_nt(dev(p.a), sa0, dev(p.b), sb0)
    torch.cuda.synchronize()
    ref0 = oracle.gemm_nt(p.a, np.full((130, 4), 0.25, np.float32), p.b, np.full((2, 4), 2.0, np.float32))
    assert_close(bits(d), ref0, "broadcast scales")


def test_errors_leave_output_untouched(gpu_device):
    p = gen.make_dense(64, 256, 512, 1, 2)
    d = sentinel_bf16((64, 256))
    with pytest.raises(ops.DGError) as e:
        ops.dg_fp8_gemm_nt(dev(p.a)[:, :500], dev(p.sa_t).t()[:, :3], dev(p.b)[:, :500],
                           dev(p.sb)[:, :3], d=d)
    torch.cuda.synchronize()
    assert np.all(bits(d) == SENTINEL)
    assert e.value.status in (2, 3)
    with pytest.raises(ValueError):
        ops.dg_fp8_gemm_nt(torch.from_numpy(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb), d=d)


def test_empty_problems(gpu_device):
    d = ops.dg_fp8_gemm_nt(torch.zeros((0, 256), dtype=torch.uint8, device="cuda"),
                           torch.zeros((0, 2), device="cuda"),
                           torch.zeros((128, 256), dtype=torch.uint8, device="cuda"),
                           torch.zeros((1, 2), device="cuda"))
    assert d.shape == (0, 128)


def test_split_k_workspace_in_graph_capture(gpu_device):
    # M=96, N=512 gives 4 tiles of 128x128, so with a workspace the K blocks
    # are split over work items whose fp32 partials go to the caller's
    # workspace, and a second kernel adds them in a fixed order. A captured
    # graph keeps the workspace it was given. A later, larger split call on
    # the same stream with its own workspace, and that workspace being freed,
    # cannot disturb the graph (the library owns no memory): every replay
    # equals the first eager result bit for bit.
    p = gen.make_dense(96, 512, 1024, 61, 62)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    a, sa, b, sb = dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)
    need = ops.dg_fp8_gemm_nt_workspace_bytes(96, 512, 1024)
    assert need == 8 * 96 * 512 * 4          # 8 slices of fp32 partials
    ws1 = ops.workspace(need)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    d = sentinel_bf16((96, 512))
    with torch.cuda.stream(s):
        ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, ws1, d=d)
    s.synchronize()
    eager = bits(d)
    assert_close(eager, ref, "split-K eager")
    unsplit = run_dense(p.a, p.sa_t.T, p.b, p.sb)          # no workspace: one K loop per tile
    assert_close(unsplit, ref, "unsplit")

    g = torch.cuda.CUDAGraph()
    d2 = sentinel_bf16((96, 512))
    with torch.cuda.graph(g, stream=s):
        ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, ws1, d=d2)

    q = gen.make_dense(200, 1024, 2048, 63, 64)           # a larger split call
    qref = oracle.gemm_nt(q.a, q.sa_t.T, q.b, q.sb)
    qa, qsa, qb, qsb = dev(q.a), dev(q.sa_t).t(), dev(q.b), dev(q.sb)
    need2 = ops.dg_fp8_gemm_nt_workspace_bytes(200, 1024, 2048)
    assert need2 > need
    for r in range(3):
        ws2 = ops.workspace(need2)
        with torch.cuda.stream(s):
            dq = ops.dg_fp8_gemm_nt_ws(qa, qsa, qb, qsb, ws2, d=sentinel_bf16((200, 1024)))
        s.synchronize()
        assert_close(bits(dq), qref, "larger split call %d" % r)
        del ws2, dq
        torch.cuda.empty_cache()
        d2.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert np.array_equal(bits(d2), eager), "replay %d" % r


def test_split_k_partial_workspace(gpu_device):
    # A workspace that holds fewer slices than the query asks for takes as
    # many as it holds (here 3 of 8): a different grouping of the fp32 sums,
    # so within tolerance of the oracle, and the same bits on every call.
    p = gen.make_dense(96, 512, 1024, 65, 66)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    a, sa, b, sb = dev(p.a), dev(p.sa_t).t(), dev(p.b), dev(p.sb)
    ws = ops.workspace(3 * 96 * 512 * 4 + 100)
    first = None
    for _ in range(5):
        d = ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, ws, d=sentinel_bf16((96, 512)))
        torch.cuda.synchronize()
        got = bits(d)
        if first is None:
            first = got
            assert_close(got, ref, "3 slices")
        assert np.array_equal(got, first)
    tiny = ops.workspace(96 * 512 * 4)                  # one slice: no split at all
    d = ops.dg_fp8_gemm_nt_ws(a, sa, b, sb, tiny, d=sentinel_bf16((96, 512)))
    torch.cuda.synchronize()
    assert np.array_equal(bits(d), run_dense(p.a, p.sa_t.T, p.b, p.sb))
