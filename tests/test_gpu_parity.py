"""GPU vs oracle parity on seeded inputs, through the C ABI.

Small and ragged shapes are compared element by element over the whole
output; the full-size workloads are compared on sampled outputs (plus whole
rows and columns) that the oracle computes one by one, and on properties that
hold everywhere (every valid element written, every other row untouched).
"""
import numpy as np
import pytest

import oracle
from synth import gen
from tests.check import SENTINEL, assert_close
from tests.gpu_util import run_contiguous, run_dense, run_masked

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [
    (64, 256, 512),       # the small dense workload
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


@pytest.mark.parametrize("M", [40, 96, 256])   # split over K: 128x128 / 256x128 tiles + reduction
def test_medium_m_full_parity(gpu_device, M):
    p = gen.make_dense(M, 4096, 7168, 3000 + M, 4000 + M)
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    assert_close(got, ref, "dense %dx4096x7168" % M)


def test_decode_full_parity(gpu_device):
    p = gen.make_config("decode_8x4096x7168")
    ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    rep = assert_close(got, ref, "decode 8x4096x7168")
    assert rep["le1ulp"] >= 0.99 * rep["n"]


def sample_points(M, N, count, seed):
    rng = np.random.default_rng(seed)
    ms = [rng.integers(0, M, count), np.zeros(N, np.int64), np.full(N, M - 1),
          np.arange(M), np.arange(M)]
    ns = [rng.integers(0, N, count), np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1)]
    return np.concatenate(ms), np.concatenate(ns)


@pytest.mark.parametrize("name", ["square_4096", "prefill_8192x7168x2048"])
def test_large_dense_sampled_parity(gpu_device, name):
    p = gen.make_config(name)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    assert not np.any(got == SENTINEL), "every output element is written"
    ms, ns = sample_points(p.M, p.N, 20000, 5)
    ref, _ = oracle.gemm_nt_points(p.a, p.sa_t.T, p.b, p.sb, ms, ns)
    assert_close(got[ms, ns], ref, name)


@pytest.mark.parametrize("M,N", [(4096, 4352), (4352, 4096)])
def test_round_cut_sampled_parity(gpu_device, M, N):
    # 272 tiles of 256x256 leave a last round of 16 on 256 CUs: the first
    # 4096 columns (rows) run as whole rounds and the remaining strip as a
    # second launch on smaller tiles. Every element written; sampled points
    # (with whole rows and columns on both sides of the cut) against the oracle.
    p = gen.make_dense(M, N, 512, 5000 + M, 6000 + N)
    got = run_dense(p.a, p.sa_t.T, p.b, p.sb)
    assert not np.any(got == SENTINEL), "every output element is written"
    ms, ns = sample_points(p.M, p.N, 20000, 9)
    cut_m = np.concatenate([np.full(N, 4095), np.full(N, min(4096, M - 1))])
    cut_n = np.concatenate([np.arange(N), np.arange(N)])
    ms, ns = np.concatenate([ms, cut_m, np.arange(M), np.arange(M)]), np.concatenate([ns, cut_n, np.full(M, 4095), np.full(M, min(4096, N - 1))])
    ref, _ = oracle.gemm_nt_points(p.a, p.sa_t.T, p.b, p.sb, ms, ns)
    assert_close(got[ms, ns], ref, "round cut %dx%d" % (M, N))


@pytest.mark.parametrize("N", [384, 512])   # 256x128 and 256x256 tiles
def test_small_contiguous_full_parity(gpu_device, N):
    # Segments of 1, 3, 1, 2 and 1 128-row blocks: three of the four 256-row
    # tiles hold two experts (a pass per expert).
    counts = [100, 300, 50, 129, 121]
    tokens = np.repeat(np.arange(5), counts)
    np.random.default_rng(14).shuffle(tokens)
    c = gen.make_contiguous(5, len(tokens), N, 640, 11, 12, 13, expert_of_token=tokens)
    assert c.M_total == 8 * 128
    ref = oracle.grouped_contiguous(c.a, c.sa_t.T, c.b, c.sb, c.ids,
                                    np.full((c.M_total, c.N), SENTINEL, np.uint16))
    got = run_contiguous(c)
    pad = c.ids < 0
    assert np.all(got[pad] == SENTINEL)
    assert_close(got[~pad], ref[~pad], "contiguous small")


def test_moe_contiguous_full_size(gpu_device):
    c = gen.make_config("moe_contiguous_g8_t8192")
    got = run_contiguous(c)
    pad = c.ids < 0
    assert np.all(got[pad] == SENTINEL), "padding rows untouched"
    assert not np.any(got[~pad] == SENTINEL), "every routed row fully written"
    real = np.nonzero(~pad)[0]
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.choice(real, 20000), np.repeat(real[[0, -1]], c.N)])
    ns = np.concatenate([rng.integers(0, c.N, 20000), np.tile(np.arange(c.N), 2)])
    ref, _, prod = oracle.grouped_contiguous_points(c.a, c.sa_t.T, c.b, c.sb, c.ids, rows, ns)
    assert prod.all()
    assert_close(got[rows, ns], ref, "moe contiguous")


@pytest.mark.parametrize("N", [256, 384])   # 256x256 and 256x128 tiles
def test_small_masked_full_parity(gpu_device, N):
    m = gen.make_masked(6, 200, N, 512, 21, 22, 23, masked_m=np.array([0, 1, 200, 77, 128, 129]))
    ref = oracle.grouped_masked(m.a, m.sa_t, m.b, m.sb, m.masked_m,
                                np.full((m.G, m.M_max, m.N), SENTINEL, np.uint16))
    got = run_masked(m)
    for g in range(m.G):
        c = int(m.masked_m[g])
        assert np.all(got[g, c:] == SENTINEL)
        if c:
            assert_close(got[g, :c], ref[g, :c], "masked small g%d" % g)


def test_moe_masked_full_size(gpu_device):
    m = gen.make_config("moe_masked_g32_m256")
    got = run_masked(m)
    for g in range(m.G):
        c = int(m.masked_m[g])
        assert np.all(got[g, c:] == SENTINEL), "rows past the count untouched"
        assert not np.any(got[g, :c] == SENTINEL), "valid rows fully written"
    valid = [(g, r) for g in range(m.G) for r in range(int(m.masked_m[g]))]
    rng = np.random.default_rng(4)
    pick = rng.integers(0, len(valid), 20000)
    gs = np.array([valid[i][0] for i in pick])
    ms = np.array([valid[i][1] for i in pick])
    ns = rng.integers(0, m.N, 20000)
    ref, _, prod = oracle.grouped_masked_points(m.a, m.sa_t, m.b, m.sb, m.masked_m, gs, ms, ns)
    assert prod.all()
    assert_close(got[gs, ms, ns], ref, "moe masked")
