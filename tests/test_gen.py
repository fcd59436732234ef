"""Pins of the seeded input generator (quantiser, encoder, routing layouts)."""
import numpy as np
import torch

import oracle
from synth import gen


def encode_e4m3_reference(v: np.ndarray) -> np.ndarray:
    """Independent e4m3 encoder: round to nearest, ties to even, |v| <= 448."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    E = np.maximum(ex - 1, -6)                 # binade; subnormals share 2^-6's quantum
    quantum = np.ldexp(1.0, E - 3)
    r = np.rint(a / quantum) * quantum         # ties to even
    _, ex2 = np.frexp(r)
    E2 = ex2 - 1
    normal = r >= 2.0 ** -6
    code = np.where(normal,
                    ((E2 + 7) << 3) + (np.where(normal, r / np.ldexp(1.0, E2 - 3), 8) - 8).astype(np.int64),
                    (r / 2.0 ** -9).astype(np.int64))
    code = np.where(r == 0, 0, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_reference_encoder_roundtrip_all_finite_codes():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = np.array([oracle.e4m3_decode(c) for c in finite])
    assert np.array_equal(encode_e4m3_reference(vals), finite)


def test_generator_encoder_matches_reference_encoder():
    rng = np.random.default_rng(0)
    x = (rng.random(2_000_000, dtype=np.float32) * 2 - 1) * np.float32(448)
    x[:1000] *= np.float32(1e-5)   # subnormal range
    ours = gen._encode(torch.from_numpy(x.copy())).numpy()
    assert np.array_equal(ours, encode_e4m3_reference(x))


def test_encoder_ties_to_even():
    vals = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 448.0, -448.0, 300.0], np.float32)
    codes = gen._encode(torch.from_numpy(vals)).numpy()
    dec = np.array([oracle.e4m3_decode(c) for c in codes])
    assert list(dec) == [1.0, 1.25, 0.0, 2.0 ** -9, 448.0, -448.0, 288.0]


def test_lhs_block_quantiser_invariants():
    rng = np.random.default_rng(1)
    x = gen.normal_with_outliers(rng, (37, 512))
    x[3, 128:256] = 0.0                         # an all-zero block
    codes, s = gen.quantize_lhs(x)
    assert codes.shape == (37, 512) and s.shape == (37, 4)
    assert s[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)])
    blocks = codes.reshape(37, 4, 128)
    for m in range(37):
        for kb in range(4):
            if m == 3 and kb == 1:
                continue
            amax = np.abs(x[m, kb * 128:(kb + 1) * 128]).max()
            assert s[m, kb] == np.float32(amax) / np.float32(448)
            assert s[m, kb] > 0
            assert np.any((blocks[m, kb] & 0x7F) == 0x7E)   # the amax lands on 448
            q = dec[blocks[m, kb]]
            # reconstruction error within half an e4m3 spacing (relative 2^-4), or
            # half the subnormal quantum
            err = np.abs(x[m, kb * 128:(kb + 1) * 128] / s[m, kb] - q)
            assert np.all(err <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) + 1e-6)


def test_rhs_block_quantiser_shares_scale_over_128x128():
    rng = np.random.default_rng(2)
    x = gen.normal_with_outliers(rng, (256, 384))
    codes, s = gen.quantize_rhs(x)
    assert s.shape == (2, 3)
    for nb in range(2):
        for kb in range(3):
            blk = x[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert s[nb, kb] == np.float32(np.abs(blk).max()) / np.float32(448)
            cb = codes[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert np.any((cb & 0x7F) == 0x7E)
            assert not np.any((cb & 0x7F) == 0x7F)   # never NaN


def test_outlier_rate_and_seed_reproducible():
    rng = np.random.default_rng(3)
    x = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(9)), (1000, 1000))
    y = gen.normal_with_outliers(np.random.Generator(np.random.PCG64(9)), (1000, 1000))
    assert np.array_equal(x, y)
    big = np.abs(x) > 10
    assert 600 < big.sum() < 1400     # ~0.1% * (P(|z|*50 > 10)) of 1e6
    del rng


def test_contiguous_layout():
    c = gen.make_contiguous(8, 1000, 128, 256, 1, 2, 3)
    assert c.M_total % 128 == 0
    assert c.counts.sum() == 1000
    row = 0
    for g in range(8):
        seg = int((c.counts[g] + 127) // 128 * 128)
        ids = c.ids[row:row + seg]
        assert np.all(ids[:c.counts[g]] == g) and np.all(ids[c.counts[g]:] == -1)
        toks = c.token_of_row[row:row + c.counts[g]]
        assert np.all(np.diff(toks) > 0)
        row += seg
    assert row == c.M_total
    pad = c.ids < 0
    assert np.all(c.a[pad] == 0) and np.all(c.sa_t[:, pad] == 1.0)
    # 128-row blocks hold one expert each
    for b in range(c.M_total // 128):
        blk = c.ids[b * 128:(b + 1) * 128]
        assert len(set(blk[blk >= 0].tolist())) == 1


def test_masked_counts_range():
    m = gen.make_masked(32, 256, 128, 128, 1, 2, 504)
    assert m.masked_m.dtype == np.int32
    assert m.masked_m.min() >= 0 and m.masked_m.max() <= 256
    assert m.sa_t.shape == (32, 1, 256)
