"""Pins of the oracle's MoE routing into the contiguous layout and its way back.

Tokens are regrouped by expert (lpnh.cn article, §5.3), each expert's rows
padded to a multiple of 128 (bhfrc.com article, §4.2), and every row carries
its group id and source token (rkmt.cn walkthrough, §5.3). Fixed by: the
generator's independent numpy routing, a hand-worked 2-expert x 8-token case,
structural invariants, and planted mistakes in compiled copies of the oracle.
"""
import ctypes
import subprocess

import numpy as np
import pytest

import oracle
from synth import gen
from tests.test_oracle_quant import ORACLE_SRC


def check_invariants(e, G, row, ids, tok, layout):
    T = len(e)
    valid = (e >= 0) & (e < G)
    counts = np.bincount(e[valid], minlength=G)
    padded = (counts + 127) // 128 * 128
    assert np.array_equal(layout, np.concatenate([[0], np.cumsum(padded)]).astype(np.int32))
    assert np.all(row[~valid] == -1)
    vt = np.nonzero(valid)[0]
    assert np.array_equal(tok[row[vt]], vt)                 # every routed token sits in its row
    assert np.array_equal(ids[row[vt]], e[vt])
    assert np.count_nonzero(tok >= 0) == len(vt)             # and only there
    for g in range(G):
        seg = slice(layout[g], layout[g + 1])
        t = tok[seg][: counts[g]]
        assert np.all(np.diff(t) > 0)                        # ascending token order
        assert np.all(ids[seg][: counts[g]] == g)
        assert np.all(ids[seg][counts[g]:] == -1) and np.all(tok[seg][counts[g]:] == -1)
    assert np.all(ids[layout[G]:] == -1) and np.all(tok[layout[G]:] == -1)
    blocks = ids.reshape(-1, 128)
    for blk in blocks:                                       # one expert per aligned 128-row block
        assert len(set(blk[blk >= 0].tolist())) <= 1


def test_two_experts_eight_tokens_by_hand():
    e = np.array([1, 0, 1, 1, 0, 0, 1, 0], np.int32)
    row, ids, tok, layout = oracle.moe_route_contiguous(e, 2, M_cap=384)
    assert layout.tolist() == [0, 128, 256]
    assert row.tolist() == [128, 0, 129, 130, 1, 2, 131, 3]
    assert tok[:4].tolist() == [1, 4, 5, 7] and tok[128:132].tolist() == [0, 2, 3, 6]
    assert ids[:4].tolist() == [0] * 4 and ids[128:132].tolist() == [1] * 4
    assert np.all(ids[4:128] == -1) and np.all(ids[132:] == -1) and np.all(tok[256:] == -1)


@pytest.mark.parametrize("T,G,seed", [(8192, 8, 403), (1000, 32, 1), (64, 256, 2), (5, 3, 3), (300, 1, 4)])
def test_routing_matches_the_generator(T, G, seed):
    e = np.random.Generator(np.random.PCG64(seed)).choice(G, T).astype(np.int32)
    row, ids, tok, layout = oracle.moe_route_contiguous(e, G)
    ids2, tok2, counts = gen.route_contiguous(e, G)
    M = len(ids2)
    assert layout[G] == M
    assert np.array_equal(ids[:M], ids2) and np.array_equal(tok[:M], tok2)
    check_invariants(e, G, row, ids, tok, layout)


def test_routing_edge_cases():
    G = 6
    e = np.array([5, -1, 2, 6, 2, 100, 5, 0], np.int32)          # ids outside [0, G) are dropped
    row, ids, tok, layout = oracle.moe_route_contiguous(e, G)
    assert row[1] == -1 and row[3] == -1 and row[5] == -1
    check_invariants(e, G, row, ids, tok, layout)
    e = np.zeros(129, np.int32)                                   # one expert, 129 tokens: two blocks
    row, ids, tok, layout = oracle.moe_route_contiguous(e, 4)
    assert layout.tolist() == [0, 256, 256, 256, 256]
    check_invariants(e, 4, row, ids, tok, layout)
    row, ids, tok, layout = oracle.moe_route_contiguous(np.zeros(0, np.int32), 4, M_cap=128)
    assert layout.tolist() == [0] * 5 and np.all(ids == -1)
    assert oracle.moe_max_rows(8192, 8) == 128 * (64 + 8)
    with pytest.raises(ValueError):
        oracle.moe_route_contiguous(np.arange(4, dtype=np.int32), 4, M_cap=256)


def test_unpermute_is_a_row_gather():
    rng = np.random.default_rng(6)
    d = rng.integers(0, 65536, size=(512, 256), dtype=np.uint16)
    r = rng.integers(-3, 515, size=300).astype(np.int32)
    out = oracle.moe_unpermute(d, r)
    ok = (r >= 0) & (r < 512)
    assert np.array_equal(out[ok], d[r[ok]]) and np.all(out[~ok] == 0)


MUTANTS = {
    "descending token order": ("for (int64_t t = 0; t < T; ++t) {\n        int64_t e = expert_of_token[t];\n        if (e < 0 || e >= G) {",
                               "for (int64_t t = T - 1; t >= 0; --t) {\n        int64_t e = expert_of_token[t];\n        if (e < 0 || e >= G) {"),
    "no padding": ("row += (count[e] + BLK - 1) / BLK * BLK;", "row += count[e];"),
    "ids not cleared": ("        expert_ids[r] = -1;\n", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, name
    (tmp_path / "m.c").write_text(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(tmp_path / "m.c"),
                           "-o", str(tmp_path / "m.so"), "-lm"])
    lib = ctypes.CDLL(str(tmp_path / "m.so"))
    G, T = 8, 1000
    e = np.random.Generator(np.random.PCG64(7)).choice(G, T).astype(np.int32)
    M_cap = oracle.moe_max_rows(T, G)
    row, ids, tok, layout = (np.zeros(T, np.int32), np.full(M_cap, 77, np.int32),
                             np.zeros(M_cap, np.int32), np.zeros(G + 1, np.int32))
    p = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    lib.dgo_moe_route_contiguous(p(e), ctypes.c_int64(T), ctypes.c_int64(G), p(row), p(ids), p(tok),
                                 p(layout), ctypes.c_int64(M_cap))
    ids2, tok2, _ = gen.route_contiguous(e, G)
    M = len(ids2)
    same = (np.array_equal(ids[:M], ids2) and np.array_equal(tok[:M], tok2) and np.all(ids[M:] == -1))
    assert not same, name
