"""Seeded synthetic inputs for the block-scaled FP8 GEMM.

Shared by the tests, the benchmark and the smoke check. This module holds none
of the GEMM's arithmetic: it only draws fp32 data, quantises it to e4m3 codes
with per-block ``amax / 448`` scales (the initial-scale recipe of the rkmt.cn
DeepGEMM walkthrough, §5.2), and lays out MoE routing.

Input recipe (the same for every workload):

* ``x = N(0, 1)`` in fp32 from ``numpy.random.PCG64(seed)``; then every entry
  independently becomes an outlier with probability 1e-3, in which case it is
  multiplied by 50 (keeping its sign).
* LHS blocks are 1x128 along K, RHS blocks are 128x128 (hotdry.top
  fine-grained scaling article, "fine-grained scaling core design").
* Per block: ``s = amax / 448`` as an fp32 division (``s = 1`` for an all-zero
  block), ``q = e4m3_rne(clamp(x / s, -448, 448))`` with ``x / s`` an fp32
  division, so that ``x ~ dec(q) * s``.

Layouts produced (logical shapes, physical order):

* LHS scales are stored M-major: an array ``[K/128, M]`` whose element
  ``[kb, m]`` is ``sA[m, kb]`` (``sa_stride_m = 1``, ``sa_stride_kb = M``).
* RHS scales are stored row-major ``[N/128, K/128]``.
* Contiguous MoE: rows grouped by expert in ascending expert id, tokens in
  ascending order inside a segment, each segment padded to a multiple of 128
  rows with padding rows whose expert id is -1 (codes 0, scale 1).
* Masked MoE: ``A [G, M_max, K]`` fully generated (rows past the count hold
  ordinary data that must not reach the output), ``masked_m[g]`` drawn
  uniformly from ``{0, ..., M_max}``.

The e4m3 encoding uses torch's CPU ``float8_e4m3fn`` cast (round to nearest,
ties to even); the tests pin it against an independent encoder.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
# operand formats: largest finite value and torch dtype of the encoder
FORMATS = {"e4m3": (E4M3_MAX, torch.float8_e4m3fn), "e5m2": (E5M2_MAX, torch.float8_e5m2)}
BLOCK = 128
OUTLIER_P = 1e-3
OUTLIER_MUL = 50.0
GEN_VERSION = 1


def normal_with_outliers(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 N(0,1) with 0.1% of entries scaled by 50 (independent Bernoulli)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    out = rng.random(shape, dtype=np.float32) < np.float32(OUTLIER_P)
    x[out] *= np.float32(OUTLIER_MUL)
    return x


def _encode(q: torch.Tensor, fmt: str = "e4m3") -> torch.Tensor:
    fmax, dtype = FORMATS[fmt]
    q = torch.clamp(q, -fmax, fmax)
    return q.to(dtype).view(torch.uint8)


def _block_scale(amax: torch.Tensor, fmt: str = "e4m3") -> torch.Tensor:
    s = amax / torch.tensor(FORMATS[fmt][0], dtype=torch.float32)
    return torch.where(amax == 0, torch.ones_like(s), s)


def quantize_lhs(x: np.ndarray, fmt: str = "e4m3"):
    """1x128 block quantisation of ``x [M, K]``.

    Returns ``(codes [M, K] uint8, scales [M, K/128] fp32)`` (row-major scales;
    callers transpose to M-major).
    """
    M, K = x.shape
    assert K % BLOCK == 0
    t = torch.from_numpy(np.ascontiguousarray(x)).view(M, K // BLOCK, BLOCK)
    amax = t.abs().amax(dim=2)
    s = _block_scale(amax, fmt)
    codes = _encode(t / s.unsqueeze(2), fmt).reshape(M, K)
    return codes.numpy(), s.numpy()


def quantize_rhs(x: np.ndarray, fmt: str = "e4m3"):
    """128x128 block quantisation of ``x [N, K]``.

    Returns ``(codes [N, K] uint8, scales [N/128, K/128] fp32)``.
    """
    N, K = x.shape
    assert N % BLOCK == 0 and K % BLOCK == 0
    t = torch.from_numpy(np.ascontiguousarray(x)).view(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = t.abs().amax(dim=(1, 3))
    s = _block_scale(amax, fmt)
    codes = _encode(t / s[:, None, :, None], fmt).reshape(N, K)
    return codes.numpy(), s.numpy()


@dataclasses.dataclass
class Dense:
    """Dense NT problem ``D[M,N] = A[M,K] . B[N,K]^T`` with block scales."""
    M: int
    N: int
    K: int
    a: np.ndarray        # uint8 [M, K]
    sa_t: np.ndarray     # fp32 [K/128, M]  (M-major sA)
    b: np.ndarray        # uint8 [N, K]
    sb: np.ndarray       # fp32 [N/128, K/128]


@dataclasses.dataclass
class Contiguous:
    """Contiguous MoE layout: rows of all experts stacked, one expert id per row."""
    G: int
    N: int
    K: int
    M_total: int
    a: np.ndarray        # uint8 [M_total, K]
    sa_t: np.ndarray     # fp32 [K/128, M_total]
    b: np.ndarray        # uint8 [G, N, K]
    sb: np.ndarray       # fp32 [G, N/128, K/128]
    ids: np.ndarray      # int32 [M_total], -1 for padding rows
    token_of_row: np.ndarray  # int64 [M_total], source token index or -1
    counts: np.ndarray   # int64 [G] tokens per expert


@dataclasses.dataclass
class Masked:
    """Masked MoE layout: per-expert fixed-capacity row blocks plus a valid-row count."""
    G: int
    M_max: int
    N: int
    K: int
    a: np.ndarray        # uint8 [G, M_max, K]
    sa_t: np.ndarray     # fp32 [G, K/128, M_max]
    b: np.ndarray        # uint8 [G, N, K]
    sb: np.ndarray       # fp32 [G, N/128, K/128]
    masked_m: np.ndarray  # int32 [G]


def make_lhs(M: int, K: int, seed: int, fmt: str = "e4m3"):
    x = normal_with_outliers(np.random.Generator(np.random.PCG64(seed)), (M, K))
    codes, s = quantize_lhs(x, fmt)
    return codes, np.ascontiguousarray(s.T)


def make_rhs(N: int, K: int, seed, fmt: str = "e4m3"):
    x = normal_with_outliers(np.random.Generator(np.random.PCG64(seed)), (N, K))
    return quantize_rhs(x, fmt)


def make_dense(M: int, N: int, K: int, seed_a: int, seed_b: int, fmt_a: str = "e4m3",
               fmt_b: str = "e4m3") -> Dense:
    """Dense problem; the operand formats (e4m3 or e5m2, scale amax / format
    maximum) only change the encoding, the recipe is the same."""
    a, sa_t = make_lhs(M, K, seed_a, fmt_a)
    b, sb = make_rhs(N, K, seed_b, fmt_b)
    return Dense(M, N, K, a, sa_t, b, sb)


def make_grouped_rhs(G: int, N: int, K: int, seed: int, workers: int = 8):
    """Per-expert RHS, each expert from its own spawned seed (bounded host memory)."""
    seqs = np.random.SeedSequence(seed).spawn(G)
    b = np.empty((G, N, K), dtype=np.uint8)
    sb = np.empty((G, N // BLOCK, K // BLOCK), dtype=np.float32)

    def one(g):
        x = normal_with_outliers(np.random.Generator(np.random.PCG64(seqs[g])), (N, K))
        b[g], sb[g] = quantize_rhs(x)

    with ThreadPoolExecutor(max_workers=max(1, min(workers, G))) as ex:
        list(ex.map(one, range(G)))
    return b, sb


def route_contiguous(expert_of_token: np.ndarray, G: int):
    """Lay tokens out by expert (ascending), padding each segment to 128 rows.

    Returns ``(ids int32 [M_total], token_of_row int64 [M_total], counts)``.
    """
    counts = np.bincount(expert_of_token, minlength=G).astype(np.int64)
    padded = (counts + BLOCK - 1) // BLOCK * BLOCK
    M_total = int(padded.sum())
    ids = np.full(M_total, -1, dtype=np.int32)
    tok = np.full(M_total, -1, dtype=np.int64)
    row = 0
    for g in range(G):
        members = np.nonzero(expert_of_token == g)[0]
        ids[row:row + len(members)] = g
        tok[row:row + len(members)] = members
        row += int(padded[g])
    return ids, tok, counts


def make_contiguous(G: int, tokens: int, N: int, K: int,
                    seed_a: int, seed_b: int, seed_route: int,
                    expert_of_token: np.ndarray | None = None) -> Contiguous:
    if expert_of_token is None:
        rng = np.random.Generator(np.random.PCG64(seed_route))
        expert_of_token = rng.choice(G, size=tokens)  # uniform top-1 routing
    ids, tok, counts = route_contiguous(np.asarray(expert_of_token), G)
    M_total = ids.shape[0]
    xa, sa_tok = make_lhs(tokens, K, seed_a)  # sa_tok is M-major [K/128, tokens]
    a = np.zeros((M_total, K), dtype=np.uint8)
    sa_t = np.ones((K // BLOCK, M_total), dtype=np.float32)
    real = tok >= 0
    a[real] = xa[tok[real]]
    sa_t[:, real] = sa_tok[:, tok[real]]
    b, sb = make_grouped_rhs(G, N, K, seed_b)
    return Contiguous(G, N, K, M_total, a, sa_t, b, sb, ids, tok, counts)


def make_masked(G: int, M_max: int, N: int, K: int,
                seed_a: int, seed_b: int, seed_count: int,
                masked_m: np.ndarray | None = None) -> Masked:
    if masked_m is None:
        rng = np.random.Generator(np.random.PCG64(seed_count))
        masked_m = rng.integers(0, M_max + 1, size=G)  # inclusive Uniform{0..M_max}
    masked_m = np.asarray(masked_m, dtype=np.int32)
    a2, sa2 = make_lhs(G * M_max, K, seed_a)
    a = a2.reshape(G, M_max, K)
    # sa2 is [K/128, G*M_max]; per-group M-major [G, K/128, M_max]
    sa_t = np.ascontiguousarray(sa2.reshape(K // BLOCK, G, M_max).transpose(1, 0, 2))
    b, sb = make_grouped_rhs(G, N, K, seed_b)
    return Masked(G, M_max, N, K, a, sa_t, b, sb, masked_m)


# Workloads. Names carry the sizes; seeds are fixed per workload.
CONFIGS = {
    "dense_64x256x512": dict(kind="dense", M=64, N=256, K=512, seeds=(101, 102)),
    "decode_8x4096x7168": dict(kind="dense", M=8, N=4096, K=7168, seeds=(201, 202)),
    "square_4096": dict(kind="dense", M=4096, N=4096, K=4096, seeds=(301, 302)),
    "square_4096_e4m3xe5m2": dict(kind="dense", M=4096, N=4096, K=4096, seeds=(301, 302), fmt=("e4m3", "e5m2")),
    "prefill_8192x7168x2048": dict(kind="dense", M=8192, N=7168, K=2048, seeds=(311, 312)),
    "moe_contiguous_g8_t8192": dict(kind="contiguous", G=8, tokens=8192, N=4096, K=7168,
                                    seeds=(401, 402, 403)),
    # the same problem with the experts' segment offsets passed to the GEMM
    "moe_contiguous_g8_t8192_seg": dict(kind="contiguous", G=8, tokens=8192, N=4096, K=7168,
                                        seeds=(401, 402, 403), segments=True),
    "moe_masked_g32_m256": dict(kind="masked", G=32, M_max=256, N=4096, K=7168,
                                seeds=(501, 502, 504)),
}


# Activations for the 1x128 quantiser: the token activations of the MoE
# workloads (8192 tokens, hidden size 7168), fp32 or bf16.
QUANT_CONFIGS = {
    "quantize_f32_8192x7168": dict(M=8192, K=7168, dtype="f32", seed=701),
    "quantize_bf16_8192x7168": dict(M=8192, K=7168, dtype="bf16", seed=702),
}


def make_activations(name: str) -> np.ndarray:
    """fp32 activations of a quantiser workload (bf16 workloads round them)."""
    c = QUANT_CONFIGS[name]
    return normal_with_outliers(np.random.Generator(np.random.PCG64(c["seed"])), (c["M"], c["K"]))


def segment_layout(counts: np.ndarray) -> np.ndarray:
    """First row of each expert's segment (segments padded to 128), then the rows used."""
    padded = (np.asarray(counts, np.int64) + BLOCK - 1) // BLOCK * BLOCK
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)


def make_config(name: str):
    c = CONFIGS[name]
    if c["kind"] == "dense":
        return make_dense(c["M"], c["N"], c["K"], *c["seeds"], *c.get("fmt", ("e4m3", "e4m3")))
    if c["kind"] == "contiguous":
        return make_contiguous(c["G"], c["tokens"], c["N"], c["K"], *c["seeds"])
    return make_masked(c["G"], c["M_max"], c["N"], c["K"], *c["seeds"])
