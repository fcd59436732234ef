"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host (these calls return before any device
access, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from fp8_block_scaled_sa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg_fp8.h")

DG_OK, DG_ERR_NULL_POINTER, DG_ERR_BAD_SHAPE, DG_ERR_MISALIGNED = 0, 1, 2, 3
DG_ERR_BAD_STRIDE, DG_ERR_UNSUPPORTED, DG_ERR_HIP, DG_ERR_ALIASING = 4, 5, 6, 7


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|dg_status|const char \*)\s*(dg_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("dg_fp8_gemm_nt", "dg_fp8_grouped_gemm_contiguous", "dg_fp8_grouped_gemm_masked",
                 "dg_fp8_quantize_1x128", "dg_fp8_gemm_nt_ws", "dg_fp8_gemm_nt_workspace_bytes",
                 "dg_fp8_grouped_gemm_contiguous_ws", "dg_fp8_grouped_gemm_contiguous_workspace_bytes",
                 "dg_abi_version", "dg_status_string", "dg_last_hip_error"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.path())
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.SIGNATURES)


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.dg_abi_version() == 2
    for s in range(8):
        assert lib.dg_status_string(s)
    assert lib.dg_status_string(99) == b"unknown status"
    assert lib.dg_last_hip_error() == 0


# Fake, never-dereferenced, 256-byte aligned addresses that do not overlap.
A, SA, B, SB, D, IDS = (0x10000000 * (i + 1) for i in range(6))


def nt(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=64, B=B, ldb=512, sB=SB, sb_nb=4, sb_kb=1,
                D=D, ldd=256, M=64, N=256, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_gemm_nt(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(K=500, lda=512, ldb=512), DG_ERR_BAD_SHAPE),
    (dict(K=0), DG_ERR_BAD_SHAPE),
    (dict(N=200), DG_ERR_BAD_SHAPE),
    (dict(M=-1), DG_ERR_BAD_SHAPE),
    (dict(A=None), DG_ERR_NULL_POINTER),
    (dict(sB=None), DG_ERR_NULL_POINTER),
    (dict(D=None), DG_ERR_NULL_POINTER),
    (dict(lda=256), DG_ERR_BAD_STRIDE),
    (dict(ldb=384), DG_ERR_BAD_STRIDE),
    (dict(ldd=128), DG_ERR_BAD_STRIDE),
    (dict(sa_m=-1), DG_ERR_BAD_STRIDE),
    (dict(A=A + 8), DG_ERR_MISALIGNED),
    (dict(D=D + 2), DG_ERR_MISALIGNED),
    (dict(lda=520), DG_ERR_MISALIGNED),
    (dict(ldd=260), DG_ERR_MISALIGNED),
    (dict(sA=SA + 2), DG_ERR_MISALIGNED),
    (dict(D=A + 1024), DG_ERR_ALIASING),
    (dict(D=SB), DG_ERR_ALIASING),
    (dict(M=2 ** 31), DG_ERR_UNSUPPORTED),
])
def test_dense_validation(kw, status):
    assert nt(**kw) == status


def test_empty_problems_return_ok_without_device():
    assert nt(M=0) == DG_OK
    assert nt(N=0) == DG_OK
    assert nt(M=0, A=None, B=None, D=None) == DG_OK


WS = 0x70000000


def nt_ws(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=64, B=B, ldb=512, sB=SB, sb_nb=4, sb_kb=1,
                D=D, ldd=256, M=64, N=256, K=512, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_gemm_nt_ws(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(K=500, lda=512, ldb=512), DG_ERR_BAD_SHAPE),
    (dict(A=None), DG_ERR_NULL_POINTER),
    (dict(ws_bytes=-1), DG_ERR_BAD_SHAPE),
    (dict(ws=WS + 8), DG_ERR_MISALIGNED),
    (dict(ws=D), DG_ERR_ALIASING),                  # the workspace overlaps the output
    (dict(ws=D - 4096, ws_bytes=8192), DG_ERR_ALIASING),
    (dict(ws=A), DG_ERR_ALIASING),                  # ... or an input
    (dict(ws=SB - 1024, ws_bytes=2048), DG_ERR_ALIASING),
    (dict(D=A + 1024), DG_ERR_ALIASING),
])
def test_dense_ws_validation(kw, status):
    assert nt_ws(**kw) == status


def test_dense_ws_empty_and_unused_workspace():
    assert nt_ws(M=0) == DG_OK
    # a NULL workspace (or zero bytes) is the plain call: nothing to check about it
    assert nt_ws(M=0, ws=None, ws_bytes=0) == DG_OK
    assert nt_ws(M=0, ws=WS + 8, ws_bytes=0) == DG_OK


def test_workspace_queries_reject_bad_shapes_on_the_host():
    lib = _lib.load()
    assert lib.dg_fp8_gemm_nt_workspace_bytes(64, 200, 512) == -DG_ERR_BAD_SHAPE
    assert lib.dg_fp8_gemm_nt_workspace_bytes(64, 256, 500) == -DG_ERR_BAD_SHAPE
    assert lib.dg_fp8_gemm_nt_workspace_bytes(-1, 256, 512) == -DG_ERR_BAD_SHAPE
    assert lib.dg_fp8_gemm_nt_workspace_bytes(0, 256, 512) == 0
    assert lib.dg_fp8_grouped_gemm_contiguous_workspace_bytes(200, 256, 512, 4) == -DG_ERR_BAD_SHAPE
    assert lib.dg_fp8_grouped_gemm_contiguous_workspace_bytes(256, 256, 512, -1) == -DG_ERR_BAD_SHAPE
    assert lib.dg_fp8_grouped_gemm_contiguous_workspace_bytes(0, 256, 512, 4) == 0
    assert lib.dg_fp8_grouped_gemm_contiguous_workspace_bytes(256, 256, 512, 0) == 0


def contig_ws(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=256, B=B, ldb=512, b_stride_g=256 * 512,
                sB=SB, sb_g=8, sb_nb=4, sb_kb=1, ids=IDS, tok=None, layout=None, D=D, ldd=256, T=0,
                M_total=256, N=256, K=512, G=4, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_contiguous_ws(*args.values())


TOK, LAYOUT = 0x80000000, 0x90000000


@pytest.mark.parametrize("kw,status", [
    (dict(M_total=200), DG_ERR_BAD_SHAPE),
    (dict(ids=None), DG_ERR_NULL_POINTER),
    (dict(ws_bytes=-5), DG_ERR_BAD_SHAPE),
    (dict(ws=WS + 4), DG_ERR_MISALIGNED),
    (dict(ws=D + 1024), DG_ERR_ALIASING),
    (dict(ws=IDS), DG_ERR_ALIASING),
    (dict(ws=TOK, tok=TOK, T=100), DG_ERR_ALIASING),
    (dict(ws=LAYOUT - 256, ws_bytes=512, layout=LAYOUT), DG_ERR_ALIASING),
    (dict(tok=TOK + 2, T=100), DG_ERR_MISALIGNED),
])
def test_contiguous_ws_validation(kw, status):
    assert contig_ws(**kw) == status


def test_contiguous_ws_empty():
    assert contig_ws(M_total=0) == DG_OK
    assert contig_ws(G=0) == DG_OK
    assert contig_ws(tok=TOK, T=0) == DG_OK     # token-order output with no rows


def contig(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=256, B=B, ldb=512, b_stride_g=256 * 512,
                sB=SB, sb_g=8, sb_nb=4, sb_kb=1, ids=IDS, D=D, ldd=256,
                M_total=256, N=256, K=512, G=4, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_contiguous(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(M_total=200), DG_ERR_BAD_SHAPE),
    (dict(G=-1), DG_ERR_BAD_SHAPE),
    (dict(ids=None), DG_ERR_NULL_POINTER),
    (dict(b_stride_g=1024), DG_ERR_BAD_STRIDE),
    (dict(b_stride_g=256 * 512 + 8), DG_ERR_MISALIGNED),
    (dict(ids=IDS + 2), DG_ERR_MISALIGNED),
    (dict(D=IDS), DG_ERR_ALIASING),
])
def test_contiguous_validation(kw, status):
    assert contig(**kw) == status


def test_contiguous_empty():
    assert contig(M_total=0) == DG_OK
    assert contig(G=0) == DG_OK


def masked(**kw):
    args = dict(A=A, lda=512, a_stride_g=64 * 512, sA=SA, sa_g=256, sa_m=1, sa_kb=64,
                B=B, ldb=512, b_stride_g=256 * 512, sB=SB, sb_g=8, sb_nb=4, sb_kb=1,
                masked_m=IDS, D=D, ldd=256, d_stride_g=64 * 256,
                G=4, M_max=64, N=256, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_masked(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), DG_ERR_BAD_SHAPE),
    (dict(masked_m=None), DG_ERR_NULL_POINTER),
    (dict(a_stride_g=512), DG_ERR_BAD_STRIDE),
    (dict(d_stride_g=256), DG_ERR_BAD_STRIDE),
    (dict(d_stride_g=64 * 256 + 4), DG_ERR_MISALIGNED),
    (dict(D=B + 4096), DG_ERR_ALIASING),
])
def test_masked_validation(kw, status):
    assert masked(**kw) == status


def test_masked_empty():
    assert masked(G=0) == DG_OK
    assert masked(M_max=0) == DG_OK


X, Q, S = A, B, SB


def quant(**kw):
    args = dict(X=X, x_dtype=0, ldx=512, Q=Q, ldq=512, S=S, s_m=1, s_kb=64, M=64, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_quantize_1x128(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(K=500, ldx=512, ldq=512), DG_ERR_BAD_SHAPE),
    (dict(K=0), DG_ERR_BAD_SHAPE),
    (dict(M=-1), DG_ERR_BAD_SHAPE),
    (dict(x_dtype=2), DG_ERR_UNSUPPORTED),
    (dict(M=2 ** 31), DG_ERR_UNSUPPORTED),
    (dict(X=None), DG_ERR_NULL_POINTER),
    (dict(Q=None), DG_ERR_NULL_POINTER),
    (dict(S=None), DG_ERR_NULL_POINTER),
    (dict(ldx=256), DG_ERR_BAD_STRIDE),
    (dict(ldq=384), DG_ERR_BAD_STRIDE),
    (dict(s_m=-1), DG_ERR_BAD_STRIDE),
    (dict(s_m=0), DG_ERR_BAD_STRIDE),          # rows would share a scale slot
    (dict(s_m=1, s_kb=32), DG_ERR_BAD_STRIDE),  # M-major with a stride shorter than M
    (dict(s_m=3, s_kb=1), DG_ERR_BAD_STRIDE),   # row-major with a stride shorter than K/128
    (dict(X=X + 8), DG_ERR_MISALIGNED),
    (dict(Q=Q + 4), DG_ERR_MISALIGNED),
    (dict(ldx=514), DG_ERR_MISALIGNED),
    (dict(x_dtype=1, ldx=516), DG_ERR_MISALIGNED),
    (dict(ldq=520), DG_ERR_MISALIGNED),
    (dict(S=S + 2), DG_ERR_MISALIGNED),
    (dict(Q=X + 4096), DG_ERR_ALIASING),
    (dict(S=X + 256), DG_ERR_ALIASING),
    (dict(S=Q + 1024), DG_ERR_ALIASING),
])
def test_quantize_validation(kw, status):
    assert quant(**kw) == status


def test_quantize_accepts_both_scale_layouts_up_to_the_device_check():
    # Valid arguments get past validation: on a machine without a GPU the call
    # then fails at the device query, never with an argument error.
    for kw in (dict(s_m=1, s_kb=64), dict(s_m=4, s_kb=1), dict(x_dtype=1, ldx=520)):
        assert quant(**kw) in (DG_OK, DG_ERR_HIP, DG_ERR_UNSUPPORTED)


def test_quantize_empty():
    assert quant(M=0) == DG_OK
    assert quant(M=0, X=None, Q=None, S=None) == DG_OK


def gather(**kw):
    args = dict(X=X, x_dtype=1, ldx=512, x_rows=100, src=IDS, Q=Q, ldq=512, S=S, s_m=1, s_kb=64,
                M=64, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_quantize_1x128_gather(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), DG_ERR_NULL_POINTER),
    (dict(src=IDS + 2), DG_ERR_MISALIGNED),
    (dict(x_rows=-1), DG_ERR_BAD_SHAPE),
    (dict(src=Q + 64), DG_ERR_ALIASING),
    (dict(K=100), DG_ERR_BAD_SHAPE),
    (dict(X=None), DG_ERR_NULL_POINTER),
])
def test_gather_quantize_validation(kw, status):
    assert gather(**kw) == status


def test_gather_quantize_all_padding_needs_no_input():
    assert gather(X=None, x_rows=0) in (DG_OK, DG_ERR_HIP, DG_ERR_UNSUPPORTED)
    assert gather(M=0, src=None) == DG_OK


E, ROW, EIDS, TOK, LAY = (0x10000000 * (i + 10) for i in range(5))


def route(**kw):
    args = dict(e=E, T=1000, G=8, row=ROW, ids=EIDS, tok=TOK, layout=LAY, M_cap=2048, stream=None)
    args.update(kw)
    return _lib.load().dg_moe_route_contiguous(*args.values())


def test_max_rows():
    lib = _lib.load()
    assert lib.dg_moe_contiguous_max_rows(8192, 8) == 128 * 72
    assert lib.dg_moe_contiguous_max_rows(5, 100) == 128 * 6
    assert lib.dg_moe_contiguous_max_rows(0, 4) == 0
    assert lib.dg_moe_contiguous_max_rows(-1, 4) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(G=0), DG_ERR_BAD_SHAPE),
    (dict(T=-1), DG_ERR_BAD_SHAPE),
    (dict(M_cap=2000), DG_ERR_BAD_SHAPE),           # not a multiple of 128
    (dict(M_cap=1024), DG_ERR_BAD_SHAPE),           # below 128 * (ceil(T/128) + min(G, T)) = 2048
    (dict(G=1025, M_cap=128 * 1008), DG_ERR_UNSUPPORTED),
    (dict(e=None), DG_ERR_NULL_POINTER),
    (dict(layout=None), DG_ERR_NULL_POINTER),
    (dict(ids=EIDS + 2), DG_ERR_MISALIGNED),
    (dict(tok=EIDS + 1024), DG_ERR_ALIASING),
    (dict(row=E), DG_ERR_ALIASING),
])
def test_route_validation(kw, status):
    assert route(**kw) == status


def unperm(**kw):
    args = dict(D=D, ldd=256, d_rows=512, row=IDS, T=300, N=256, out=A, ldo=256, stream=None)
    args.update(kw)
    return _lib.load().dg_moe_unpermute(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(N=100), DG_ERR_BAD_SHAPE),
    (dict(row=None), DG_ERR_NULL_POINTER),
    (dict(ldo=128), DG_ERR_BAD_STRIDE),
    (dict(ldd=260), DG_ERR_MISALIGNED),
    (dict(out=A + 8), DG_ERR_MISALIGNED),
    (dict(out=D + 1024), DG_ERR_ALIASING),
])
def test_unpermute_validation(kw, status):
    assert unperm(**kw) == status


def test_unpermute_empty():
    assert unperm(T=0) == DG_OK


def nt_fmt(a_fmt=1, b_fmt=0, **kw):
    args = dict(A=A, a_fmt=a_fmt, lda=512, sA=SA, sa_m=1, sa_kb=64, B=B, b_fmt=b_fmt, ldb=512, sB=SB, sb_nb=4,
                sb_kb=1, D=D, ldd=256, M=64, N=256, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_gemm_nt_fmt(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(a_fmt=2), DG_ERR_UNSUPPORTED),
    (dict(b_fmt=-1), DG_ERR_UNSUPPORTED),
    (dict(K=500, lda=512, ldb=512), DG_ERR_BAD_SHAPE),
    (dict(A=None), DG_ERR_NULL_POINTER),
    (dict(lda=256), DG_ERR_BAD_STRIDE),
    (dict(D=D + 2), DG_ERR_MISALIGNED),
    (dict(D=SB), DG_ERR_ALIASING),
    (dict(a_fmt=0, b_fmt=0, D=SB), DG_ERR_ALIASING),     # e4m3 x e4m3 goes through dg_fp8_gemm_nt
])
def test_fmt_validation(kw, status):
    assert nt_fmt(**kw) == status


def test_fmt_empty():
    assert nt_fmt(M=0) == DG_OK and nt_fmt(a_fmt=1, b_fmt=1, N=0) == DG_OK


def contig_tokens(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=256, B=B, ldb=512, b_stride_g=256 * 512,
                sB=SB, sb_g=8, sb_nb=4, sb_kb=1, ids=IDS, tok=E, layout=None, out=D, ldo=256, T=200,
                M_total=256, N=256, K=512, G=4, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_contiguous_to_tokens(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(tok=None), DG_ERR_NULL_POINTER),
    (dict(tok=E + 2), DG_ERR_MISALIGNED),
    (dict(T=-1), DG_ERR_BAD_SHAPE),
    (dict(M_total=200), DG_ERR_BAD_SHAPE),
    (dict(out=E), DG_ERR_ALIASING),
    (dict(ldo=128), DG_ERR_BAD_STRIDE),
])
def test_contiguous_to_tokens_validation(kw, status):
    assert contig_tokens(**kw) == status


def test_contiguous_to_tokens_empty():
    assert contig_tokens(T=0) == DG_OK and contig_tokens(M_total=0, tok=None) == DG_OK


def contig_fmt(a_fmt=1, b_fmt=1, **kw):
    args = dict(A=A, a_fmt=a_fmt, lda=512, sA=SA, sa_m=1, sa_kb=256, B=B, b_fmt=b_fmt, ldb=512,
                b_stride_g=256 * 512, sB=SB, sb_g=8, sb_nb=4, sb_kb=1, ids=IDS, D=D, ldd=256,
                M_total=256, N=256, K=512, G=4, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_contiguous_fmt(*args.values())


def masked_fmt(a_fmt=1, b_fmt=0, **kw):
    args = dict(A=A, a_fmt=a_fmt, lda=512, a_stride_g=64 * 512, sA=SA, sa_g=256, sa_m=1, sa_kb=64,
                B=B, b_fmt=b_fmt, ldb=512, b_stride_g=256 * 512, sB=SB, sb_g=8, sb_nb=4, sb_kb=1,
                masked_m=IDS, D=D, ldd=256, d_stride_g=64 * 256, G=4, M_max=64, N=256, K=512, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_masked_fmt(*args.values())


@pytest.mark.parametrize("fn,kw,status", [
    (contig_fmt, dict(a_fmt=3), DG_ERR_UNSUPPORTED),
    (contig_fmt, dict(M_total=200), DG_ERR_BAD_SHAPE),
    (contig_fmt, dict(ids=None), DG_ERR_NULL_POINTER),
    (contig_fmt, dict(D=IDS), DG_ERR_ALIASING),
    (masked_fmt, dict(b_fmt=7), DG_ERR_UNSUPPORTED),
    (masked_fmt, dict(masked_m=None), DG_ERR_NULL_POINTER),
    (masked_fmt, dict(d_stride_g=256), DG_ERR_BAD_STRIDE),
    (masked_fmt, dict(D=B + 4096), DG_ERR_ALIASING),
])
def test_grouped_fmt_validation(fn, kw, status):
    assert fn(**kw) == status


def test_grouped_fmt_empty():
    assert contig_fmt(M_total=0) == DG_OK and masked_fmt(G=0) == DG_OK


def contig_layout(**kw):
    args = dict(A=A, lda=512, sA=SA, sa_m=1, sa_kb=256, B=B, ldb=512, b_stride_g=256 * 512,
                sB=SB, sb_g=8, sb_nb=4, sb_kb=1, ids=IDS, layout=LAY, D=D, ldd=256,
                M_total=256, N=256, K=512, G=4, stream=None)
    args.update(kw)
    return _lib.load().dg_fp8_grouped_gemm_contiguous_layout(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(layout=None), DG_ERR_NULL_POINTER),
    (dict(layout=LAY + 2), DG_ERR_MISALIGNED),
    (dict(G=1025), DG_ERR_UNSUPPORTED),
    (dict(D=LAY - 64), DG_ERR_ALIASING),
    (dict(M_total=200), DG_ERR_BAD_SHAPE),
])
def test_contiguous_layout_validation(kw, status):
    assert contig_layout(**kw) == status


def test_contiguous_layout_empty():
    assert contig_layout(M_total=0, layout=None) == DG_OK
