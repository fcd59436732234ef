"""Python binding of the C ABI (include/dg_fp8.h), same names, torch tensors in.

Argument marshalling only: every step of the GEMM runs in the HIP library.
Operands are CUDA (HIP) tensors: e4m3 codes as ``torch.uint8`` or
``torch.float8_e4m3fn``, scales ``torch.float32`` (any strides, read through
the logical index), routing arrays ``torch.int32``, output ``torch.bfloat16``.
The call is enqueued on torch's current stream unless ``stream`` is given.
"""
from __future__ import annotations

import torch

from . import _lib

BLOCK = 128


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.dg_status_string(status).decode()
        if status == 6:  # DG_ERR_HIP
            msg += " (hipError %d)" % lib.dg_last_hip_error()
        super().__init__("%s: status %d: %s" % (where, status, msg))
        self.status = status


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    return t.data_ptr()


def _codes(t: torch.Tensor, name: str, ndim: int) -> torch.Tensor:
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("%s must hold e4m3 codes (uint8 or float8_e4m3fn)" % name)
    if t.dim() != ndim or t.stride(-1) != 1:
        raise ValueError("%s must be %d-D with a contiguous last (K) dimension" % (name, ndim))
    return t


def _scales(t: torch.Tensor, name: str, ndim: int) -> torch.Tensor:
    if t.dtype != torch.float32 or t.dim() != ndim:
        raise TypeError("%s must be a %d-D float32 tensor" % (name, ndim))
    return t


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise DGError(status, where)


def dg_fp8_gemm_nt(a, sa, b, sb, d=None, stream=None):
    """D[M,N] (bf16) from A[M,K], sA[M,K/128], B[N,K], sB[N/128,K/128]."""
    _codes(a, "a", 2), _codes(b, "b", 2), _scales(sa, "sa", 2), _scales(sb, "sb", 2)
    M, K = a.shape
    N = b.shape[0]
    if d is None:
        d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1:
        raise TypeError("d must be a 2-D bfloat16 tensor with contiguous rows")
    if b.shape[1] != K or tuple(d.shape) != (M, N):
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (M, K // BLOCK) or tuple(sb.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_gemm_nt(_dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
                            _dev(b, "b"), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1),
                            _dev(d, "d"), d.stride(0), M, N, K, _stream(stream))
    _check(st, "dg_fp8_gemm_nt")
    return d


def _ws(workspace):
    """(pointer, bytes) of a caller workspace: a device tensor or None."""
    if workspace is None or workspace.numel() == 0:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _query(n: int, where: str) -> int:
    if n < 0:
        raise DGError(-n, where)
    return int(n)


def dg_fp8_gemm_nt_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes the fastest path of dg_fp8_gemm_nt_ws takes (0: none)."""
    return _query(_lib.load().dg_fp8_gemm_nt_workspace_bytes(M, N, K), "dg_fp8_gemm_nt_workspace_bytes")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A caller-owned workspace tensor of at least nbytes bytes (torch allocates it)."""
    return torch.empty(max(int(nbytes), 0), dtype=torch.uint8, device=device)


def dg_fp8_gemm_nt_ws(a, sa, b, sb, workspace, d=None, stream=None):
    """dg_fp8_gemm_nt with a caller workspace (a uint8 device tensor, or None)
    for its split-K path."""
    _codes(a, "a", 2), _codes(b, "b", 2), _scales(sa, "sa", 2), _scales(sb, "sb", 2)
    M, K = a.shape
    N = b.shape[0]
    if d is None:
        d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1:
        raise TypeError("d must be a 2-D bfloat16 tensor with contiguous rows")
    if b.shape[1] != K or tuple(d.shape) != (M, N):
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (M, K // BLOCK) or tuple(sb.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    wp, wb = _ws(workspace)
    lib = _lib.load()
    st = lib.dg_fp8_gemm_nt_ws(_dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
                               _dev(b, "b"), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1),
                               _dev(d, "d"), d.stride(0), M, N, K, wp, wb, _stream(stream))
    _check(st, "dg_fp8_gemm_nt_ws")
    return d


def dg_fp8_gemm_nt_noalloc(a, sa, b, sb, d, stream=None):
    """dg_fp8_gemm_nt_ws with the library's static scratch array as the
    workspace: allocates nothing (d must be given)."""
    _codes(a, "a", 2), _codes(b, "b", 2), _scales(sa, "sa", 2), _scales(sb, "sb", 2)
    M, K = a.shape
    N = b.shape[0]
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1 or tuple(d.shape) != (M, N):
        raise TypeError("d must be a bfloat16 [M, N] tensor with contiguous rows")
    if b.shape[1] != K:
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (M, K // BLOCK) or tuple(sb.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    st = _lib.load().dg_fp8_gemm_nt_noalloc(_dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
                                            _dev(b, "b"), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1),
                                            _dev(d, "d"), d.stride(0), M, N, K, _stream(stream))
    _check(st, "dg_fp8_gemm_nt_noalloc")
    return d


FORMATS = {"e4m3": 0, "e5m2": 1}   # DG_FP8_E4M3, DG_FP8_E5M2


def dg_fp8_gemm_nt_fmt(a, sa, b, sb, a_fmt="e4m3", b_fmt="e4m3", d=None, stream=None):
    """dg_fp8_gemm_nt with a per-operand fp8 format ("e4m3" or "e5m2"). Codes
    are uint8 (or the matching torch float8 dtype)."""
    for t, name in ((a, "a"), (b, "b")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2) or t.dim() != 2 or t.stride(-1) != 1:
            raise TypeError("%s must be a 2-D fp8 code tensor with a contiguous last (K) dimension" % name)
    _scales(sa, "sa", 2), _scales(sb, "sb", 2)
    M, K = a.shape
    N = b.shape[0]
    if d is None:
        d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1:
        raise TypeError("d must be a 2-D bfloat16 tensor with contiguous rows")
    if b.shape[1] != K or tuple(d.shape) != (M, N):
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (M, K // BLOCK) or tuple(sb.shape) != (N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_gemm_nt_fmt(_dev(a, "a"), FORMATS[a_fmt], a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
                                _dev(b, "b"), FORMATS[b_fmt], b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1),
                                _dev(d, "d"), d.stride(0), M, N, K, _stream(stream))
    _check(st, "dg_fp8_gemm_nt_fmt")
    return d


def dg_fp8_grouped_gemm_contiguous(a, sa, b, sb, expert_ids, d=None, stream=None):
    """Contiguous MoE layout: A[M_total,K], sA[M_total,K/128], B[G,N,K],
    sB[G,N/128,K/128], expert_ids[M_total] int32 -> D[M_total,N]; rows whose
    id is not in [0, G) are not written."""
    _codes(a, "a", 2), _codes(b, "b", 3), _scales(sa, "sa", 2), _scales(sb, "sb", 3)
    if expert_ids.dtype != torch.int32 or expert_ids.dim() != 1 or expert_ids.stride(0) != 1:
        raise TypeError("expert_ids must be a contiguous 1-D int32 tensor")
    M_total, K = a.shape
    G, N, _ = b.shape
    if d is None:
        d = torch.empty((M_total, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1:
        raise TypeError("d must be a 2-D bfloat16 tensor with contiguous rows")
    if b.shape[2] != K or tuple(d.shape) != (M_total, N) or expert_ids.shape[0] != M_total:
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (M_total, K // BLOCK) or tuple(sb.shape) != (G, N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_contiguous(
        _dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        _dev(b, "b"), b.stride(1), b.stride(0),
        _dev(sb, "sb"), sb.stride(0), sb.stride(1), sb.stride(2),
        _dev(expert_ids, "expert_ids"), _dev(d, "d"), d.stride(0),
        M_total, N, K, G, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_contiguous")
    return d


def dg_fp8_grouped_gemm_contiguous_to_tokens(a, sa, b, sb, expert_ids, token_of_row, T, layout=None, out=None,
                                             stream=None):
    """The contiguous grouped GEMM with row r of the result written to
    out[token_of_row[r]] (out [T, N] bf16; rows of dropped tokens untouched).
    With the routing's segment offsets `layout` [G+1] the tiles follow the
    experts' segments."""
    _codes(a, "a", 2), _codes(b, "b", 3), _scales(sa, "sa", 2), _scales(sb, "sb", 3)
    M_total, K = a.shape
    G, N, _ = b.shape
    for t, name in ((expert_ids, "expert_ids"), (token_of_row, "token_of_row")):
        if t.dtype != torch.int32 or tuple(t.shape) != (M_total,):
            raise ValueError("%s must be int32 [M_total]" % name)
    if layout is not None and (layout.dtype != torch.int32 or tuple(layout.shape) != (G + 1,)):
        raise ValueError("layout must be int32 [G+1]")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (T, N) or out.stride(-1) != 1:
        raise ValueError("out must be a bfloat16 [T, N] tensor with contiguous rows")
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_contiguous_to_tokens(
        _dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        _dev(b, "b"), b.stride(1), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1), sb.stride(2),
        _dev(expert_ids, "expert_ids"), _dev(token_of_row, "token_of_row"),
        None if layout is None else _dev(layout, "layout"), _dev(out, "out"), out.stride(0), T,
        M_total, N, K, G, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_contiguous_to_tokens")
    return out


def dg_fp8_grouped_gemm_contiguous_layout(a, sa, b, sb, expert_ids, layout, d=None, stream=None):
    """The contiguous grouped GEMM with the experts' segment offsets
    (layout [G+1] int32): tiles follow the segments."""
    _codes(a, "a", 2), _codes(b, "b", 3), _scales(sa, "sa", 2), _scales(sb, "sb", 3)
    M_total, K = a.shape
    G, N, _ = b.shape
    if layout.dtype != torch.int32 or tuple(layout.shape) != (G + 1,):
        raise ValueError("layout must be int32 [G+1]")
    if d is None:
        d = torch.empty((M_total, N), dtype=torch.bfloat16, device=a.device)
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_contiguous_layout(
        _dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        _dev(b, "b"), b.stride(1), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1), sb.stride(2),
        _dev(expert_ids, "expert_ids"), _dev(layout, "layout"), _dev(d, "d"), d.stride(0),
        M_total, N, K, G, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_contiguous_layout")
    return d


def dg_fp8_grouped_gemm_contiguous_workspace_bytes(M_total: int, N: int, K: int, G: int) -> int:
    """Workspace bytes the fastest path of dg_fp8_grouped_gemm_contiguous_ws takes (0: none)."""
    return _query(_lib.load().dg_fp8_grouped_gemm_contiguous_workspace_bytes(M_total, N, K, G),
                  "dg_fp8_grouped_gemm_contiguous_workspace_bytes")


def dg_fp8_grouped_gemm_contiguous_ws(a, sa, b, sb, expert_ids, workspace, token_of_row=None, T=None, layout=None,
                                      d=None, stream=None):
    """The contiguous grouped GEMM with a caller workspace (uint8 device
    tensor or None): segment offsets derived on the device when no layout is
    given, the segments' last 128 rows split over K. With token_of_row the
    rows go to d [T, N] in token order, else to d [M_total, N]."""
    _codes(a, "a", 2), _codes(b, "b", 3), _scales(sa, "sa", 2), _scales(sb, "sb", 3)
    M_total, K = a.shape
    G, N, _ = b.shape
    if expert_ids.dtype != torch.int32 or tuple(expert_ids.shape) != (M_total,) or expert_ids.stride(0) != 1:
        raise ValueError("expert_ids must be a contiguous int32 [M_total] tensor")
    if token_of_row is not None:
        if token_of_row.dtype != torch.int32 or tuple(token_of_row.shape) != (M_total,):
            raise ValueError("token_of_row must be int32 [M_total]")
        if T is None:
            raise ValueError("T (rows of the token-order output) is needed with token_of_row")
    rows = M_total if token_of_row is None else T
    if layout is not None and (layout.dtype != torch.int32 or tuple(layout.shape) != (G + 1,)):
        raise ValueError("layout must be int32 [G+1]")
    if tuple(sa.shape) != (M_total, K // BLOCK) or tuple(sb.shape) != (G, N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    if d is None:
        d = torch.empty((rows, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or tuple(d.shape) != (rows, N) or d.stride(-1) != 1:
        raise ValueError("d must be a bfloat16 [%d, N] tensor with contiguous rows" % rows)
    wp, wb = _ws(workspace)
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_contiguous_ws(
        _dev(a, "a"), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        _dev(b, "b"), b.stride(1), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1), sb.stride(2),
        _dev(expert_ids, "expert_ids"), None if token_of_row is None else _dev(token_of_row, "token_of_row"),
        None if layout is None else _dev(layout, "layout"), _dev(d, "d"), d.stride(0), rows,
        M_total, N, K, G, wp, wb, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_contiguous_ws")
    return d


def dg_fp8_grouped_gemm_masked(a, sa, b, sb, masked_m, d=None, stream=None):
    """Masked MoE layout: A[G,M_max,K], sA[G,M_max,K/128], B[G,N,K],
    sB[G,N/128,K/128], masked_m[G] int32 -> D[G,M_max,N]; group g writes rows
    m < clamp(masked_m[g], 0, M_max) only."""
    _codes(a, "a", 3), _codes(b, "b", 3), _scales(sa, "sa", 3), _scales(sb, "sb", 3)
    if masked_m.dtype != torch.int32 or masked_m.dim() != 1 or masked_m.stride(0) != 1:
        raise TypeError("masked_m must be a contiguous 1-D int32 tensor")
    G, M_max, K = a.shape
    N = b.shape[1]
    if d is None:
        d = torch.empty((G, M_max, N), dtype=torch.bfloat16, device=a.device)
    if d.dtype != torch.bfloat16 or d.dim() != 3 or d.stride(-1) != 1:
        raise TypeError("d must be a 3-D bfloat16 tensor with contiguous rows")
    if (b.shape[0] != G or b.shape[2] != K or tuple(d.shape) != (G, M_max, N)
            or masked_m.shape[0] != G):
        raise ValueError("shape mismatch")
    if tuple(sa.shape) != (G, M_max, K // BLOCK) or tuple(sb.shape) != (G, N // BLOCK, K // BLOCK):
        raise ValueError("scale shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_masked(
        _dev(a, "a"), a.stride(1), a.stride(0),
        _dev(sa, "sa"), sa.stride(0), sa.stride(1), sa.stride(2),
        _dev(b, "b"), b.stride(1), b.stride(0),
        _dev(sb, "sb"), sb.stride(0), sb.stride(1), sb.stride(2),
        _dev(masked_m, "masked_m"), _dev(d, "d"), d.stride(1), d.stride(0),
        G, M_max, N, K, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_masked")
    return d


DTYPES = {torch.float32: 0, torch.bfloat16: 1}   # DG_DTYPE_F32, DG_DTYPE_BF16


def dg_fp8_quantize_1x128(x, q=None, s=None, stream=None):
    """Codes Q[M,K] (uint8 e4m3) and scales S[M,K/128] (fp32) of activations
    x[M,K] (float32 or bfloat16), one scale per 1x128 block. A new S is
    M-major (stored [K/128, M], returned as its transposed view), the layout
    the GEMM calls read fastest. Returns (q, s)."""
    if x.dtype not in DTYPES:
        raise TypeError("x must be float32 or bfloat16")
    if x.dim() != 2 or x.stride(-1) != 1:
        raise ValueError("x must be 2-D with a contiguous last (K) dimension")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // BLOCK, M), dtype=torch.float32, device=x.device).t()
    _codes(q, "q", 2), _scales(s, "s", 2)
    if tuple(q.shape) != (M, K) or tuple(s.shape) != (M, K // BLOCK):
        raise ValueError("shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_quantize_1x128(_dev(x, "x"), DTYPES[x.dtype], x.stride(0), _dev(q, "q"), q.stride(0),
                                   _dev(s, "s"), s.stride(0), s.stride(1), M, K, _stream(stream))
    _check(st, "dg_fp8_quantize_1x128")
    return q, s


def _dev_or_null(t, name):
    return None if t is None or t.numel() == 0 else _dev(t, name)


def dg_fp8_quantize_1x128_gather(x, src_rows, q=None, s=None, stream=None):
    """Quantise rows x[src_rows[r]] into Q[r] (a source index outside
    [0, x.shape[0]) gives a zero row: codes 0, scale 1). Returns (q, s) with
    s M-major as in dg_fp8_quantize_1x128."""
    if x.dtype not in DTYPES:
        raise TypeError("x must be float32 or bfloat16")
    if x.dim() != 2 or x.stride(-1) != 1:
        raise ValueError("x must be 2-D with a contiguous last (K) dimension")
    if src_rows.dtype != torch.int32 or src_rows.dim() != 1:
        raise TypeError("src_rows must be a 1-D int32 tensor")
    M, K = src_rows.shape[0], x.shape[1]
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((K // BLOCK, M), dtype=torch.float32, device=x.device).t()
    _codes(q, "q", 2), _scales(s, "s", 2)
    if tuple(q.shape) != (M, K) or tuple(s.shape) != (M, K // BLOCK):
        raise ValueError("shape mismatch")
    lib = _lib.load()
    st = lib.dg_fp8_quantize_1x128_gather(_dev_or_null(x, "x"), DTYPES[x.dtype], x.stride(0), x.shape[0],
                                          _dev_or_null(src_rows, "src_rows"), _dev(q, "q"), q.stride(0),
                                          _dev(s, "s"), s.stride(0), s.stride(1), M, K, _stream(stream))
    _check(st, "dg_fp8_quantize_1x128_gather")
    return q, s


def dg_moe_contiguous_max_rows(T: int, G: int) -> int:
    return int(_lib.load().dg_moe_contiguous_max_rows(T, G))


def dg_moe_route_contiguous(expert_of_token, G, M_cap=None, stream=None):
    """Routing of top-1 tokens into the contiguous layout. Returns
    (row_of_token [T], expert_ids [M_cap], token_of_row [M_cap], layout [G+1]),
    all int32 device tensors; M_cap defaults to the worst case."""
    if expert_of_token.dtype != torch.int32 or expert_of_token.dim() != 1:
        raise TypeError("expert_of_token must be a 1-D int32 tensor")
    T = expert_of_token.shape[0]
    dev = expert_of_token.device
    M_cap = dg_moe_contiguous_max_rows(T, G) if M_cap is None else M_cap
    row = torch.empty(T, dtype=torch.int32, device=dev)
    ids = torch.empty(M_cap, dtype=torch.int32, device=dev)
    tok = torch.empty(M_cap, dtype=torch.int32, device=dev)
    layout = torch.empty(G + 1, dtype=torch.int32, device=dev)
    lib = _lib.load()
    st = lib.dg_moe_route_contiguous(_dev_or_null(expert_of_token, "expert_of_token"), T, G,
                                     _dev_or_null(row, "row"), _dev_or_null(ids, "ids"),
                                     _dev_or_null(tok, "tok"), _dev(layout, "layout"), M_cap, _stream(stream))
    _check(st, "dg_moe_route_contiguous")
    return row, ids, tok, layout


def dg_moe_unpermute(d, row_of_token, out=None, stream=None):
    """out[t] = d[row_of_token[t]] (bf16 rows); out-of-range rows give zeros."""
    if d.dtype != torch.bfloat16 or d.dim() != 2 or d.stride(-1) != 1:
        raise TypeError("d must be a 2-D bfloat16 tensor with contiguous rows")
    if row_of_token.dtype != torch.int32 or row_of_token.dim() != 1:
        raise TypeError("row_of_token must be a 1-D int32 tensor")
    T, N = row_of_token.shape[0], d.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=d.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (T, N) or out.stride(-1) != 1:
        raise ValueError("out must be a bfloat16 [T, N] tensor with contiguous rows")
    lib = _lib.load()
    st = lib.dg_moe_unpermute(_dev_or_null(d, "d"), d.stride(0), d.shape[0],
                              _dev_or_null(row_of_token, "row_of_token"), T, N,
                              _dev_or_null(out, "out"), out.stride(0), _stream(stream))
    _check(st, "dg_moe_unpermute")
    return out


def _fmt_codes(t, name, ndim):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2) or t.dim() != ndim or t.stride(-1) != 1:
        raise TypeError("%s must be a %d-D fp8 code tensor with a contiguous last (K) dimension" % (name, ndim))


def dg_fp8_grouped_gemm_contiguous_fmt(a, sa, b, sb, expert_ids, a_fmt="e4m3", b_fmt="e4m3", d=None, stream=None):
    """dg_fp8_grouped_gemm_contiguous with a per-operand fp8 format ("e4m3" or "e5m2")."""
    _fmt_codes(a, "a", 2), _fmt_codes(b, "b", 3), _scales(sa, "sa", 2), _scales(sb, "sb", 3)
    M_total, K = a.shape
    G, N, _ = b.shape
    if d is None:
        d = torch.empty((M_total, N), dtype=torch.bfloat16, device=a.device)
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_contiguous_fmt(
        _dev(a, "a"), FORMATS[a_fmt], a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        _dev(b, "b"), FORMATS[b_fmt], b.stride(1), b.stride(0), _dev(sb, "sb"), sb.stride(0), sb.stride(1),
        sb.stride(2), _dev(expert_ids, "expert_ids"), _dev(d, "d"), d.stride(0), M_total, N, K, G, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_contiguous_fmt")
    return d


def dg_fp8_grouped_gemm_masked_fmt(a, sa, b, sb, masked_m, a_fmt="e4m3", b_fmt="e4m3", d=None, stream=None):
    """dg_fp8_grouped_gemm_masked with a per-operand fp8 format ("e4m3" or "e5m2")."""
    _fmt_codes(a, "a", 3), _fmt_codes(b, "b", 3), _scales(sa, "sa", 3), _scales(sb, "sb", 3)
    G, M_max, K = a.shape
    N = b.shape[1]
    if d is None:
        d = torch.empty((G, M_max, N), dtype=torch.bfloat16, device=a.device)
    lib = _lib.load()
    st = lib.dg_fp8_grouped_gemm_masked_fmt(
        _dev(a, "a"), FORMATS[a_fmt], a.stride(1), a.stride(0), _dev(sa, "sa"), sa.stride(0), sa.stride(1),
        sa.stride(2), _dev(b, "b"), FORMATS[b_fmt], b.stride(1), b.stride(0), _dev(sb, "sb"), sb.stride(0),
        sb.stride(1), sb.stride(2), _dev(masked_m, "masked_m"), _dev(d, "d"), d.stride(1), d.stride(0),
        G, M_max, N, K, _stream(stream))
    _check(st, "dg_fp8_grouped_gemm_masked_fmt")
    return d
