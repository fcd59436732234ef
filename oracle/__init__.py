"""ctypes binding of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never does. All
arguments are numpy arrays on the host; strides are in elements.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def configure(cdll):
    """Set the return and argument types of an oracle library (also used by
    the tests that load copies of the oracle with planted mistakes)."""
    _lib_setup(cdll)
    return cdll


def lib():
    global _lib
    if _lib is None:
        _lib = configure(ctypes.CDLL(build()))
    return _lib


def _lib_setup(cdll):
    cdll.dgo_e4m3_decode.restype = ctypes.c_double
    cdll.dgo_e4m3_decode.argtypes = [ctypes.c_uint8]
    cdll.dgo_bf16_rne.restype = ctypes.c_uint16
    cdll.dgo_bf16_rne.argtypes = [ctypes.c_double]
    cdll.dgo_block_partial.restype = ctypes.c_double
    cdll.dgo_block_partial.argtypes = [_p, _p]
    cdll.dgo_max_threads.restype = ctypes.c_int
    cdll.dgo_e4m3_encode.restype = ctypes.c_uint8
    cdll.dgo_e4m3_encode.argtypes = [ctypes.c_float]
    cdll.dgo_quantize_1x128.restype = None
    cdll.dgo_moe_route_contiguous.restype = ctypes.c_int
    cdll.dgo_e5m2_decode.restype = ctypes.c_double
    cdll.dgo_e5m2_decode.argtypes = [ctypes.c_uint8]
    cdll.dgo_block_partial_fmt.restype = ctypes.c_double
    cdll.dgo_block_partial_fmt.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int]
    cdll.dgo_gemm_nt_fmt.restype = None
    cdll.dgo_gemm_nt_fmt_points.restype = None
    cdll.dgo_moe_unpermute.restype = None
    for name in ("dgo_gemm_nt", "dgo_gemm_nt_points", "dgo_grouped_contiguous",
                 "dgo_grouped_contiguous_points", "dgo_grouped_masked",
                 "dgo_grouped_masked_points"):
        getattr(cdll, name).restype = None


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return ctypes.c_void_p(a.ctypes.data)


def _threads(threads):
    return ctypes.c_int(0 if threads is None else int(threads))


def max_threads() -> int:
    return int(lib().dgo_max_threads())


def e4m3_decode(code: int) -> float:
    return float(lib().dgo_e4m3_decode(int(code)))


def bf16_rne(x: float) -> int:
    return int(lib().dgo_bf16_rne(float(x)))


def block_partial(a128: np.ndarray, b128: np.ndarray) -> float:
    a = np.ascontiguousarray(a128, dtype=np.uint8)
    b = np.ascontiguousarray(b128, dtype=np.uint8)
    assert a.size == 128 and b.size == 128
    return float(lib().dgo_block_partial(_ptr(a), _ptr(b)))


def gemm_nt(a, sa, b, sb, want_acc=False, threads=None):
    """Dense NT. ``a [M,K]`` u8, ``sa`` logical ``[M, K/128]`` fp32 (any strides),
    ``b [N,K]`` u8, ``sb [N/128, K/128]`` fp32. Returns bf16 bits ``[M,N]`` (u16)
    and, if asked, the fp64 values."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    sa = np.asarray(sa, dtype=np.float32)
    sb = np.asarray(sb, dtype=np.float32)
    sa_base, sa_m, sa_kb = _strided(sa)
    sb_base, sb_nb, sb_kb = _strided(sb)
    d = np.zeros((M, N), dtype=np.uint16)
    acc = np.zeros((M, N), dtype=np.float64) if want_acc else None
    lib().dgo_gemm_nt(_ptr(a), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                      _ptr(b), _i64(K), sb_base, _i64(sb_nb), _i64(sb_kb),
                      _i64(M), _i64(N), _i64(K),
                      _ptr(acc) if acc is not None else None, _ptr(d), _i64(N), _threads(threads))
    return (d, acc) if want_acc else d


def gemm_nt_points(a, sa, b, sb, ms, ns, threads=None):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    K = a.shape[1]
    sa_base, sa_m, sa_kb = _strided(np.asarray(sa, dtype=np.float32))
    sb_base, sb_nb, sb_kb = _strided(np.asarray(sb, dtype=np.float32))
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    cnt = ms.shape[0]
    acc = np.zeros(cnt, dtype=np.float64)
    d = np.zeros(cnt, dtype=np.uint16)
    lib().dgo_gemm_nt_points(_ptr(a), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                             _ptr(b), _i64(K), sb_base, _i64(sb_nb), _i64(sb_kb),
                             _i64(K), _ptr(ms), _ptr(ns), _i64(cnt), _ptr(acc), _ptr(d),
                             _threads(threads))
    return d, acc


def grouped_contiguous(a, sa, b, sb, ids, d_init, threads=None):
    """``a [M_total,K]``, ``sa`` logical ``[M_total,K/128]``, ``b [G,N,K]``,
    ``sb [G,N/128,K/128]``, ``ids [M_total]`` int32. ``d_init [M_total,N]`` u16 is
    copied and the produced rows overwritten; other rows keep their bits."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M_total, K = a.shape
    G, N, _ = b.shape
    sa_base, sa_m, sa_kb = _strided(np.asarray(sa, dtype=np.float32))
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    d = np.array(d_init, dtype=np.uint16, copy=True, order="C")
    lib().dgo_grouped_contiguous(_ptr(a), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                                 _ptr(b), _i64(K), _i64(N * K),
                                 _ptr(sb), _i64(sb.shape[1] * sb.shape[2]), _i64(sb.shape[2]), _i64(1),
                                 _ptr(ids), _ptr(d), _i64(N),
                                 _i64(M_total), _i64(N), _i64(K), _i64(G), _threads(threads))
    return d


def grouped_contiguous_points(a, sa, b, sb, ids, rows, ns, threads=None):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M_total, K = a.shape
    G, N, _ = b.shape
    sa_base, sa_m, sa_kb = _strided(np.asarray(sa, dtype=np.float32))
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    cnt = rows.shape[0]
    acc = np.zeros(cnt, dtype=np.float64)
    d = np.zeros(cnt, dtype=np.uint16)
    produced = np.zeros(cnt, dtype=np.uint8)
    lib().dgo_grouped_contiguous_points(_ptr(a), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                                        _ptr(b), _i64(K), _i64(N * K),
                                        _ptr(sb), _i64(sb.shape[1] * sb.shape[2]), _i64(sb.shape[2]),
                                        _i64(1), _ptr(ids), _i64(K), _i64(G),
                                        _ptr(rows), _ptr(ns), _i64(cnt),
                                        _ptr(acc), _ptr(d), _ptr(produced), _threads(threads))
    return d, acc, produced.astype(bool)


def grouped_masked(a, sa_t, b, sb, masked_m, d_init, threads=None):
    """``a [G,M_max,K]``, ``sa_t [G,K/128,M_max]`` (per-group M-major),
    ``b [G,N,K]``, ``sb [G,N/128,K/128]``, ``masked_m [G]`` int32,
    ``d_init [G,M_max,N]`` u16 copied; produced rows overwritten."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    G, M_max, K = a.shape
    N = b.shape[1]
    sa_t = np.ascontiguousarray(sa_t, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    mm = np.ascontiguousarray(masked_m, dtype=np.int32)
    d = np.array(d_init, dtype=np.uint16, copy=True, order="C")
    lib().dgo_grouped_masked(_ptr(a), _i64(K), _i64(M_max * K),
                             _ptr(sa_t), _i64(sa_t.shape[1] * sa_t.shape[2]), _i64(1), _i64(M_max),
                             _ptr(b), _i64(K), _i64(N * K),
                             _ptr(sb), _i64(sb.shape[1] * sb.shape[2]), _i64(sb.shape[2]), _i64(1),
                             _ptr(mm), _ptr(d), _i64(N), _i64(M_max * N),
                             _i64(G), _i64(M_max), _i64(N), _i64(K), _threads(threads))
    return d


def grouped_masked_points(a, sa_t, b, sb, masked_m, gs, ms, ns, threads=None):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    G, M_max, K = a.shape
    N = b.shape[1]
    sa_t = np.ascontiguousarray(sa_t, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    mm = np.ascontiguousarray(masked_m, dtype=np.int32)
    gs = np.ascontiguousarray(gs, dtype=np.int64)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    cnt = gs.shape[0]
    acc = np.zeros(cnt, dtype=np.float64)
    d = np.zeros(cnt, dtype=np.uint16)
    produced = np.zeros(cnt, dtype=np.uint8)
    lib().dgo_grouped_masked_points(_ptr(a), _i64(K), _i64(M_max * K),
                                    _ptr(sa_t), _i64(sa_t.shape[1] * sa_t.shape[2]), _i64(1), _i64(M_max),
                                    _ptr(b), _i64(K), _i64(N * K),
                                    _ptr(sb), _i64(sb.shape[1] * sb.shape[2]), _i64(sb.shape[2]), _i64(1),
                                    _ptr(mm), _i64(M_max), _i64(K),
                                    _ptr(gs), _ptr(ms), _ptr(ns), _i64(cnt),
                                    _ptr(acc), _ptr(d), _ptr(produced), _threads(threads))
    return d, acc, produced.astype(bool)


def e4m3_encode(v: float) -> int:
    """Nearest e4m3 code (ties to even) of the fp32 value ``v`` clamped to +-448."""
    return int(lib().dgo_e4m3_encode(float(v)))


def quantize_1x128(x, threads=None):
    """1x128 block quantisation of activations ``x [M, K]``: fp32, or bf16 given
    as a torch bfloat16 tensor or as uint16 bit patterns. Returns
    ``(codes [M, K] u8, scales [M, K/128] fp32)``."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = (x.contiguous().view(torch.int16).numpy().view(np.uint16)
                 if x.dtype == torch.bfloat16 else x.contiguous().numpy())
    except ImportError:
        pass
    is_bf16 = x.dtype == np.uint16
    x = np.ascontiguousarray(x, dtype=np.uint16 if is_bf16 else np.float32)
    M, K = x.shape
    assert K % 128 == 0
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, K // 128), dtype=np.float32)
    lib().dgo_quantize_1x128(_ptr(x), ctypes.c_int(int(is_bf16)), _i64(K), _i64(M), _i64(K),
                             _ptr(q), _i64(K), _ptr(s), _i64(K // 128), _i64(1), _threads(threads))
    return q, s


FMTS = {"e4m3": 0, "e5m2": 1}


def e5m2_decode(code: int) -> float:
    return float(lib().dgo_e5m2_decode(int(code)))


def block_partial_fmt(a128, fa, b128, fb) -> float:
    a = np.ascontiguousarray(a128, dtype=np.uint8)
    b = np.ascontiguousarray(b128, dtype=np.uint8)
    assert a.size == 128 and b.size == 128
    return float(lib().dgo_block_partial_fmt(_ptr(a), ctypes.c_int(FMTS[fa]), _ptr(b), ctypes.c_int(FMTS[fb])))


def gemm_nt_fmt(a, fa, sa, b, fb, sb, want_acc=False, threads=None):
    """Dense NT with operand formats ``fa``/``fb`` ("e4m3" or "e5m2"); else as gemm_nt."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    sa_base, sa_m, sa_kb = _strided(np.asarray(sa, dtype=np.float32))
    sb_base, sb_nb, sb_kb = _strided(np.asarray(sb, dtype=np.float32))
    d = np.zeros((M, N), dtype=np.uint16)
    acc = np.zeros((M, N), dtype=np.float64) if want_acc else None
    lib().dgo_gemm_nt_fmt(_ptr(a), ctypes.c_int(FMTS[fa]), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                          _ptr(b), ctypes.c_int(FMTS[fb]), _i64(K), sb_base, _i64(sb_nb), _i64(sb_kb),
                          _i64(M), _i64(N), _i64(K), _ptr(acc) if acc is not None else None, _ptr(d), _i64(N),
                          _threads(threads))
    return (d, acc) if want_acc else d


def gemm_nt_fmt_points(a, fa, sa, b, fb, sb, ms, ns, threads=None):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    K = a.shape[1]
    sa_base, sa_m, sa_kb = _strided(np.asarray(sa, dtype=np.float32))
    sb_base, sb_nb, sb_kb = _strided(np.asarray(sb, dtype=np.float32))
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    cnt = ms.shape[0]
    acc = np.zeros(cnt, dtype=np.float64)
    d = np.zeros(cnt, dtype=np.uint16)
    lib().dgo_gemm_nt_fmt_points(_ptr(a), ctypes.c_int(FMTS[fa]), _i64(K), sa_base, _i64(sa_m), _i64(sa_kb),
                                 _ptr(b), ctypes.c_int(FMTS[fb]), _i64(K), sb_base, _i64(sb_nb), _i64(sb_kb),
                                 _i64(K), _ptr(ms), _ptr(ns), _i64(cnt), _ptr(acc), _ptr(d), _threads(threads))
    return d, acc


def moe_max_rows(T: int, G: int) -> int:
    """Rows that always hold the padded contiguous layout of T tokens over G
    experts: each used expert wastes fewer than 128 rows."""
    return 128 * (-(-T // 128) + min(G, T))


def moe_route_contiguous(expert_of_token, G, M_cap=None):
    """Returns ``(row_of_token [T], expert_ids [M_cap], token_of_row [M_cap],
    layout [G+1])`` as int32 arrays."""
    e = np.ascontiguousarray(expert_of_token, dtype=np.int32)
    T = e.shape[0]
    M_cap = moe_max_rows(T, G) if M_cap is None else M_cap
    row = np.zeros(T, np.int32)
    ids = np.zeros(max(M_cap, 1), np.int32)
    tok = np.zeros(max(M_cap, 1), np.int32)
    layout = np.zeros(G + 1, np.int32)
    st = lib().dgo_moe_route_contiguous(_ptr(e), _i64(T), _i64(G), _ptr(row), _ptr(ids), _ptr(tok),
                                        _ptr(layout), _i64(M_cap))
    if st != 0:
        raise ValueError("M_cap too small for this routing")
    return row, ids[:M_cap], tok[:M_cap], layout


def moe_unpermute(d_bits, row_of_token):
    """``out[t] = d[row_of_token[t]]`` (bf16 bits, u16); out-of-range rows give zeros."""
    d = np.ascontiguousarray(d_bits, dtype=np.uint16)
    r = np.ascontiguousarray(row_of_token, dtype=np.int32)
    rows, N = d.shape
    T = r.shape[0]
    out = np.zeros((T, N), np.uint16)
    lib().dgo_moe_unpermute(_ptr(d), _i64(N), _i64(rows), _ptr(r), _i64(T), _i64(N), _ptr(out), _i64(N))
    return out


def _strided(s: np.ndarray):
    """Pointer and element strides of a 2-D fp32 view (any layout, base kept alive by caller)."""
    assert s.ndim == 2 and s.dtype == np.float32
    st = [x // 4 for x in s.strides]
    assert all(x >= 0 for x in st)
    return ctypes.c_void_p(s.ctypes.data), st[0], st[1]
