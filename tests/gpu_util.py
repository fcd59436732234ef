"""Device-side helpers shared by the GPU tests (marshalling only)."""
import numpy as np
import torch

from fp8_block_scaled_sa_amd import ops
from tests.check import SENTINEL


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel_bf16(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def run_dense(a, sa, b, sb, stream=None, d=None):
    """a [M,K] u8, sa logical [M,K/128] (numpy, any layout), b [N,K], sb [N/128,K/128]."""
    M, N = a.shape[0], b.shape[0]
    sa = np.asarray(sa, np.float32)
    if sa.strides[0] < sa.strides[1]:           # M-major: keep the layout on the device
        sa_d = dev(np.ascontiguousarray(sa.T)).t()
    else:
        sa_d = dev(sa)
    if d is None:
        d = sentinel_bf16((M, N))
    ops.dg_fp8_gemm_nt(dev(a), sa_d, dev(b), dev(sb), d=d, stream=stream)
    torch.cuda.synchronize()
    return bits(d)


def run_contiguous(c, ids=None):
    ids = c.ids if ids is None else ids
    d = sentinel_bf16((c.M_total, c.N))
    ops.dg_fp8_grouped_gemm_contiguous(dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb),
                                       dev(np.asarray(ids, np.int32)), d=d)
    torch.cuda.synchronize()
    return bits(d)


def run_masked(m, masked_m=None):
    mm = m.masked_m if masked_m is None else masked_m
    d = sentinel_bf16((m.G, m.M_max, m.N))
    ops.dg_fp8_grouped_gemm_masked(dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb),
                                   dev(np.asarray(mm, np.int32)), d=d)
    torch.cuda.synchronize()
    return bits(d)
