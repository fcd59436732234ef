"""Device-side helpers shared by the GPU tests (marshalling only)."""
import numpy as np
import torch

from fp8_block_scaled_sa_amd import ops
from tests.check import SENTINEL


# Guard bands: every output made by sentinel_bf16 sits between GUARD bf16
# elements (4 KB) of sentinel on either side, inside one allocation, and
# bits() checks that both bands are still untouched whenever it reads such an
# output back.
GUARD = 2048


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def guards_intact(t) -> bool:
    """Both 4 KB sentinel bands around an output of sentinel_bf16 are unwritten."""
    whole = torch.empty(0, dtype=torch.int16, device=t.device).set_(t.untyped_storage())
    n = whole.numel()
    band = torch.cat([whole[:GUARD], whole[n - GUARD:]])
    return bool((band == SENTINEL).all().item())


def bits(t):
    if getattr(t, "_guarded", False):
        assert guards_intact(t), "a kernel wrote into the guard band around its output"
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel_bf16(shape):
    """A bf16 output filled with the sentinel, with a 4 KB sentinel guard band
    before and after it in the same allocation."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int16, device="cuda")
    view = buf[GUARD:GUARD + n].view(tuple(shape)).view(torch.bfloat16)
    view._guarded = True
    return view


def run_dense(a, sa, b, sb, stream=None, d=None, ws=False):
    """a [M,K] u8, sa logical [M,K/128] (numpy, any layout), b [N,K], sb [N/128,K/128].
    ws: call dg_fp8_gemm_nt_ws with the workspace its query asks for."""
    M, N = a.shape[0], b.shape[0]
    sa = np.asarray(sa, np.float32)
    if sa.strides[0] < sa.strides[1]:           # M-major: keep the layout on the device
        sa_d = dev(np.ascontiguousarray(sa.T)).t()
    else:
        sa_d = dev(sa)
    if d is None:
        d = sentinel_bf16((M, N))
    if ws:
        w = ops.workspace(ops.dg_fp8_gemm_nt_workspace_bytes(M, N, a.shape[1]))
        ops.dg_fp8_gemm_nt_ws(dev(a), sa_d, dev(b), dev(sb), w, d=d, stream=stream)
    else:
        ops.dg_fp8_gemm_nt(dev(a), sa_d, dev(b), dev(sb), d=d, stream=stream)
    torch.cuda.synchronize()
    return bits(d)


def run_contiguous(c, ids=None, ws=False, layout=None):
    """ws: call dg_fp8_grouped_gemm_contiguous_ws with the workspace its query
    asks for (segment offsets derived on the device, split tails); layout:
    the segment offsets to pass (numpy [G+1])."""
    ids = c.ids if ids is None else ids
    d = sentinel_bf16((c.M_total, c.N))
    args = (dev(c.a), dev(c.sa_t).t(), dev(c.b), dev(c.sb), dev(np.asarray(ids, np.int32)))
    lay = None if layout is None else dev(np.asarray(layout, np.int32))
    if ws:
        w = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(c.M_total, c.N, c.K, c.G))
        ops.dg_fp8_grouped_gemm_contiguous_ws(*args, w, layout=lay, d=d)
    elif lay is not None:
        ops.dg_fp8_grouped_gemm_contiguous_layout(*args, lay, d=d)
    else:
        ops.dg_fp8_grouped_gemm_contiguous(*args, d=d)
    torch.cuda.synchronize()
    return bits(d)


def run_masked(m, masked_m=None):
    mm = m.masked_m if masked_m is None else masked_m
    d = sentinel_bf16((m.G, m.M_max, m.N))
    ops.dg_fp8_grouped_gemm_masked(dev(m.a), dev(m.sa_t).transpose(1, 2), dev(m.b), dev(m.sb),
                                   dev(np.asarray(mm, np.int32)), d=d)
    torch.cuda.synchronize()
    return bits(d)
