"""MI355X (gfx950) fine-grained block-scaled FP8 GEMM.

D = A . B^T with e4m3 operands, 1x128 LHS scales, 128x128 RHS scales, fp32
per-K-block promotion and a bf16 output, as a dense NT GEMM and as two MoE
grouped layouts (contiguous, masked), plus the 1x128 activation quantiser
that produces the GEMM's LHS and the MoE routing steps around the
contiguous layout. The kernels live in libdg_fp8.so behind
the C ABI of include/dg_fp8.h; this package is its thin Python binding.
"""
from .ops import (DGError, dg_fp8_gemm_nt, dg_fp8_gemm_nt_fmt, dg_fp8_grouped_gemm_contiguous,  # noqa: F401
                  dg_fp8_gemm_nt_ws, dg_fp8_gemm_nt_workspace_bytes, dg_fp8_grouped_gemm_contiguous_ws,
                  dg_fp8_grouped_gemm_contiguous_workspace_bytes, workspace,
                  dg_fp8_grouped_gemm_contiguous_fmt, dg_fp8_grouped_gemm_contiguous_layout,
                  dg_fp8_grouped_gemm_contiguous_to_tokens,
                  dg_fp8_grouped_gemm_masked_fmt,
                  dg_fp8_grouped_gemm_masked, dg_fp8_quantize_1x128, dg_fp8_quantize_1x128_gather,
                  dg_moe_contiguous_max_rows, dg_moe_route_contiguous, dg_moe_unpermute)
