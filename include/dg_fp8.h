/*
 * dg_fp8.h -- C ABI of the MI355X (gfx950) fine-grained block-scaled FP8 GEMM.
 *
 * Operation (all three entry points):
 *
 *   D[m, n] = bf16_rne( sum_kb  sA[m, kb] * sB[n/128, kb]
 *                               * sum_{k in [128 kb, 128 kb + 128)} A[m, k] * B[n, k] )
 *
 *   - A and B hold OCP e4m3 codes (1 sign, 4 exponent bits with bias 7,
 *     3 mantissa bits, largest finite 448, no infinity): rkmt.cn DeepGEMM
 *     walkthrough §2.1 and §5.2; lpnh.cn DeepGEMM article §2.1.
 *   - LHS scales cover 1x128 tiles (one fp32 per row and 128-wide K block),
 *     RHS scales cover 128x128 tiles: hotdry.top fine-grained scaling article,
 *     "fine-grained scaling core design".
 *   - Each 128-wide K block's partial product is multiplied by sA*sB before
 *     it is added to an fp32 accumulator, because the scale product changes
 *     from block to block: lpnh.cn §2.3; hotdry.top "two-level accumulation".
 *   - The output is bf16 (round to nearest even). D is overwritten; there is
 *     no C/bias term and no accumulation into D.
 *
 * "NT": A is [M, K] and B is [N, K], both with K contiguous, D = A . B^T.
 *
 * dg_fp8_quantize_1x128 (at the end) produces A and sA from fp32 or bf16
 * activations: the quantisation step that precedes the GEMM. For the
 * contiguous MoE layout, dg_moe_route_contiguous lays tokens out by expert,
 * dg_fp8_quantize_1x128_gather quantises them into that layout and
 * dg_moe_unpermute brings the GEMM's rows back into token order.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers owned by the caller; the library never
 *     keeps one past return.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). The call
 *     validates its arguments on the host, enqueues its kernels and returns.
 *     The library never allocates or frees device memory and never
 *     synchronises a stream. Scratch memory (split-K partial sums, segment
 *     offsets derived on the device) is the caller's: the *_ws entry points
 *     take a workspace pointer and size (a caller workspace, 16-byte aligned:
 *     bhfrc.com DeepGEMM article, §5.2), and the matching *_workspace_bytes
 *     query says how much the fastest path takes. Calls without a workspace
 *     take the paths that need none. Every call is therefore safe to capture
 *     into a HIP graph: its kernels only read and write memory the caller
 *     passed, at addresses fixed at capture (bhfrc.com §4.3).
 *   - Strides are in elements. e4m3 is one byte, so A/B strides are also byte
 *     strides; D strides count bf16 elements. Scale tables are addressed
 *     logically through explicit strides: sA[m, kb] = sA[m*sa_stride_m +
 *     kb*sa_stride_kb], sB[nb, kb] = sB[nb*sb_stride_nb + kb*sb_stride_kb].
 *     Row-major and M-major scale layouts are both legal; a zero stride
 *     broadcasts (e.g. per-tensor scales).
 *   - Alignment: A, B and D base addresses 16-byte aligned; lda, ldb and the
 *     grouped byte strides multiples of 16; ldd (and d_stride_g) multiples of
 *     8 elements; scale pointers 4-byte aligned.
 *   - Shapes: K > 0 and K % 128 == 0; N % 128 == 0; M arbitrary (>= 0).
 *   - D must not overlap A, B, sA, sB or the routing arrays.
 *   - Results are deterministic: no atomics, a fixed reduction order.
 *   - Thread-safe: the only global state is a per-device property cache,
 *     filled once under a lock. Calls that share a workspace must not run
 *     concurrently (issue them on one stream, or give each its own).
 *
 * Errors: every error is detected on the host before anything is enqueued,
 * and D is left untouched. DG_ERR_HIP reports a failed launch; the HIP error
 * code is kept per thread (dg_last_hip_error). An empty problem (M = 0,
 * N = 0, M_total = 0 or G = 0) returns DG_OK without launching.
 */
#ifndef DG_FP8_H
#define DG_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_ABI_VERSION 2

typedef enum dg_status {
    DG_OK = 0,
    DG_ERR_NULL_POINTER = 1, /* a required pointer is NULL for a non-empty problem */
    DG_ERR_BAD_SHAPE = 2,    /* negative dim, K <= 0, K % 128, N % 128, M_total % 128 */
    DG_ERR_MISALIGNED = 3,   /* base pointer or stride violates the alignment rules */
    DG_ERR_BAD_STRIDE = 4,   /* lda < K, ldb < K, ldd < N, negative or too small group stride */
    DG_ERR_UNSUPPORTED = 5,  /* current device is not gfx950, or a size exceeds int32 */
    DG_ERR_HIP = 6,          /* the HIP runtime failed (query or launch) */
    DG_ERR_ALIASING = 7,     /* D (or the workspace) overlaps an input or the output */
    DG_ERR_SCRATCH = 8       /* dg_fp8_gemm_nt_noalloc: more scratch needed than its static buffer holds */
} dg_status;

/* Version of this ABI (DG_ABI_VERSION). */
int dg_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *dg_status_string(dg_status status);

/* hipError_t of the last DG_ERR_HIP returned on the calling thread (0 if none). */
int dg_last_hip_error(void);

/*
 * Dense NT GEMM.
 *   A  [M, K] e4m3, row stride lda          sA fp32, logical [M, K/128]
 *   B  [N, K] e4m3, row stride ldb          sB fp32, logical [N/128, K/128]
 *   D  [M, N] bf16, row stride ldd (written)
 * Operation as in the header comment (lpnh.cn §2.3; hotdry.top, fine-grained
 * scaling core design).
 *
 * Without a workspace this call never splits a tile's K loop: medium M
 * (64 < M up to ~2000 at N = 4096, where the output tiles would fill at most
 * half of the CUs) then runs with few busy CUs. dg_fp8_gemm_nt_ws gives it
 * the workspace for the split-K path.
 *
 * Large grids: when the 256x256 output tiles fill the CUs but leave a last
 * round at most half full, the call is issued as two launches on the same
 * stream, the whole-round part of the columns (else rows) on 256x256 tiles
 * and the remaining strip on smaller tiles. The cut depends only on the
 * shape and the CU count.
 */
dg_status dg_fp8_gemm_nt(const void *A, int64_t lda,
                         const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                         const void *B, int64_t ldb,
                         const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                         void *D, int64_t ldd,
                         int64_t M, int64_t N, int64_t K, void *stream);

/*
 * dg_fp8_gemm_nt with a caller workspace for its split-K path.
 *   workspace        device memory owned by the caller, 16-byte aligned, or NULL
 *   workspace_bytes  its size in bytes (>= 0)
 * When the output tiles would fill at most half of the CUs (M > 64, or
 * 24 < M <= 64 where the small-M kernel's LDS staging does not fit and
 * K >= 2048), each tile's K blocks are split over up to 8 work items that
 * write fp32 partial sums (slices x M x N x 4 bytes) to the workspace, and a
 * second kernel adds the slices in a fixed order (deterministic). A workspace
 * smaller than dg_fp8_gemm_nt_workspace_bytes takes as many slices as it
 * holds (none below two: then this is dg_fp8_gemm_nt). The split only
 * regroups the fp32 additions; results stay within the oracle tolerance.
 * The workspace must not overlap D or an input (DG_ERR_ALIASING); its
 * contents on entry do not matter and are garbage on return. Calls that use
 * one workspace must be ordered (one stream): a later call overwrites it.
 */
dg_status dg_fp8_gemm_nt_ws(const void *A, int64_t lda,
                            const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                            const void *B, int64_t ldb,
                            const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                            void *D, int64_t ldd,
                            int64_t M, int64_t N, int64_t K,
                            void *workspace, int64_t workspace_bytes, void *stream);

/*
 * dg_fp8_gemm_nt_ws for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it): the
 * split-K partial sums go to a 32 MiB array inside the library's code object
 * instead of a caller workspace. Each GPU the library runs on holds its own
 * copy of the array until the process ends; the call allocates nothing and
 * calls no allocating routine. Results are bit-identical to dg_fp8_gemm_nt_ws
 * given a workspace of dg_fp8_gemm_nt_workspace_bytes bytes.
 * Limit: a problem whose split-K path needs more than 32 MiB returns
 * DG_ERR_SCRATCH before anything is enqueued (no dense shape does on a
 * 256-CU MI355X: at most 256 partial tiles of 256x128 fp32).
 * Every call on one GPU shares that GPU's array: calls whose kernels may
 * overlap in time (different streams without ordering, several host threads)
 * race on it and must not be issued; calls on one stream are ordered and
 * safe. Other arguments and errors as dg_fp8_gemm_nt.
 */
dg_status dg_fp8_gemm_nt_noalloc(const void *A, int64_t lda,
                                 const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                 const void *B, int64_t ldb,
                                 const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                                 void *D, int64_t ldd,
                                 int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Workspace bytes the fastest path of dg_fp8_gemm_nt_ws takes for this shape
 * on the current device (0: that path needs none), assuming operands with
 * K-contiguous rows (lda = ldb = K). A negative value is -dg_status: a bad
 * shape, or a device that is not gfx950. Launches nothing.
 */
int64_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Operand formats of dg_fp8_gemm_nt_fmt. */
#define DG_FP8_E4M3 0
#define DG_FP8_E5M2 1

/*
 * Dense NT GEMM with a choice of fp8 format per operand: OCP e4m3 (largest
 * finite 448) or e5m2 (1 sign, 5 exponent bits with bias 15, 2 mantissa
 * bits, largest finite 57344): rkmt.cn walkthrough §2.1; mixing an e4m3 A
 * with an e5m2 B trades precision for range: lpnh.cn article §2.1. The
 * operation, the scale granularity, the arguments and the errors are those
 * of dg_fp8_gemm_nt; a_fmt / b_fmt are DG_FP8_E4M3 or DG_FP8_E5M2 (else
 * DG_ERR_UNSUPPORTED). Infinity and NaN codes in an operand give unspecified
 * results. With both operands e4m3 this is dg_fp8_gemm_nt; every other
 * combination runs on the tile kernel at every M (never split over K: this
 * call takes no workspace).
 */
dg_status dg_fp8_gemm_nt_fmt(const void *A, int a_fmt, int64_t lda,
                             const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                             const void *B, int b_fmt, int64_t ldb,
                             const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                             void *D, int64_t ldd,
                             int64_t M, int64_t N, int64_t K, void *stream);

/*
 * Grouped GEMM, contiguous layout (MoE): the rows of all experts are stacked
 * in one LHS, each expert's rows contiguous and padded to a multiple of 128,
 * and expert_ids[r] names the expert of row r (one launch for all experts:
 * rkmt.cn walkthrough §1.2 and §5.3; hotdry.top, grouped GEMM parameters).
 *   A  [M_total, K] e4m3, row stride lda    sA logical [M_total, K/128]
 *   B  [G, N, K] e4m3: expert e at B + e*b_stride_g, row stride ldb
 *   sB logical [G, N/128, K/128]: sB[e, nb, kb] = sB[e*sb_stride_g + nb*sb_stride_nb + kb*sb_stride_kb]
 *   expert_ids [M_total] int32, device memory
 *   D  [M_total, N] bf16, row stride ldd
 * Row r is computed against expert expert_ids[r] when 0 <= id < G. Rows whose
 * id is -1 (padding) or outside [0, G) are NOT written.
 * Layout contract: M_total % 128 == 0 and within every aligned 128-row block
 * all ids in [0, G) are equal (segments padded to 128). A block's expert is
 * the largest id in the block; a row whose id differs from it is not written.
 * Tiling: this call takes no workspace, so its tiles cover the rows
 * uniformly (256-row tiles that straddle two experts run one K loop per
 * expert). dg_fp8_grouped_gemm_contiguous_ws with a workspace instead
 * derives the experts' segment offsets on the device and tiles along them.
 */
dg_status dg_fp8_grouped_gemm_contiguous(const void *A, int64_t lda,
                                         const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                         const void *B, int64_t ldb, int64_t b_stride_g,
                                         const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                         int64_t sb_stride_kb,
                                         const int32_t *expert_ids,
                                         void *D, int64_t ldd,
                                         int64_t M_total, int64_t N, int64_t K, int64_t G, void *stream);

/*
 * The contiguous grouped GEMM given each expert's segment offsets as well
 * (the token offsets of the routing: rkmt.cn walkthrough, §5.3):
 *   layout [G + 1] int32 (device): layout[e] is the first row of expert e's
 *   segment, layout[G] the rows used, as written by dg_moe_route_contiguous.
 * Every segment must be a multiple of 128 rows and hold only rows of its
 * expert (or padding rows with id -1), as the contiguous layout requires.
 * With the offsets the GEMM tiles each segment on its own: whole 256-row
 * tiles first, then the segments' last 128 rows, so no tile spans two
 * experts. Result and other arguments as dg_fp8_grouped_gemm_contiguous;
 * 1 <= G <= 1024. A layout that does not match expert_ids leaves rows
 * unwritten (no fault).
 * This call takes no workspace: the segments' last 128 rows run on 256-row
 * tiles in the same launch. dg_fp8_grouped_gemm_contiguous_ws with a
 * workspace splits them over K (see there).
 */
dg_status dg_fp8_grouped_gemm_contiguous_layout(const void *A, int64_t lda,
                                                const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                                const void *B, int64_t ldb, int64_t b_stride_g,
                                                const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                                int64_t sb_stride_kb,
                                                const int32_t *expert_ids, const int32_t *layout,
                                                void *D, int64_t ldd,
                                                int64_t M_total, int64_t N, int64_t K, int64_t G, void *stream);

/*
 * The contiguous grouped GEMM written straight to token order: row r of the
 * result (a row dg_fp8_grouped_gemm_contiguous would write) goes to row
 * token_of_row[r] of out instead of row r of D, when 0 <= token_of_row[r] < T.
 * This folds dg_moe_unpermute into the GEMM's epilogue.
 *   token_of_row [M_total] int32 (device), as written by dg_moe_route_contiguous
 *   layout [G + 1] int32 (device) or NULL: segment offsets as in
 *   dg_fp8_grouped_gemm_contiguous_layout (then tiles follow the segments);
 *   with NULL the tiles cover the rows uniformly
 *   out [T, N] bf16, row stride ldo: rows of tokens that no row names (dropped
 *   tokens) are NOT written.
 * Precondition: no token appears twice in token_of_row (the routing call
 * guarantees it); otherwise which row lands last is unspecified.
 * Other arguments, constraints and errors as dg_fp8_grouped_gemm_contiguous,
 * with out/ldo/T in place of D/ldd/M_total for the output.
 */
dg_status dg_fp8_grouped_gemm_contiguous_to_tokens(const void *A, int64_t lda,
                                                   const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                                   const void *B, int64_t ldb, int64_t b_stride_g,
                                                   const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                                   int64_t sb_stride_kb,
                                                   const int32_t *expert_ids, const int32_t *token_of_row,
                                                   const int32_t *layout,
                                                   void *out, int64_t ldo, int64_t T,
                                                   int64_t M_total, int64_t N, int64_t K, int64_t G, void *stream);

/*
 * The contiguous grouped GEMM (all three forms above) with a caller
 * workspace for its faster paths.
 *   token_of_row [M_total] int32 or NULL: as in _to_tokens (D is then out
 *   [T, N]); NULL writes row r to row r of D [M_total, N] (T is ignored)
 *   layout [G + 1] int32 or NULL: segment offsets as in _layout
 *   workspace        device memory owned by the caller, 16-byte aligned, or NULL
 *   workspace_bytes  its size in bytes (>= 0)
 * With the workspace:
 *   - without a layout (e4m3, N % 256 == 0, G <= 128, at most 4096 blocks of
 *     128 rows), a one-workgroup kernel first derives each expert's segment
 *     offsets from expert_ids into the workspace's first bytes ((G + 2)
 *     int32, rounded up to 256 bytes), and the GEMM tiles along the segments
 *     as with a layout. If the block experts are not in ascending order
 *     (padding blocks anywhere are fine), the derivation says so on the
 *     device and a uniform-grid launch covers the rows instead; either way
 *     the rows written are the same;
 *   - the segments' last 128 rows (a segment whose size is an odd multiple
 *     of 128) are split over K when those tails would fill under two rounds
 *     of the CUs: at most 8 slices of at least 4 K blocks, the count chosen
 *     on the device from the number of such segments, fp32 partials (slices
 *     x G x 128 x N x 4 bytes, after the offsets) added in slice order by a
 *     reduction kernel. Those rows then differ from the unsplit sum only in
 *     the grouping of the fp32 additions (within the oracle tolerance,
 *     deterministic).
 * A workspace smaller than dg_fp8_grouped_gemm_contiguous_workspace_bytes
 * takes the paths it holds (fewer slices, or none). The workspace must not
 * overlap D or an input; its contents on entry do not matter. Calls that use
 * one workspace must be ordered (one stream).
 * Other arguments, constraints and errors as the calls above.
 */
dg_status dg_fp8_grouped_gemm_contiguous_ws(const void *A, int64_t lda,
                                             const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                             const void *B, int64_t ldb, int64_t b_stride_g,
                                             const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                             int64_t sb_stride_kb,
                                             const int32_t *expert_ids, const int32_t *token_of_row,
                                             const int32_t *layout,
                                             void *D, int64_t ldd, int64_t T,
                                             int64_t M_total, int64_t N, int64_t K, int64_t G,
                                             void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Workspace bytes the fastest path of dg_fp8_grouped_gemm_contiguous_ws takes
 * for this shape on the current device (derived offsets plus split tails; a
 * call given a layout needs no more), assuming K-contiguous operand rows.
 * 0: none is used. A negative value is -dg_status (bad shape, not gfx950).
 */
int64_t dg_fp8_grouped_gemm_contiguous_workspace_bytes(int64_t M_total, int64_t N, int64_t K, int64_t G);

/*
 * The contiguous grouped GEMM with a choice of fp8 format per operand
 * (a_fmt / b_fmt: DG_FP8_E4M3 or DG_FP8_E5M2, as in dg_fp8_gemm_nt_fmt);
 * otherwise identical to dg_fp8_grouped_gemm_contiguous.
 */
dg_status dg_fp8_grouped_gemm_contiguous_fmt(const void *A, int a_fmt, int64_t lda,
                                             const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                                             const void *B, int b_fmt, int64_t ldb, int64_t b_stride_g,
                                             const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                             int64_t sb_stride_kb,
                                             const int32_t *expert_ids,
                                             void *D, int64_t ldd,
                                             int64_t M_total, int64_t N, int64_t K, int64_t G, void *stream);

/*
 * Grouped GEMM, masked layout (MoE decode): every expert owns a fixed block
 * of M_max rows and masked_m[g] (device memory, read by the kernel, so the
 * call needs no host synchronisation and the counts may change between
 * replays of a captured launch: bhfrc.com DeepGEMM article §4.3) says how
 * many of them are valid.
 *   A  [G, M_max, K] e4m3: A_g = A + g*a_stride_g, row stride lda
 *   sA logical [G, M_max, K/128]: sA[g*sa_stride_g + m*sa_stride_m + kb*sa_stride_kb]
 *   B  [G, N, K], sB [G, N/128, K/128] as in the contiguous call
 *   masked_m [G] int32, device memory
 *   D  [G, M_max, N] bf16: D_g = D + g*d_stride_g, row stride ldd
 * Group g writes rows m < clamp(masked_m[g], 0, M_max); all other rows of D
 * are NOT written.
 */
dg_status dg_fp8_grouped_gemm_masked(const void *A, int64_t lda, int64_t a_stride_g,
                                     const float *sA, int64_t sa_stride_g, int64_t sa_stride_m,
                                     int64_t sa_stride_kb,
                                     const void *B, int64_t ldb, int64_t b_stride_g,
                                     const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                     int64_t sb_stride_kb,
                                     const int32_t *masked_m,
                                     void *D, int64_t ldd, int64_t d_stride_g,
                                     int64_t G, int64_t M_max, int64_t N, int64_t K, void *stream);

/*
 * The masked grouped GEMM with a choice of fp8 format per operand (a_fmt /
 * b_fmt: DG_FP8_E4M3 or DG_FP8_E5M2, as in dg_fp8_gemm_nt_fmt); otherwise
 * identical to dg_fp8_grouped_gemm_masked.
 */
dg_status dg_fp8_grouped_gemm_masked_fmt(const void *A, int a_fmt, int64_t lda, int64_t a_stride_g,
                                         const float *sA, int64_t sa_stride_g, int64_t sa_stride_m,
                                         int64_t sa_stride_kb,
                                         const void *B, int b_fmt, int64_t ldb, int64_t b_stride_g,
                                         const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                         int64_t sb_stride_kb,
                                         const int32_t *masked_m,
                                         void *D, int64_t ldd, int64_t d_stride_g,
                                         int64_t G, int64_t M_max, int64_t N, int64_t K, void *stream);

/* Element types of the quantiser's input. */
#define DG_DTYPE_F32 0
#define DG_DTYPE_BF16 1

/*
 * 1x128 activation quantiser: produces the LHS of the calls above (codes and
 * one scale per 1x128 tile: hotdry.top, "fine-grained scaling core design")
 * from fp32 or bf16 activations.
 *   X  [M, K] fp32 (x_dtype DG_DTYPE_F32) or bf16 (DG_DTYPE_BF16), row stride ldx elements
 *   Q  [M, K] e4m3 codes, row stride ldq (written)
 *   S  fp32 logical [M, K/128]: S[m, kb] at S[m*s_stride_m + kb*s_stride_kb] (written)
 * For row m and block kb (columns [128 kb, 128 kb + 128)):
 *   amax = max |X[m, k]| over the block;
 *   s    = amax / 448 as an fp32 division (the initial scale max_val / 448 of
 *          the rkmt.cn walkthrough, §5.2), or 1 when amax is 0;
 *   Q    = the e4m3 code nearest to clamp(X / s, -448, 448), X / s an fp32
 *          division, ties to the even code (round to nearest: lpnh.cn §6.3);
 *          a negative value that rounds to zero gives -0 (0x80).
 * So X ~ dec(Q) * s, and Q/S are directly the A/sA of the GEMM calls (pass
 * sa_stride_m = s_stride_m, sa_stride_kb = s_stride_kb).
 * Inputs must be finite; the codes and scale of a block holding NaN or
 * infinity are unspecified (no fault).
 * Constraints: K > 0, K % 128 == 0; X and Q 16-byte aligned, ldx * element
 * size and ldq multiples of 16; S 4-byte aligned; ldx >= K, ldq >= K; every
 * (m, kb) owns a distinct scale slot (row-major-like or M-major-like strides,
 * >= 0); Q, S and X pairwise disjoint. Errors as for the GEMM calls, plus
 * DG_ERR_UNSUPPORTED for an unknown x_dtype. Deterministic; M = 0 returns
 * DG_OK without launching. Asynchronous on `stream`, allocates nothing.
 */
dg_status dg_fp8_quantize_1x128(const void *X, int x_dtype, int64_t ldx,
                                void *Q, int64_t ldq,
                                float *S, int64_t s_stride_m, int64_t s_stride_kb,
                                int64_t M, int64_t K, void *stream);

/*
 * The quantiser over a gathered row order: output row r quantises row
 * src_rows[r] of X (device memory, int32 [M]); a source index outside
 * [0, x_rows) reads as a row of zeros, which gives codes 0 and scale 1 (the
 * padding rows of the contiguous MoE layout). With src_rows = token_of_row of
 * dg_moe_route_contiguous this quantises token activations straight into the
 * contiguous layout in one pass.
 *   X  [x_rows, K] fp32/bf16, row stride ldx;  Q, S as in dg_fp8_quantize_1x128, M output rows.
 * Errors as dg_fp8_quantize_1x128; also DG_ERR_NULL_POINTER for a NULL
 * src_rows when M > 0, DG_ERR_BAD_SHAPE for x_rows < 0.
 */
dg_status dg_fp8_quantize_1x128_gather(const void *X, int x_dtype, int64_t ldx, int64_t x_rows,
                                       const int32_t *src_rows,
                                       void *Q, int64_t ldq,
                                       float *S, int64_t s_stride_m, int64_t s_stride_kb,
                                       int64_t M, int64_t K, void *stream);

/*
 * MoE routing into the contiguous layout that dg_fp8_grouped_gemm_contiguous
 * takes: tokens regrouped by expert (lpnh.cn article, §5.3), each expert's
 * rows padded to a multiple of 128 (bhfrc.com article, §4.2), with the group
 * id and source token of every row (rkmt.cn walkthrough, §5.3).
 *   expert_of_token [T] int32 (device): top-1 expert of each token
 *   row_of_token    [T] int32 (written): the token's row, -1 if dropped
 *   expert_ids      [M_cap] int32 (written): expert of each row, -1 for padding
 *   token_of_row    [M_cap] int32 (written): source token of each row, -1 for padding
 *   layout          [G + 1] int32 (written): first row of each expert; layout[G] = rows used
 * Experts are laid out in ascending id order, tokens in ascending order
 * within an expert. A token whose id is outside [0, G) is dropped. Rows from
 * layout[G] to M_cap are padding, so the GEMM may run over all M_cap rows
 * (its blocks of padding rows are skipped) without reading layout[G] on the
 * host. Everything stays on the device: no synchronisation, capture-safe.
 * Deterministic (no atomics). One workgroup.
 * Constraints: 1 <= G <= 1024; M_cap % 128 == 0 and
 * M_cap >= dg_moe_contiguous_max_rows(T, G) (else DG_ERR_BAD_SHAPE); all
 * arrays 4-byte aligned and pairwise disjoint.
 */
dg_status dg_moe_route_contiguous(const int32_t *expert_of_token, int64_t T, int64_t G,
                                  int32_t *row_of_token, int32_t *expert_ids, int32_t *token_of_row,
                                  int32_t *layout, int64_t M_cap, void *stream);

/* Rows that always hold the padded layout of T tokens over G experts:
 * 128 * (ceil(T / 128) + min(G, T)). -1 for negative arguments. */
int64_t dg_moe_contiguous_max_rows(int64_t T, int64_t G);

/*
 * The way back from the contiguous layout: out[t, :] = D[row_of_token[t], :]
 * (bf16, bit copy), for t < T; a row index outside [0, d_rows) (a dropped
 * token) gives a row of zeros.
 *   D [d_rows, N] bf16, row stride ldd;  out [T, N] bf16, row stride ldo (written)
 * Constraints: N % 8 == 0; D and out 16-byte aligned, ldd and ldo multiples
 * of 8; out disjoint from D and row_of_token.
 */
dg_status dg_moe_unpermute(const void *D, int64_t ldd, int64_t d_rows,
                           const int32_t *row_of_token, int64_t T, int64_t N,
                           void *out, int64_t ldo, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_FP8_H */
