// quant.hpp -- gfx950 kernel of the 1x128 activation quantiser, the step that
// turns activations into the GEMM's LHS codes and scales.
//
// Per row m and 128-wide K block kb (one scale per 1x128 tile: hotdry.top
// fine-grained scaling article, "fine-grained scaling core design"):
//   amax = max |x| over the block,
//   s    = amax / 448 (fp32 division; the initial scale max_val / 448 of the
//          rkmt.cn walkthrough, §5.2), or 1 for an all-zero block,
//   q    = e4m3(clamp(x / s, -448, 448)), x / s an fp32 division, rounded to
//          the nearest code with ties to even (lpnh.cn article, §6.3).
//
// The work is a single pass over HBM (read x once, write codes and scales
// once) with a 128-element reduction per block, so the kernel is shaped for
// streaming, not for the matrix cores:
//   - one wave owns a span of consecutive blocks of one row, in groups of 8
//     blocks; 8 lanes (half a DPP row) hold one block, 16 elements per lane.
//     The block's amax is taken on the integer bit patterns of |x| (which
//     order like the values) with three DPP max steps; no LDS is used. All of
//     a wave's loads are in flight before the first block is reduced.
//     Lane i of a block holds elements 8i..8i+7 and 64+8i..64+8i+7 (bf16,
//     two 16-byte loads) or 4i+32t..4i+32t+3 for t = 0..3 (fp32, four
//     16-byte loads), so every load instruction reads eight whole 128-byte
//     lines;
//   - an IEEE fp32 division per element (x / s) would cost about 10 VALU
//     instructions and make the kernel VALU-bound. Instead each block
//     computes r = 1/s correctly rounded (one division per block) and its
//     residual r_lo = (1 - s r) r, and each element takes
//       q0 = fma(x, r, x r_lo)          (faithful: within one ulp of x/s)
//       q  = fma(fma(-q0, s, x), r, q0) (Markstein's correction step)
//     which is the correctly rounded x / s whenever no intermediate
//     underflows (Markstein's theorem on division with a correctly rounded
//     reciprocal; also checked against IEEE division on 2.5e9 pairs). The
//     sign is copied from x so that -0 stays -0. Quotients below 2^-12 may
//     differ from the IEEE ones by an ulp when they underflow, but every
//     value below 2^-11 encodes to a signed zero either way. Blocks with
//     s < 2^-64 (amax < 2^-55) take the plain division;
//   - the e4m3 conversion is the hardware's round-to-nearest-even packed
//     conversion (v_cvt_pk_fp8_f32, OCP e4m3 on gfx950), after the clamp, so
//     it never sees a value outside +-448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgq {

struct QuantParams {
    const void *X;   // fp32 or bf16 [x_rows, K], row stride ldx elements
    int64_t ldx;
    const int32_t *src_rows;  // output row r quantises X[src_rows[r]] (NULL: X[r]);
    int64_t x_rows;           // a source row outside [0, x_rows) reads as zeros
    uint8_t *Q;      // e4m3 codes [M, K], row stride ldq bytes
    int64_t ldq;
    float *S;        // S[m, kb] at S[m * s_m + kb * s_kb]
    int64_t s_m, s_kb;
    int M, K;
    int spans;       // spans per row: ceil(K / (1024 * groups per wave))
    int64_t units;   // M * spans: one wave each
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerGroup = 4;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// DPP lane permutes inside a row of 16 lanes (GFX9 DPP control codes).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over each group of 8 lanes: swap neighbours, swap pairs (quad
// permutes [1,0,3,2] and [2,3,0,1]), then mirror the half-row (lane i sees
// 7 - i, the other quad).
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v)
{
    v = max(v, dpp<0xB1>(v));
    v = max(v, dpp<0x4E>(v));
    return max(v, dpp<0x141>(v));
}

// Correctly rounded x / s for a block whose s >= 2^-64 (see above).
__device__ __forceinline__ float quotient(float x, float s, float r, float r_lo)
{
    const float q0 = __builtin_fmaf(x, r, x * r_lo);
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
    return __builtin_copysignf(q, x);
}

// Groups of 8 blocks per wave. One group per wave measured fastest for both
// input types on 8192 x 7168 (more groups per wave keep more bytes in flight
// per wave but leave fewer waves to hide the VALU work).
template <bool BF16>
constexpr int groups_per_wave() { return 1; }

template <bool BF16>
__global__ __launch_bounds__(64 * kWavesPerGroup) void quantize_1x128_kernel(QuantParams p)
{
    constexpr int G = groups_per_wave<BF16>();
    constexpr int NL = BF16 ? 2 : 4;      // 16-byte loads per lane and block
    constexpr int EL = BF16 ? 8 : 4;      // elements per load
    const int lane = threadIdx.x & 63;
    // Workgroups are dealt to the 8 XCDs in turn. For bf16 input they are
    // renumbered so that each XCD takes one contiguous range of rows: the
    // M-major scales of 32 consecutive rows share a 128-byte line, which then
    // fills in one XCD's L2 instead of being written back in pieces from
    // several (8192 x 7168: 11 MB of extra writes gone, 35.7 -> 32.9 us). For
    // fp32 input, whose time is mostly the input read, the hardware order
    // measured faster (53 against 56.5 us) despite those extra writes.
    const int nwg = gridDim.x, xcd = blockIdx.x % 8, per = nwg / 8, extra = nwg % 8;
    const int wg = BF16 ? xcd * per + min(xcd, extra) + (int)blockIdx.x / 8 : (int)blockIdx.x;
    const int64_t unit = (int64_t)wg * kWavesPerGroup + (threadIdx.x >> 6);
    if (unit >= p.units)
        return;
    // row and span are the same for every lane of the wave: keep them (and the
    // source-row lookup) in scalar registers
    const int row = __builtin_amdgcn_readfirstlane((int)(unit / p.spans));
    const int span = __builtin_amdgcn_readfirstlane((int)(unit - (int64_t)row * p.spans));
    const int64_t src = p.src_rows ? (int64_t)p.src_rows[row] : (int64_t)row;
    const bool present = src >= 0 && src < p.x_rows;
    const int nkb = p.K >> 7;
    const int sub = lane & 7;
    auto offset = [&](int t) { return BF16 ? 8 * sub + 64 * t : 4 * sub + 32 * t; };

    // Every load is issued unconditionally (a block past the row's end reads
    // the row's last block instead, and its results are not stored), so the
    // compiler issues all of a wave's loads before the first wait.
    float x[G][NL * EL];
    if (present) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int kb = min(span * 8 * G + 8 * g + (lane >> 3), nkb - 1);
            const int64_t base = src * p.ldx + kb * 128;
#pragma unroll
            for (int t = 0; t < NL; ++t) {
                if (BF16) {
                    const u32x4 v =
                        __builtin_nontemporal_load((const u32x4 *)((const uint16_t *)p.X + base + offset(t)));
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        x[g][EL * t + 2 * c] = bf16_to_f32(v[c] & 0xffffu);
                        x[g][EL * t + 2 * c + 1] = bf16_to_f32(v[c] >> 16);
                    }
                } else {
                    const f32x4 v =
                        __builtin_nontemporal_load((const f32x4 *)((const float *)p.X + base + offset(t)));
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        x[g][EL * t + c] = v[c];
                }
            }
        }
    } else {  // a padding row of a gathered layout: zeros, so codes 0 and scale 1
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NL * EL; ++c)
                x[g][c] = 0.0f;
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int kb = span * 8 * G + 8 * g + (lane >> 3);
        uint32_t abits = 0;
#pragma unroll
        for (int c = 0; c < NL * EL; ++c)
            abits = max(abits, __float_as_uint(x[g][c]) & 0x7fffffffu);
        const float amax = __uint_as_float(max_over_8_lanes(abits));
        const float s = amax == 0.0f ? 1.0f : amax / kE4m3Max;
        float q[NL * EL];
        if (s >= 0x1p-64f) {
            const float r = 1.0f / s;
            const float r_lo = __builtin_fmaf(-s, r, 1.0f) * r;
#pragma unroll
            for (int c = 0; c < NL * EL; ++c)
                q[c] = quotient(x[g][c], s, r, r_lo);
        } else {
#pragma unroll
            for (int c = 0; c < NL * EL; ++c)
                q[c] = x[g][c] / s;
        }
        uint32_t w[NL * EL / 4];
#pragma unroll
        for (int h = 0; h < NL * EL / 4; ++h) {
            float v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[c] = fminf(fmaxf(q[4 * h + c], -kE4m3Max), kE4m3Max);
            int packed = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
            w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], packed, true);
        }
        if (kb < nkb) {
            uint8_t *qblk = p.Q + (int64_t)row * p.ldq + kb * 128;
#pragma unroll
            for (int t = 0; t < NL; ++t) {
                if (BF16)
                    *(u32x2 *)(qblk + offset(t)) = u32x2{w[2 * t], w[2 * t + 1]};
                else
                    *(uint32_t *)(qblk + offset(t)) = w[t];
            }
            if (sub == 0)
                p.S[(int64_t)row * p.s_m + (int64_t)kb * p.s_kb] = s;
        }
    }
}

}  // namespace dgq
