// kernels.hpp -- gfx950 kernels of the fine-grained block-scaled FP8 GEMM.
//
// D[m, n] = bf16( sum_kb sA[m, kb] * sB[n/128, kb] * P_kb[m, n] ),
// P_kb = the 128-wide K-block product of the e4m3 operands.
//
// Each K block (128 bytes of K) is exactly one v_mfma_f32_16x16x128_f8f6f4:
// the MFMA produces the block's fp32 partial from a zero accumulator, and the
// VALU folds it into the fp32 accumulator with the block's scale product
// (the two-level accumulation of the hotdry.top fine-grained scaling article;
// per-block scaling of lpnh.cn §2.3). The hardware's block-scaled MFMA takes
// power-of-two E8M0 scales per 32 K elements, which cannot represent arbitrary
// fp32 scales per 128, so promotion stays on the VALU.
//
// Operand orientation: the MFMA's "A" operand (16 rows of the output) is fed
// with 16 rows of B and its "B" operand with 16 rows of A, so every lane ends
// up with ONE row m of D (lane % 16) and four consecutive columns n
// (4 * (lane / 16) + r). One scale product per lane per K block, and an
// 8-byte store per 16x16 sub-tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

// Kernel arguments, packed once on the host after validation.
struct Params {
    const uint8_t *A;
    int64_t lda, a_stride_g;
    const float *sA;
    int64_t sa_m, sa_kb, sa_g;
    const uint8_t *B;
    int64_t ldb, b_stride_g;
    const float *sB;
    int64_t sb_nb, sb_kb, sb_g;
    uint16_t *D;
    int64_t ldd, d_stride_g;
    const int32_t *ids;       // contiguous layout: expert id per row
    const int32_t *masked_m;  // masked layout: valid rows per group
    int M;                    // dense M, contiguous M_total, masked M_max
    int N, K, G;
    int tiles_m, tiles_n, num_tiles;
};

// One e4m3 x e4m3 -> fp32 MFMA over a 16x16x128 block, C = 0 + A.B.
// Format selectors 0/0 = OCP e4m3 for both operands; zero scale operands make
// the compiler emit the plain (unscaled) v_mfma_f32_16x16x128_f8f6f4.
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i &a, const v8i &b)
{
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint2 pack_bf16x4(const v4f &v)
{
    uint2 r;
    r.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    r.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
    return r;
}

__device__ __forceinline__ v8i join(const uint4 &lo, const uint4 &hi)
{
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// ---------------------------------------------------------------------------
// LDS tile layout: a tile of R rows x 128 bytes (one K block), row-major, with
// the eight 16-byte chunks of each row XOR-permuted by swz(row). A 128-bit
// LDS read by 16 lanes of 16 consecutive rows at one logical chunk then hits
// 16 distinct 16-byte bank groups (and any 8 consecutive rows hit 8), and a
// 128-bit write of one row's 8 chunks by 8 lanes is conflict-free as well.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// 32 bytes of one row's K block for the MFMA operand of lane group lg.
__device__ __forceinline__ v8i lds_frag(const uint8_t *tile, int row, int lg)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(tile + lds_off(row, 2 * lg));
    const uint4 hi = *reinterpret_cast<const uint4 *>(tile + lds_off(row, 2 * lg + 1));
    return join(lo, hi);
}

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kGroupM = 8;     // tile-order super-row height (L2 reuse)

// Tile index -> (m tile, n tile): runs of kGroupM m-tiles are walked m-first,
// so any window of consecutive tile indices is close to square in (m, n).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int &mt, int &nt)
{
    const int per_group = kGroupM * tiles_n;
    const int group = t / per_group;
    const int within = t - group * per_group;
    const int first_m = group * kGroupM;
    const int gm = min(kGroupM, tiles_m - first_m);
    mt = first_m + within % gm;
    nt = within / gm;
}

// Workgroups are dispatched round-robin over the 8 XCDs. Renumber them so each
// XCD owns a contiguous range of the persistent grid, i.e. a compact window
// of tiles that share operand rows in that XCD's L2.
__device__ __forceinline__ int xcd_local_id(int b, int grid)
{
    if ((grid & 7) != 0)
        return b;
    return (b & 7) * (grid >> 3) + (b >> 3);
}

template <int BM, int BN>
struct TileSmem {
    uint8_t a[2][BM * 128];
    uint8_t b[2][BN * 128];
    float sa[2][BM];
};

// Persistent, LDS double-buffered tile kernel. Workgroup tile BM x BN, 2x2
// waves, each wave a (BM/2) x (BN/2) block of 16x16 MFMA sub-tiles.
template <int L, int BM, int BN>
__global__ void __launch_bounds__(kThreads) tile_kernel(Params p)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 16, NJ = WN / 16;
    constexpr int LA = BM * 8 / kThreads;  // 16-byte chunks per thread per K block
    constexpr int LB = BN * 8 / kThreads;
    static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
    static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "tile loads");
    static_assert(WN <= 128 && (128 % WN) == 0, "a wave's columns share one sB block");
    static_assert(L != kContiguous || (128 % BM) == 0, "contiguous tiles stay inside one 128-row block");

    __shared__ __attribute__((aligned(16))) TileSmem<BM, BN> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
    const int nk = p.K >> 7;
    const int tiles_per_group = p.tiles_m * p.tiles_n;

    for (int t = xcd_local_id(blockIdx.x, gridDim.x); t < p.num_tiles; t += gridDim.x) {
        int g = 0, mt, nt;
        if (L == kMasked) {
            g = t / tiles_per_group;
            tile_coords(t - g * tiles_per_group, p.tiles_m, p.tiles_n, mt, nt);
        } else {
            tile_coords(t, p.tiles_m, p.tiles_n, mt, nt);
        }
        const int m0 = mt * BM, n0 = nt * BN;

        int rows;        // rows of this tile that are loaded (others read as 0)
        int limit = 0;   // masked: valid rows of the group
        int expert = 0;  // group whose B/sB this tile uses
        if (L == kDense) {
            rows = min(BM, p.M - m0);
        } else if (L == kMasked) {
            limit = min(max(p.masked_m[g], 0), p.M);
            if (m0 >= limit)
                continue;  // uniform over the workgroup
            rows = min(BM, limit - m0);
            expert = g;
        } else {
            // Expert of the aligned 128-row block: the largest valid id in it.
            const int blk0 = m0 & ~127;
            int e0 = p.ids[blk0 + lane], e1 = p.ids[blk0 + 64 + lane];
            e0 = (e0 >= 0 && e0 < p.G) ? e0 : -1;
            e1 = (e1 >= 0 && e1 < p.G) ? e1 : -1;
            int e = max(e0, e1);
            for (int o = 32; o > 0; o >>= 1)
                e = max(e, __shfl_xor(e, o));
            if (e < 0)
                continue;
            expert = e;
            rows = BM;
        }

        const uint8_t *Ab = p.A + (int64_t)g * p.a_stride_g + (int64_t)m0 * p.lda;
        const uint8_t *Bb = p.B + (int64_t)expert * p.b_stride_g + (int64_t)n0 * p.ldb;
        const float *sAb = p.sA + (int64_t)g * p.sa_g + (int64_t)m0 * p.sa_m;
        const float *sBw = p.sB + (int64_t)expert * p.sb_g + (int64_t)((n0 + wn0) >> 7) * p.sb_nb;

        uint4 ra[LA], rb[LB];
        float rsa = 0.f;

        auto load_stage = [&](int kb) {
#pragma unroll
            for (int q = 0; q < LA; ++q) {
                const int c = q * kThreads + tid, row = c >> 3, ch = c & 7;
                if (row < rows)
                    ra[q] = *reinterpret_cast<const uint4 *>(Ab + (int64_t)row * p.lda + kb * 128 + ch * 16);
                else
                    ra[q] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < LB; ++q) {
                const int c = q * kThreads + tid, row = c >> 3, ch = c & 7;
                rb[q] = *reinterpret_cast<const uint4 *>(Bb + (int64_t)row * p.ldb + kb * 128 + ch * 16);
            }
            if (tid < BM)
                rsa = (tid < rows) ? sAb[(int64_t)tid * p.sa_m + (int64_t)kb * p.sa_kb] : 0.f;
        };
        auto store_stage = [&](int s) {
#pragma unroll
            for (int q = 0; q < LA; ++q) {
                const int c = q * kThreads + tid, row = c >> 3, ch = c & 7;
                *reinterpret_cast<uint4 *>(&sm.a[s][lds_off(row, ch)]) = ra[q];
            }
#pragma unroll
            for (int q = 0; q < LB; ++q) {
                const int c = q * kThreads + tid, row = c >> 3, ch = c & 7;
                *reinterpret_cast<uint4 *>(&sm.b[s][lds_off(row, ch)]) = rb[q];
            }
            if (tid < BM)
                sm.sa[s][tid] = rsa;
        };

        v4f acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        __syncthreads();  // the previous tile's LDS reads are complete
        load_stage(0);
        float sb_cur = sBw[0];
        store_stage(0);
        __syncthreads();

        for (int kb = 0; kb < nk; ++kb) {
            const int cur = kb & 1;
            const bool more = kb + 1 < nk;
            float sb_next = 0.f;
            if (more) {
                load_stage(kb + 1);
                sb_next = sBw[(int64_t)(kb + 1) * p.sb_kb];
            }
            v8i bf[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                bf[j] = lds_frag(sm.b[cur], wn0 + 16 * j + l16, lg);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm0 + 16 * i + l16;
                const v8i af = lds_frag(sm.a[cur], row, lg);
                const float s = sm.sa[cur][row] * sb_cur;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const v4f part = mfma_e4m3_16x16x128(bf[j], af);
                    acc[i][j] += part * s;
                }
            }
            if (more)
                store_stage(cur ^ 1);
            sb_cur = sb_next;
            __syncthreads();
        }

        uint16_t *Dg = p.D + (int64_t)g * p.d_stride_g;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int m = m0 + wm0 + 16 * i + l16;
            bool ok;
            if (L == kDense)
                ok = m < p.M;
            else if (L == kMasked)
                ok = m < limit;
            else
                ok = p.ids[m] == expert;
            if (!ok)
                continue;
            uint16_t *drow = Dg + (int64_t)m * p.ldd + n0 + wn0 + 4 * lg;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                *reinterpret_cast<uint2 *>(drow + 16 * j) = pack_bf16x4(acc[i][j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel (decode shapes, M <= 16 * MT). One workgroup per 16 rows of
// B; its four waves split the K blocks, read B straight from HBM into MFMA
// operand registers (B is streamed exactly once, no LDS staging), and reduce
// their fp32 accumulators through LDS at the end.
constexpr int kDecodeUnroll = 8;  // K blocks whose loads are issued together

template <int MT>
__global__ void __launch_bounds__(kThreads) decode_kernel(Params p)
{
    __shared__ v4f red[4][MT][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nk = p.K >> 7;
    const int kb_begin = (wave * nk) >> 2, kb_end = ((wave + 1) * nk) >> 2;

    const uint8_t *brow = p.B + (int64_t)(n0 + l16) * p.ldb + 32 * lg;
    const float *sbp = p.sB + (int64_t)(n0 >> 7) * p.sb_nb;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kDecodeUnroll) {
        v8i bf[kDecodeUnroll];
        v8i af[kDecodeUnroll][MT];
        float sb[kDecodeUnroll];
        float sa[kDecodeUnroll][MT];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int kb = kb0 + u;
            if (kb < kb_end) {
                const uint4 *src = reinterpret_cast<const uint4 *>(brow + (int64_t)kb * 128);
                bf[u] = join(src[0], src[1]);
                sb[u] = sbp[(int64_t)kb * p.sb_kb];
            }
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int kb = kb0 + u;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + l16;
                if (kb < kb_end && m < p.M) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(p.A + (int64_t)m * p.lda + (int64_t)kb * 128 + 32 * lg);
                    af[u][mt] = join(src[0], src[1]);
                    sa[u][mt] = p.sA[(int64_t)m * p.sa_m + (int64_t)kb * p.sa_kb];
                } else {
                    af[u][mt] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    sa[u][mt] = 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            if (kb0 + u < kb_end) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const v4f part = mfma_e4m3_16x16x128(bf[u], af[u][mt]);
                    acc[mt] += part * (sa[u][mt] * sb[u]);
                }
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        red[wave][mt][lane] = acc[mt];
    __syncthreads();
    // Wave w finishes m-subtiles mt = w, w + 4, ... in a fixed order (deterministic).
    for (int mt = wave; mt < MT; mt += 4) {
        const v4f v = ((red[0][mt][lane] + red[1][mt][lane]) + red[2][mt][lane]) + red[3][mt][lane];
        const int m = mt * 16 + l16;
        if (m < p.M)
            *reinterpret_cast<uint2 *>(p.D + (int64_t)m * p.ldd + n0 + 4 * lg) = pack_bf16x4(v);
    }
}

}  // namespace dgk
