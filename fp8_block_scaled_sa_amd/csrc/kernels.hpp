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
//
// K order inside a block: lane group lg = lane / 16 hands the MFMA bytes
// [16 lg, 16 lg + 16) and [64 + 16 lg, 64 + 16 lg + 16) of the block, for A
// and B alike. The MFMA sums over all 128 positions, so any permutation of K
// that is the same for both operands gives the same dot product; this one
// makes each 16-lane group of a load instruction read 64 contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
    // Dense split-K: each tile's K blocks are split over ksplit work items,
    // which write fp32 partials to ws[ksplit][M][N]; splitk_reduce_kernel
    // adds them in slice order. ksplit <= 1: no split, bf16 written directly.
    int ksplit;
    float *ws;
    // Contiguous layout written straight to token order: row m of the
    // result goes to row row_dst[m] of D, for 0 <= row_dst[m] < dst_rows.
    const int32_t *row_dst;
    int dst_rows;
    // Contiguous layout with segment offsets: layout[e] is the first row of
    // expert e's segment (a multiple of 128 rows), layout[G] the rows used.
    const int32_t *layout;
    // Segment tiles to run: 0 all, 1 the whole 256-row tiles only, 2 the
    // 128-row tails only, each split over K (at most ksplit slices, chosen by
    // tail_split for tail_slots workgroups) into work items whose fp32
    // partials go to ws[slice][128 * tail + row][N] (ws_rows rows per slice).
    int seg_mode;
    int ws_rows;
    int tail_slots;
    // Contiguous layout on the uniform grid: when set, the launch does
    // nothing unless *gate != 0 (segment offsets derived on the device were
    // not usable, so this launch covers the rows instead).
    const int32_t *gate;
};

// One e4m3 x e4m3 -> fp32 MFMA over a 16x16x128 block, C = 0 + A.B.
// Format selectors 0/0 = OCP e4m3 for both operands; zero scale operands make
// the compiler emit the plain (unscaled) v_mfma_f32_16x16x128_f8f6f4.
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i &a, const v8i &b)
{
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Operand formats of the tile kernel: bit 0 set = the GEMM's A holds e5m2,
// bit 1 set = B holds e5m2 (else e4m3). The MFMA takes them as its format
// selectors (0 = e4m3, 1 = e5m2): the first MFMA operand is fed from B, the
// second from A (see the orientation above).
template <int F>
__device__ __forceinline__ v4f mfma_fmt_16x16x128(const v8i &b_rows, const v8i &a_rows)
{
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, zero, (F >> 1) & 1, F & 1, 0, 0, 0, 0);
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
// Low-level pieces of the LDS pipeline.
//
// Operand tiles are copied HBM -> LDS with gfx950's LDS-DMA loads
// (global_load_lds_dwordx4 / _dword): each lane names a global address and
// the data lands at M0 + 16 * lane (4 * lane for the dword form), bypassing
// VGPRs. They are issued through inline asm, together with the waits and the
// barrier, so that the compiler neither serialises them (it would wait for
// every outstanding DMA before each LDS read) nor fences the barrier (HIP's
// __syncthreads waits for all outstanding loads). The pipeline tracks
// completion itself with vmcnt: vector loads of a wave complete in issue
// order, so "at most n outstanding" means everything but the last n issued
// has landed.

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from base + voff into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma_b128(const void *base, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory", "m0");
}

// 4 bytes per lane from base + voff into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma_b32(const void *base, uint32_t voff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(m0)
                 : "memory", "m0");
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Buffer resource (V#) for raw byte addressing of [base, base + bytes):
// lanes whose offset lies past `bytes` read zeros instead of memory.
__device__ __forceinline__ v4i buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    v4i r;
    r[0] = (int)(uint32_t)b;
    r[1] = (int)((uint32_t)(b >> 32) & 0xffffu);  // stride 0
    r[2] = (int)bytes;
    r[3] = 0x00020000;                             // 32-bit data format, raw access
    return r;
}

// 16 bytes per lane from rsrc at voff + soff into LDS at m0 + 16 * lane;
// out-of-range lanes deliver zeros.
__device__ __forceinline__ void dma_buf_b128(const v4i &rsrc, uint32_t voff, uint32_t soff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "s"(m0)
                 : "memory", "m0");
}

// The same with the non-temporal hint, for data read once: it is not kept in
// L2 at the expense of data that is re-read (another tile's operand rows).
__device__ __forceinline__ void dma_buf_b128_nt(const v4i &rsrc, uint32_t voff, uint32_t soff, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(rsrc),
                 "s"(soff), "s"(m0)
                 : "memory", "m0");
}

// v + s, computed where it is written: the compiler cannot hoist it out of
// the K loop, so the per-segment DMA offsets are not all kept live in VGPRs
// (one add per copy instead of one VGPR per segment).
__device__ __forceinline__ uint32_t add_in_place(uint32_t v, uint32_t s)
{
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(s), "v"(v));
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS tile layout: R rows x 128 bytes (one K block), row-major, with the
// eight 16-byte chunks of each row XOR-permuted by swz(row) = row & 6.
//
// gfx950's LDS serves a 128-bit access in four passes of 16 consecutive
// lanes; a pass is conflict-free when its 16 lanes hit 16 distinct 16-byte
// bank groups, and the bank group of address a is ((a >> 4) ^ (a >> 10)) & 15
// (64 four-byte banks, with address bits 10+ hashed in; fitted to
// SQ_LDS_BANK_CONFLICT measurements of twelve access patterns). An MFMA
// fragment read has one pass read 16 consecutive rows at one logical chunk.
// With the row-dependent XOR confined to bits 1-2 of the chunk, the 16 rows
// land on 16 distinct groups for any 1 KB-aligned tile base, and the DMA's
// 1 KB contiguous writes are conflict-free as well.
__device__ __forceinline__ int swz(int row) { return row & 6; }

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// The 32 operand bytes of lane group lg for one tile row: chunks lg and lg+4.
__device__ __forceinline__ v8i lds_frag(const uint8_t *tile, int row, int lg)
{
    const uint4 lo = *reinterpret_cast<const uint4 *>(tile + lds_off(row, lg));
    const uint4 hi = *reinterpret_cast<const uint4 *>(tile + lds_off(row, lg + 4));
    return join(lo, hi);
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

// Tile index -> (m tile, n tile): runs of group_m m-tiles are walked m-first,
// so any window of consecutive tile indices is close to square in (m, n).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int &mt, int &nt)
{
    const int per_group = group_m * tiles_n;
    const int group = t / per_group;
    const int within = t - group * per_group;
    const int first_m = group * group_m;
    const int gm = min(group_m, tiles_m - first_m);
    mt = first_m + within % gm;
    nt = within / gm;
}

// ---------------------------------------------------------------------------
// Persistent, multi-stage LDS-DMA pipelined tile kernel.
//
// Workgroup tile BM x BN (BN a multiple of 128 is not required, but a wave's
// columns must lie in one 128-wide sB block), WAVES_M x WAVES_N waves, each
// owning a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 sub-tiles. STAGES LDS
// buffers, each holding one K block of the A tile, the B tile and sA.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int GROUP_M, bool STREAM_B = false,
          bool EARLY_B = false>
struct TileCfg {
    // B rows are read once per launch (each group's B feeds a single M tile):
    // load them non-temporally.
    static constexpr bool kStreamB = STREAM_B;
    // Two stages only: every wave holds all of its B fragments of a K block in
    // registers from row 0 on, so the B half of a stage is free once every
    // wave is past row 0. A second barrier there lets the copy of B for block
    // k + 2 start during block k, about one block earlier than the A copy of
    // the same stage: B, the operand streamed from HBM in the grouped
    // layouts, gets about two blocks of lead instead of one.
    static constexpr bool kEarlyB = EARLY_B;
    static constexpr int kBM = BM, kBN = BN, kStages = STAGES, kGroupM = GROUP_M;
    static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N;
    static constexpr int kWaves = WAVES_M * WAVES_N;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kWM = BM / WAVES_M, kWN = BN / WAVES_N;
    static constexpr int kMI = kWM / 16, kNJ = kWN / 16;
    static constexpr int kSegA = BM / 8, kSegB = BN / 8;     // 1 KB LDS segments (8 rows)
    static constexpr int kSegPerWave = (kSegA + kSegB) / kWaves;
    static constexpr int kSaLoads = BM / 64;                  // dword DMA instructions for sA
    static constexpr int kOffB = BM * 128, kOffSa = kOffB + BN * 128, kOffSb = kOffSa + BM * 4;
    static constexpr int kStageBytes = (kOffSb + 256 + 1023) / 1024 * 1024;  // + 64 sB slots; 1 KB aligned
    static constexpr int kNB = BN / 128;                    // sB blocks per tile
    static constexpr int kSmemBytes = STAGES * kStageBytes;
    // With two stages every wave waits for all of its DMA before each
    // barrier, so which waves issue the copies is free. The operand DMA then
    // goes to the upper half of the waves: each SIMD's lower (older, issued
    // first) wave starts its MFMAs right after the barrier, and the copies'
    // issue stalls land on the wave that would otherwise wait for it there.
    static constexpr bool kDmaUpper = STAGES == 2 && ((BM + BN) / 8) % (WAVES_M * WAVES_N / 2) == 0;
    static constexpr int kDmaWaves = kDmaUpper ? WAVES_M * WAVES_N / 2 : WAVES_M * WAVES_N;  // waves issuing copies
    static constexpr int kDmaQ = ((BM + BN) / 8) / kDmaWaves;  // 1 KB segments per issuing wave
    static constexpr int kDmaQA = (BM / 8) / kDmaWaves;        // of which A segments
    static_assert((BM / 8) % kDmaWaves == 0, "A and B segments split evenly over the issuing waves");
    static_assert(kWM % 16 == 0 && kWN % 16 == 0, "wave tile");
    static_assert((kSegA + kSegB) % kWaves == 0, "segments split evenly over waves");
    static_assert(BM % 64 == 0 && kSaLoads <= kWaves, "sA loads");
    static_assert(kWN <= 128 && (128 % kWN) == 0, "a wave's columns share one sB block");
    static_assert(BN % 128 == 0, "tile columns cover whole sB blocks");
    static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth (the K loop is unrolled by at most 4)");
    static_assert(kSmemBytes <= 160 * 1024, "LDS");
    static_assert(!EARLY_B || (STAGES == 2 && kDmaUpper), "early B copies: two stages, copies on the upper waves");
    static_assert((kSegPerWave + 2) * (STAGES - 2) < 64, "vmcnt range");
};

// Wait until this wave's DMA for the oldest pipeline stage has landed: at most
// `later` stages of `per_stage` loads each may still be in flight.
template <int SEGW, int LATER>
__device__ __forceinline__ void wait_stage(int per_stage)
{
    if (per_stage == SEGW)
        wait_vmcnt<SEGW * LATER>();
    else if (per_stage == SEGW + 1)
        wait_vmcnt<(SEGW + 1) * LATER>();
    else
        wait_vmcnt<(SEGW + 2) * LATER>();
}

// K slices for `tiles` segment-tail tiles on `slots` workgroups: the count in
// 1..max_split with the lowest estimated time, the smaller on a tie. The
// estimate, in K-block times of one round: rounds x (K blocks per item + the
// fp32 partial-tile store) + the reduction's re-read of every slice (each
// about kTailSliceCost K blocks per round's worth of tiles). The tail kernel
// and its reduction both call it with the same values.
// 32-bit arithmetic: tiles < 2 x slots and max_split <= kMaxTailSplit.
constexpr int kTailSliceCost = 4;
constexpr int kMaxTailSplit = 8;

__device__ inline int tail_split(int tiles, int nk, int max_split, int slots)
{
    int best = 1;
    int best_cost = INT32_MAX;
    for (int k = 1; k <= max_split; ++k) {
        const int items = tiles * k;
        const int rounds = (items + slots - 1) / slots;
        const int cost = rounds * ((nk + k - 1) / k + kTailSliceCost) + (kTailSliceCost * items + slots - 1) / slots;
        if (cost < best_cost) {
            best = k;
            best_cost = cost;
        }
    }
    return best;
}

// Sum of v over the wave's 64 lanes, the same in every lane.
__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive prefix sum of v over lanes 0..lane.
__device__ __forceinline__ int wave_incl_sum(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d)
            v += u;
    }
    return v;
}

template <int L, class C, int F = 0, bool SCATTER = false, bool SEG = false>
__global__ void __launch_bounds__(C::kThreads, 1) tile_kernel(Params p)
{
    constexpr int BM = C::kBM, BN = C::kBN, S = C::kStages;
    constexpr int MI = C::kMI, NJ = C::kNJ;
    constexpr int SEGW = C::kSegPerWave;
    static_assert(L != kContiguous || BM <= 256, "contiguous tiles span at most two 128-row blocks");
    static_assert(L != kContiguous || C::kWM <= 128, "a wave's rows lie in one 128-row block");
    static_assert(L != kContiguous || BM == 256 || 128 % BM == 0, "contiguous tile rows");
    // SEG on 128-row tiles serves the tails-only launch (seg_mode 2)
    static_assert(!SEG || (L == kContiguous && (BM == 256 || BM == 128)), "segment tiles are 256 or 128 rows of one expert");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kSmemBytes];

    if constexpr (L == kContiguous && !SEG) {
        if (p.gate && *p.gate == 0)
            return;  // uniform over the grid
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int wm0 = (wave / C::kWavesN) * C::kWM;
    const int wn0 = (wave % C::kWavesN) * C::kWN;
    const int nk_all = p.K >> 7;
    const int tiles_per_group = p.tiles_m * p.tiles_n;
    const uint32_t smem_base = lds_addr(smem);
    const bool loads_sa = wave < C::kSaLoads;
    const bool loads_sb = wave == C::kWaves - 1;
    const int per_stage = SEGW + (loads_sa ? 1 : 0) + (loads_sb ? 1 : 0);  // DMA ops per stage

    // SEG: tiles follow the experts' segments, so that every tile holds rows
    // of one expert only: first the whole 256-row tiles of every segment
    // (expert by expert), then each segment's last 128 rows where its size is
    // an odd multiple of 128. full / half: how many of each.
    // A segment launch of whole tiles whose offsets were derived on the device
    // covers the rows block by block instead when the derivation found the
    // experts out of order (*gate != 0; the offsets are then all zero): every
    // aligned 128-row block is a tile of its own, half of the workgroup's
    // rows, with the block's expert taken from the ids as on the uniform grid.
    const bool by_block = SEG && p.seg_mode != 2 && p.gate && *p.gate != 0;
    const int num_tiles = by_block ? (p.M >> 7) * p.tiles_n : p.num_tiles;
    // Expert of an aligned 128-row block: the largest valid id in it (-1 if it
    // holds padding only or lies past M_total).
    auto block_expert = [&](int blk0) {
        if (blk0 >= p.M)
            return -1;
        int e0 = p.ids[blk0 + lane], e1 = p.ids[blk0 + 64 + lane];
        e0 = (e0 >= 0 && e0 < p.G) ? e0 : -1;
        e1 = (e1 >= 0 && e1 < p.G) ? e1 : -1;
        int e = max(e0, e1);
        for (int o = 32; o > 0; o >>= 1)
            e = max(e, __shfl_xor(e, o));
        return __builtin_amdgcn_readfirstlane(e);
    };
    // The segments are read 64 experts at a time, one per lane (a loop over
    // the experts on the scalar unit would wait for each offset in turn).
    // Round e0: lane e0 + lane's segment start and size (0 past G).
    auto seg_of_lane = [&](int e0, int &start, int &size) {
        const int e = e0 + lane;
        start = 0;
        size = 0;
        if (e < p.G) {
            start = p.layout[e];
            size = max(p.layout[e + 1] - start, 0);
        }
    };
    int seg_full = 0, seg_half = 0;
    if (SEG && !by_block) {
        for (int e0 = 0; e0 < p.G; e0 += 64) {
            int st, sz;
            seg_of_lane(e0, st, sz);
            seg_full += wave_sum(sz >> 8);
            seg_half += wave_sum((sz >> 7) & 1);
        }
    }
    // K slices per work item; segment tails write every slice to the workspace
    const bool to_ws = (L == kDense && p.ksplit > 1) || (SEG && p.seg_mode == 2);
    const int ks = L == kDense ? max(p.ksplit, 1)
                               : (SEG && p.seg_mode == 2 ? tail_split(seg_half * p.tiles_n, nk_all, p.ksplit, p.tail_slots) : 1);

    for (int t = xcd_local_id(blockIdx.x, gridDim.x); t < num_tiles; t += gridDim.x) {
        int g = 0, mt, nt;
        // split-K: work item t is K slice t % ks of tile t / ks
        const int slice = t % ks;
        const int kb_lo = (int)((int64_t)slice * nk_all / ks);
        const int nk = (int)((int64_t)(slice + 1) * nk_all / ks) - kb_lo;  // K blocks of this item
        int seg_m0 = 0, seg_rows = 0, seg_e = 0, seg_h = 0;
        if (SEG && by_block) {
            mt = 0;
            int blk;
            tile_coords(t, p.M >> 7, p.tiles_n, C::kGroupM, blk, nt);
            seg_m0 = 128 * blk;
            seg_rows = 128;
            seg_e = block_expert(seg_m0);
            if (seg_e < 0)
                continue;  // padding only (uniform over the workgroup)
        } else if (SEG) {
            mt = 0;
            // tails-only mode numbers its items from 0 after the whole tiles
            const int ts = p.seg_mode == 2 ? seg_full * p.tiles_n + t / ks : t;
            if ((p.seg_mode == 1 && ts >= seg_full * p.tiles_n) || (BM == 128 && ts < seg_full * p.tiles_n))
                continue;
            if (ts < seg_full * p.tiles_n) {
                int ft;
                tile_coords(ts, seg_full, p.tiles_n, C::kGroupM, ft, nt);
                // the expert whose whole tiles hold tile ft: the first one where
                // the running count of whole tiles passes ft
                int before = 0;  // whole tiles of the experts before this round
                seg_e = -1;
                for (int e0 = 0; e0 < p.G; e0 += 64) {
                    int st, sz;
                    seg_of_lane(e0, st, sz);
                    const int f = sz >> 8, incl = wave_incl_sum(f, lane);
                    const uint64_t hit = __ballot(ft < before + incl);
                    if (hit) {
                        const int l = (int)__builtin_ctzll(hit);
                        seg_e = e0 + l;
                        seg_m0 = __builtin_amdgcn_readfirstlane(__shfl(st + 256 * (ft - before - (incl - f)), l));
                        break;
                    }
                    before += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
                }
                if (seg_e < 0)
                    continue;  // past the segments (uniform over the workgroup)
                seg_rows = 256;
            } else {
                const int h = (ts - seg_full * p.tiles_n) / p.tiles_n;
                if (h >= seg_half)
                    continue;  // past the real tiles (uniform over the workgroup)
                nt = ts - seg_full * p.tiles_n - h * p.tiles_n;
                seg_h = h;
                // the expert of the h-th tail: the h-th segment (in expert
                // order) whose size is an odd multiple of 128
                int seen = 0;
                seg_e = -1;
                for (int e0 = 0; e0 < p.G; e0 += 64) {
                    int st, sz;
                    seg_of_lane(e0, st, sz);
                    const bool tail = (sz >> 7) & 1;
                    const uint64_t tails = __ballot(tail);
                    const int n = __popcll(tails);
                    if (h < seen + n) {
                        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(tails >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)tails, 0));
                        const int l = (int)__builtin_ctzll(__ballot(tail && below == h - seen));
                        seg_e = e0 + l;
                        seg_m0 = __builtin_amdgcn_readfirstlane(__shfl(st + (sz & ~255), l));
                        break;
                    }
                    seen += n;
                }
                if (seg_e < 0)
                    continue;
                seg_rows = 128;
            }
            if (seg_m0 < 0 || seg_m0 >= p.M)
                continue;  // a layout that does not fit the rows: nothing to do
        } else if (L == kMasked) {
            g = t / tiles_per_group;
            tile_coords(t - g * tiles_per_group, p.tiles_m, p.tiles_n, C::kGroupM, mt, nt);
        } else {
            tile_coords(t / ks, p.tiles_m, p.tiles_n, C::kGroupM, mt, nt);
        }
        const int m0 = SEG ? seg_m0 : mt * BM, n0 = nt * BN;

        int rows;        // valid rows of this tile (the rest re-read the last valid row)
        int limit = 0;   // masked: valid rows of the group
        int npass = 1;   // contiguous: one K loop per expert met in the tile
        int ex0 = 0, ex1 = 0;  // contiguous: expert of the tile's first / second 128-row block
        if (L == kDense) {
            rows = min(BM, p.M - m0);
        } else if (L == kMasked) {
            limit = min(max(p.masked_m[g], 0), p.M);
            if (m0 >= limit)
                continue;  // uniform over the workgroup
            rows = min(BM, limit - m0);
        } else if (SEG) {
            ex0 = ex1 = seg_e;
            rows = min(seg_rows, p.M - m0);
        } else {
            ex0 = block_expert(m0 & ~127);
            ex1 = BM > 128 ? block_expert(m0 + 128) : ex0;
            if (ex0 < 0 && ex1 < 0)
                continue;
            // Blocks of two experts (a segment boundary) take two passes,
            // each computing the half of its own expert; a padding-only half
            // takes none.
            if (ex0 != ex1 && ex0 >= 0 && ex1 >= 0)
                npass = 2;
            else if (ex0 < 0)
                ex0 = ex1;
            else
                ex1 = ex0;
            rows = min(BM, p.M - m0);
        }

        for (int pass = 0; pass < npass; ++pass) {
        int expert = 0;  // group whose B/sB this pass uses
        if (L == kMasked)
            expert = g;
        else if (L == kContiguous)
            expert = pass == 0 ? ex0 : ex1;

        const uint8_t *Ab = p.A + (int64_t)g * p.a_stride_g + (int64_t)m0 * p.lda + (int64_t)kb_lo * 128;
        const uint8_t *Bb = p.B + (int64_t)expert * p.b_stride_g + (int64_t)n0 * p.ldb + (int64_t)kb_lo * 128;
        const float *sAb = p.sA + (int64_t)g * p.sa_g + (int64_t)m0 * p.sa_m + (int64_t)kb_lo * p.sa_kb;
        const float *sBb = p.sB + (int64_t)expert * p.sb_g + (int64_t)(n0 >> 7) * p.sb_nb + (int64_t)kb_lo * p.sb_kb;

        // DMA of one K block. Segment s covers tile rows 8s..8s+7 (A rows
        // first, then B rows); lane i fills LDS bytes 16 i of it: row
        // 8s + i/8, physical chunk i%8, i.e. logical chunk (i%8) ^ swz(row).
        // As swz(row) only depends on row bits 1-2, a lane's offset is
        // (8s + i/8) * ld + 16 * ((i%8) ^ swz(i/8)). One buffer resource per
        // operand tile covers exactly its valid rows, so rows past them
        // (M edge, masked counts) read as zeros.
        const int seg_row = lane >> 3;
        const int seg_ch = (lane & 7) ^ swz(seg_row);
        const uint32_t voff_a = (uint32_t)(seg_row * p.lda + seg_ch * 16);
        const uint32_t voff_b = (uint32_t)(seg_row * p.ldb + seg_ch * 16);
        const v4i rsrc_a = buffer_rsrc(Ab, (uint32_t)(rows * p.lda));
        const v4i rsrc_b = buffer_rsrc(Bb, (uint32_t)(BN * p.ldb));
        const uint32_t voff_sa = (uint32_t)(min(wave * 64 + lane, rows - 1) * p.sa_m * 4);
        const uint32_t voff_sb = (uint32_t)(min(lane, C::kNB - 1) * p.sb_nb * 4);

        // Issuing wave w (of kDmaWaves) copies segments w, w + kDmaWaves, ...:
        // its A segments first, then its B segments. The lane offset walks
        // through them by one add per copy (see add_in_place).
        const int w_dma = C::kDmaUpper ? wave - C::kWaves / 2 : wave;
        const uint32_t va0 = voff_a + (uint32_t)(w_dma * 8 * p.lda);
        const uint32_t vb0 = voff_b + (uint32_t)(w_dma * 8 * p.ldb);
        const uint32_t step_a = (uint32_t)(C::kDmaWaves * 8 * p.lda);
        const uint32_t step_b = (uint32_t)(C::kDmaWaves * 8 * p.ldb);
        const bool issues_ops = !(C::kDmaUpper && wave < C::kWaves / 2);  // the lower half issues no operand copies
        // The copies of one K block into `stage`: the A tile (with sA and sB),
        // then the B tile.
        auto issue_a = [&](int kb, int stage) {
            const uint32_t sbase = smem_base + stage * C::kStageBytes;
            const uint32_t seg0 = sbase + w_dma * 1024;  // this wave's first segment
            if (issues_ops) {
                uint32_t o = va0;
#pragma unroll
                for (int q = 0; q < C::kDmaQA; ++q) {
                    dma_buf_b128(rsrc_a, o, kb * 128, seg0 + q * C::kDmaWaves * 1024);
                    if (q + 1 < C::kDmaQA)
                        o = add_in_place(o, step_a);
                }
            }
            if (loads_sa)
                dma_b32(sAb + (int64_t)kb * p.sa_kb, voff_sa, sbase + C::kOffSa + wave * 256);
            if (loads_sb)
                dma_b32(sBb + (int64_t)kb * p.sb_kb, voff_sb, sbase + C::kOffSb);
        };
        auto issue_b = [&](int kb, int stage) {
            const uint32_t seg0 = smem_base + stage * C::kStageBytes + w_dma * 1024;
            if (issues_ops) {
                uint32_t o = vb0;
#pragma unroll
                for (int q = C::kDmaQA; q < C::kDmaQ; ++q) {
                    if (C::kStreamB)
                        dma_buf_b128_nt(rsrc_b, o, kb * 128, seg0 + q * C::kDmaWaves * 1024);
                    else
                        dma_buf_b128(rsrc_b, o, kb * 128, seg0 + q * C::kDmaWaves * 1024);
                    if (q + 1 < C::kDmaQ)
                        o = add_in_place(o, step_b);
                }
            }
        };
        auto issue = [&](int kb, int stage) {
            if (C::kEarlyB) {   // only the A copy here; B was issued a block earlier
                issue_a(kb, stage);
                return;
            }
            if (issues_ops) {
                const uint32_t seg0 = smem_base + stage * C::kStageBytes + w_dma * 1024;
                uint32_t o = va0;
#pragma unroll
                for (int q = 0; q < C::kDmaQA; ++q) {
                    dma_buf_b128(rsrc_a, o, kb * 128, seg0 + q * C::kDmaWaves * 1024);
                    if (q + 1 < C::kDmaQA)
                        o = add_in_place(o, step_a);
                }
                issue_b(kb, stage);
            }
            const uint32_t sbase = smem_base + stage * C::kStageBytes;
            if (loads_sa)
                dma_b32(sAb + (int64_t)kb * p.sa_kb, voff_sa, sbase + C::kOffSa + wave * 256);
            if (loads_sb)
                dma_b32(sBb + (int64_t)kb * p.sb_kb, voff_sb, sbase + C::kOffSb);
        };

        v4f acc[MI][NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        // LDS byte offsets of this lane's fragments: rows wm0 + l16 + 16 i of
        // A and wn0 + l16 + 16 j of B, logical chunks lg and lg + 4. Rows 16
        // apart share swz(), so sub-tile i is the same offset + 2048 i.
        const int fsw = swz(l16);
        const int fa_lo = (wm0 + l16) * 128 + ((lg ^ fsw) << 4), fa_hi = (wm0 + l16) * 128 + (((lg + 4) ^ fsw) << 4);
        const int fb_lo = (wn0 + l16) * 128 + ((lg ^ fsw) << 4), fb_hi = (wn0 + l16) * 128 + (((lg + 4) ^ fsw) << 4);

        // The rows of MFMA partials form one stream across K blocks: row i's
        // partials are folded into acc (times sA * sB of their block) while
        // the MFMAs of the next row run, and the last row of a block is
        // folded during row 0 of the next block, so the matrix core is not
        // left idle around the block barrier waiting for a promotion.
        v4f part[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            part[j] = v4f{0.f, 0.f, 0.f, 0.f};
        float part_sc = 0.f;   // scale of the row held in part

        // Waves whose rows are all padding, or (contiguous) belong to the other
        // pass's expert, skip the math.
        bool wave_active = wm0 < rows;
        if (L == kContiguous && npass == 2)
            wave_active = wave_active && ((wm0 < 128) == (pass == 0));
        auto compute = [&](auto stage_c, auto &&after_row0) {
            constexpr int st = decltype(stage_c)::value;
            const uint8_t *As = smem + st * C::kStageBytes;
            const uint8_t *Bs = As + C::kOffB;
            const float *sas = reinterpret_cast<const float *>(As + C::kOffSa);
            auto frag = [&](const uint8_t *t, int lo, int hi, int k) {
                return join(*reinterpret_cast<const uint4 *>(t + lo + 2048 * k),
                            *reinterpret_cast<const uint4 *>(t + hi + 2048 * k));
            };
            // LDS reads in the order the MFMAs consume them (in-order
            // completion lets each MFMA wait for just its own operands): A
            // row 0, the B fragments, A row 1, then the scales, which only
            // the promotions need.
            v8i af[2], bf[NJ];
            af[0] = frag(As, fa_lo, fa_hi, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bf[j] = frag(Bs, fb_lo, fb_hi, j);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (MI > 1)
                af[1] = frag(As, fa_lo, fa_hi, 1);
            __builtin_amdgcn_sched_barrier(0);
            const float sb = reinterpret_cast<const float *>(As + C::kOffSb)[wn0 >> 7];
            float sa = sas[wm0 + l16];  // sA of row i, read one row at a time
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (i >= 1 && i + 1 < MI)
                    af[(i + 1) & 1] = frag(As, fa_lo, fa_hi, i + 1);
                if (i >= 1)
                    sa = sas[wm0 + 16 * i + l16];
                __builtin_amdgcn_sched_barrier(0);
                // part holds row i-1 (the previous block's last row when i == 0)
                const float sc = part_sc;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const v4f nx = mfma_fmt_16x16x128<F>(bf[j], af[i & 1]);
                    if (i == 0)
                        acc[MI - 1][j] += part[j] * sc;
                    else
                        acc[i - 1][j] += part[j] * sc;
                    part[j] = nx;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
                }
                __builtin_amdgcn_sched_barrier(0);
                part_sc = sa * sb;
                if (i == 0)
                    after_row0();
            }
        };

        // One pipeline step for K block kb held in stage st = kb % S.
        auto step = [&](auto stage_c, int kb) {
            constexpr int st = decltype(stage_c)::value;
            if constexpr (C::kEarlyB) {
                // In flight after this block's A copy: the B copy of block
                // kb + 1 (this wave's B segments), if there is one.
                if (issues_ops && kb + 1 < nk)
                    wait_vmcnt<C::kDmaQ - C::kDmaQA>();
                else
                    wait_vmcnt<0>();
            } else {
                // Stage kb has landed once at most (S-2) later stages are in flight.
                if (kb + S - 2 < nk)
                    wait_stage<SEGW, S - 2>(per_stage);
                else
                    wait_vmcnt<0>();
            }
            // this wave's reads of the previous block have returned, so the
            // stage they read may be overwritten once every wave is here
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wg_barrier();  // every wave's DMA for kb is visible; stage (kb-1)%S is free
            if (kb + S - 1 < nk)
                issue(kb + S - 1, (st + S - 1) % S);
            // Early B: once every wave holds its B fragments of block kb (row 0
            // has issued its MFMAs, so they have been read), B of block kb + 2
            // goes into this stage's B half.
            auto early_b = [&]() {
                if constexpr (C::kEarlyB) {
                    // this wave's B fragment reads have returned
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wg_barrier();
                    if (kb + 2 < nk)
                        issue_b(kb + 2, st);
                }
            };
            if (wave_active)
                compute(stage_c, early_b);
            else
                early_b();
        };

        // The previous tile's stores have completed (the vmcnt bookkeeping
        // counts only this tile's DMA) and its LDS reads are done.
        wait_vmcnt<0>();
        wg_barrier();
        if constexpr (C::kEarlyB) {
            // block 0 whole, and B of block 1 (A of block 1 follows in step 0)
            issue_a(0, 0);
            issue_b(0, 0);
            if (1 < nk)
                issue_b(1, 1);
        } else {
#pragma unroll
            for (int s = 0; s < S - 1; ++s)
                if (s < nk)
                    issue(s, s);
        }
        for (int kb0 = 0; kb0 < nk; kb0 += S) {
            step(std::integral_constant<int, 0>{}, kb0);
            if (kb0 + 1 < nk)
                step(std::integral_constant<int, 1 % S>{}, kb0 + 1);
            if (S > 2 && kb0 + 2 < nk)
                step(std::integral_constant<int, 2 % S>{}, kb0 + 2);
            if (S > 3 && kb0 + 3 < nk)
                step(std::integral_constant<int, 3 % S>{}, kb0 + 3);
        }
        // fold the last row
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[MI - 1][j] += part[j] * part_sc;

        uint16_t *Dg = p.D + (int64_t)g * p.d_stride_g;
        // Contiguous: the expert id (and with SCATTER the token) of each of
        // this lane's rows, all read before the first store. The compiler
        // cannot tell the stores from these arrays apart, so a load left
        // between two rows' stores would wait for the stores' round trip.
        // Indices are clamped so that every lane loads; bit i of row_bits
        // says whether this lane's row i is written. (The row numbers are
        // formed in place: hoisted out of the tile loop, they would be kept
        // across the K loop.)
        const int mb = m0 + wm0 + l16;
        auto row_m = [&](int i) { return (int)add_in_place((uint32_t)mb, 16 * i); };
        uint32_t row_bits = 0;
        int row_tok[SCATTER ? MI : 1];
        if constexpr (L == kContiguous) {
            int row_id[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int mc = min(row_m(i), p.M - 1);
                row_id[i] = p.ids[mc];
                if constexpr (SCATTER)
                    row_tok[i] = p.row_dst[mc];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                // a segment tile covers seg_rows rows (128 for a segment's
                // tail or a block on its own): the rows after them belong to
                // another tile, possibly of the same expert
                const int m = row_m(i);
                if (m < p.M && (!SEG || m - m0 < seg_rows) && row_id[i] == expert)
                    row_bits |= 1u << i;
            }
        }
        auto row_ok = [&](int i) {
            if (L == kDense)
                return row_m(i) < p.M;
            if (L == kMasked)
                return row_m(i) < limit;
            return ((row_bits >> i) & 1) != 0;
        };
        if (to_ws) {
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int m = row_m(i);
                if (!row_ok(i) || (SEG && m - m0 >= seg_rows))
                    continue;
                // dense: row m of slice `slice`; segment tails: row 128 h + (m - m0)
                const int64_t wr = SEG ? (int64_t)slice * p.ws_rows + 128 * seg_h + (m - m0)
                                       : (int64_t)slice * p.M + m;
                float *wrow = p.ws + wr * p.N + n0 + wn0 + 4 * lg;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    *reinterpret_cast<v4f *>(wrow + 16 * j) = acc[i][j];
            }
            continue;
        }
        if constexpr (L == kContiguous) {
            // Direct stores (8 bytes per lane): staging through LDS made the
            // contiguous kernel spill in its K loop.
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (!row_ok(i))
                    continue;
                int64_t dm = row_m(i);
                if constexpr (SCATTER) {  // the row's token: its row of D in token order
                    dm = row_tok[i];
                    if (dm < 0 || dm >= p.dst_rows)
                        continue;
                }
                uint16_t *drow = Dg + dm * p.ldd + n0 + wn0 + 4 * lg;
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    *reinterpret_cast<uint2 *>(drow + 16 * j) = pack_bf16x4(acc[i][j]);
            }
            continue;
        }
        // bf16 results go through this wave's own LDS area (the stages are
        // free once every wave is past its last block), so that each store
        // instruction writes whole rows of the wave's tile: RPI rows of RB
        // bytes, 16 bytes per lane. Chunks are XOR-permuted by row & 7.
        constexpr int RB = C::kWN * 2, CPR = RB / 16, RPI = 64 / CPR;
        static_assert(C::kWaves * C::kWM * RB <= C::kSmemBytes, "epilogue staging fits the stages");
        static_assert(CPR >= 8 && 64 % CPR == 0, "epilogue row layout");
        uint8_t *ep = smem + wave * (C::kWM * RB);
        wg_barrier();
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int r = 16 * i + l16;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int c = 2 * j + (lg >> 1);
                *reinterpret_cast<uint2 *>(ep + r * RB + ((c ^ (r & 7)) << 4) + ((lg & 1) << 3)) =
                    pack_bf16x4(acc[i][j]);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own area: no barrier needed
#pragma unroll
        for (int q = 0; q < C::kWM / RPI; ++q) {
            const int r = q * RPI + lane / CPR, c = lane % CPR;
            const uint4 v = *reinterpret_cast<const uint4 *>(ep + r * RB + ((c ^ (r & 7)) << 4));
            const int m = m0 + wm0 + r;
            if (L == kDense ? m < p.M : m < limit)
                *reinterpret_cast<uint4 *>(Dg + (int64_t)m * p.ldd + n0 + wn0 + c * 8) = v;
        }
        }  // pass
    }
}

// Second half of a dense split-K GEMM: D = bf16(sum over slices of ws[slice]),
// slices added in order 0, 1, ... so the result does not depend on which work
// item finished first. One thread per 4 consecutive outputs of a row.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *ws, int ksplit, int M, int N,
                                                            uint16_t *D, int64_t ldd)
{
    const int nq = N >> 2;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)M * nq)
        return;
    const int m = (int)(q / nq), c = (int)(q - (int64_t)m * nq) * 4;
    v4f s = *reinterpret_cast<const v4f *>(ws + (int64_t)m * N + c);
    for (int k = 1; k < ksplit; ++k)
        s += *reinterpret_cast<const v4f *>(ws + ((int64_t)k * M + m) * N + c);
    *reinterpret_cast<uint2 *>(D + (int64_t)m * ldd + c) = pack_bf16x4(s);
}

// Second half of the segment tails split over K: for tail h (the h-th
// segment whose size is an odd multiple of 128, expert e, rows m0..m0+127),
// row r goes to D[m0 + r] (or, with row_dst, to row row_dst[m0 + r] of D) when
// that row belongs to e, as the sum of the slices in order 0, 1, ...
// One workgroup per tail row (blockIdx.x = r, blockIdx.y = h); each thread
// takes 4 consecutive columns at a time with every slice's load in flight.
__global__ void __launch_bounds__(256) seg_tail_reduce_kernel(Params p)
{
    const int h = blockIdx.y, r = blockIdx.x;
    int tails = 0, e = -1;
    for (int g = 0; g < p.G; ++g) {
        const int sz = p.layout[g + 1] - p.layout[g];
        if (sz > 0 && ((sz >> 7) & 1)) {
            if (tails == h)
                e = g;
            ++tails;
        }
    }
    if (e < 0)
        return;  // fewer tails than the grid allows
    const int m0 = p.layout[e] + ((p.layout[e + 1] - p.layout[e]) & ~255);
    const int m = m0 + r;
    if (m0 < 0 || m >= p.M || p.ids[m] != e)
        return;
    int64_t dm = m;
    if (p.row_dst) {
        const int t = p.row_dst[m];
        if (t < 0 || t >= p.dst_rows)
            return;
        dm = t;
    }
    const int ks = tail_split(tails * p.tiles_n, p.K >> 7, p.ksplit, p.tail_slots);
    const float *src = p.ws + (int64_t)(128 * h + r) * p.N;
    const int64_t slice = (int64_t)p.ws_rows * p.N;
    for (int c = 4 * threadIdx.x; c < p.N; c += 1024) {
        v4f v[kMaxTailSplit];
#pragma unroll
        for (int k = 0; k < kMaxTailSplit; ++k)
            if (k < ks)
                v[k] = *reinterpret_cast<const v4f *>(src + k * slice + c);
        v4f s = v[0];
#pragma unroll
        for (int k = 1; k < kMaxTailSplit; ++k)
            if (k < ks)
                s += v[k];
        *reinterpret_cast<uint2 *>(p.D + dm * p.ldd + c) = pack_bf16x4(s);
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel (decode shapes, M <= 16 * MT). One workgroup per 16 rows of
// B; its eight waves split the K blocks, read B straight from HBM into MFMA
// operand registers (B is streamed exactly once, no LDS staging) with every
// load of a chunk issued before the first MFMA, and reduce their fp32
// accumulators through LDS at the end in a fixed order.
constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = kDecodeWaves * 64;

template <int MT>
struct DecodeCfg {
    static constexpr int kUnroll = MT == 1 ? 8 : (MT == 2 ? 4 : 2);  // K blocks per load batch
};

template <int MT>
__global__ void __launch_bounds__(kDecodeThreads, 1) decode_kernel(Params p)
{
    constexpr int U = DecodeCfg<MT>::kUnroll;
    __shared__ v4f red[kDecodeWaves][MT][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nk = p.K >> 7;
    const int kb_begin = (wave * nk) / kDecodeWaves, kb_end = ((wave + 1) * nk) / kDecodeWaves;

    const uint8_t *brow = p.B + (int64_t)(n0 + l16) * p.ldb + 16 * lg;
    const float *sbp = p.sB + (int64_t)(n0 >> 7) * p.sb_nb;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += U) {
        v8i bf[U];
        v8i af[U][MT];
        float sb[U];
        float sa[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = kb0 + u;
            if (kb < kb_end) {
                const uint8_t *src = brow + (int64_t)kb * 128;
                bf[u] = join(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 64));
                sb[u] = sbp[(int64_t)kb * p.sb_kb];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = kb0 + u;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = mt * 16 + l16;
                if (kb < kb_end && m < p.M) {
                    const uint8_t *src = p.A + (int64_t)m * p.lda + (int64_t)kb * 128 + 16 * lg;
                    af[u][mt] = join(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 64));
                    sa[u][mt] = p.sA[(int64_t)m * p.sa_m + (int64_t)kb * p.sa_kb];
                } else {
                    af[u][mt] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    sa[u][mt] = 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
    // Wave w finishes m-subtiles mt = w, w + 8, ... summing the waves in order.
    for (int mt = wave; mt < MT; mt += kDecodeWaves) {
        v4f v = red[0][mt][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            v += red[w][mt][lane];
        const int m = mt * 16 + l16;
        if (m < p.M)
            *reinterpret_cast<uint2 *>(p.D + (int64_t)m * p.ldd + n0 + 4 * lg) = pack_bf16x4(v);
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel with the whole LHS staged in LDS (M <= 16 and M*K bytes
// within kDecodeLdsA): the decode-shaped case, bound by streaming B once.
// Per workgroup (16 rows of B, eight waves splitting the K blocks):
//   1. every wave issues the non-temporal loads of its B blocks first (the
//      long pole, HBM), then its share of the LDS-DMA of A and sA (served
//      by L2, shared by all workgroups), then one load of its sB values;
//   2. one wait and one barrier, then MFMA + promotion per block from
//      registers (B) and LDS (A, sA); sB is broadcast from its lane;
//   3. fixed-order reduction of the eight waves through LDS, bf16 store.
constexpr int kDecodeLdsA = 120 * 1024;   // LHS bytes held in LDS
constexpr int kDecodeLdsSa = 1024;        // LHS scales (floats) held in LDS
constexpr int kDecodeLdsUnroll = 8;       // B blocks per wave held in registers per pass

__device__ __forceinline__ v8i load_nt_b256(const uint8_t *p)
{
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u lo = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    const v4u hi = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p + 64));
    v8i r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

__global__ void __launch_bounds__(kDecodeThreads, 1) decode_lds_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t a_lds[kDecodeLdsA];
    __shared__ float sa_lds[kDecodeLdsSa];
    __shared__ v4f red[kDecodeWaves][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nk = p.K >> 7;
    const int M = p.M;
    const int kb_begin = (wave * nk) / kDecodeWaves, kb_end = ((wave + 1) * nk) / kDecodeWaves;

    const uint8_t *brow = p.B + (int64_t)(n0 + l16) * p.ldb + 16 * lg;
    const float *sbp = p.sB + (int64_t)(n0 >> 7) * p.sb_nb;
    const uint32_t a_base = lds_addr(a_lds), sa_base = lds_addr(sa_lds);
    const v4i rsrc_a = buffer_rsrc(p.A, (uint32_t)((int64_t)(M - 1) * p.lda + p.K));

    v4f acc = {0.f, 0.f, 0.f, 0.f};
    bool staged = false;
    for (int kb0 = kb_begin; kb0 < kb_end || !staged; kb0 += kDecodeLdsUnroll) {
        v8i bf[kDecodeLdsUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeLdsUnroll; ++u)
            if (kb0 + u < kb_end)
                bf[u] = load_nt_b256(brow + (int64_t)(kb0 + u) * 128);
        if (!staged) {
            // LHS rows [0, M) -> LDS as M rows of K bytes, 1 KB per DMA op.
            const int a_ops = (M * p.K) >> 10;
            for (int q = wave; q < a_ops; q += kDecodeWaves) {
                const int b = (q << 10) + 16 * lane;     // byte in the LDS image
                const int row = b / p.K, col = b - row * p.K;
                dma_buf_b128(rsrc_a, (uint32_t)(row * p.lda + col), 0u, a_base + (q << 10));
            }
            const int sa_ops = (M * nk + 63) >> 6;
            for (int q = wave; q < sa_ops; q += kDecodeWaves) {
                int e = (q << 6) + lane;
                e = e < M * nk ? e : 0;
                const int m = e / nk, kb = e - m * nk;
                dma_b32(p.sA, (uint32_t)((m * p.sa_m + kb * p.sa_kb) * 4), sa_base + (q << 8));
            }
        }
        // This wave's sB values, one per lane, broadcast per block below.
        const int cnt = min(kDecodeLdsUnroll, kb_end - kb0);
        const float sbv = cnt > 0 ? sbp[(int64_t)(kb0 + min(lane, cnt - 1)) * p.sb_kb] : 0.f;
        wait_vmcnt<0>();
        if (!staged) {
            wg_barrier();  // A and sA are in LDS for every wave
            staged = true;
        }
#pragma unroll
        for (int u = 0; u < kDecodeLdsUnroll; ++u) {
            const int kb = kb0 + u;
            if (kb < kb_end) {
                v8i af = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                float sa = 0.f;
                if (l16 < M) {
                    const uint8_t *ar = a_lds + l16 * p.K + kb * 128 + 16 * lg;
                    af = join(*reinterpret_cast<const uint4 *>(ar), *reinterpret_cast<const uint4 *>(ar + 64));
                    sa = sa_lds[l16 * nk + kb];
                }
                const float sb = __shfl(sbv, u);
                const v4f part = mfma_e4m3_16x16x128(bf[u], af);
                acc += part * (sa * sb);
            }
        }
    }

    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        v4f v = red[0][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            v += red[w][lane];
        if (l16 < M)
            *reinterpret_cast<uint2 *>(p.D + (int64_t)l16 * p.ldd + n0 + 4 * lg) = pack_bf16x4(v);
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel with a fixed number of K blocks per wave (M <= 16, K =
// 8 * NB * 128): every load is unconditional and issued up front in block
// order (A fragments and sA first, they come from L2; then sB; then B, the
// HBM stream), so the compiler waits for each block's B alone and the MFMA
// and promotion of block u run while blocks u+1.. are still in flight. Only
// the last block's math and the cross-wave reduction follow the last byte.
template <int NB>
__global__ void __launch_bounds__(kDecodeThreads, 1) decode_static_kernel(Params p)
{
    __shared__ v4f red[kDecodeWaves][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int kb0 = wave * NB;
    const bool arow = l16 < p.M;

    const uint8_t *arow_p = p.A + (int64_t)l16 * p.lda + (int64_t)kb0 * 128 + 16 * lg;
    const float *sarow_p = p.sA + (int64_t)l16 * p.sa_m + (int64_t)kb0 * p.sa_kb;
    v8i af[NB];
    float sa[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        if (arow) {
            const uint8_t *src = arow_p + u * 128;
            af[u] = join(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 64));
            sa[u] = sarow_p[(int64_t)u * p.sa_kb];
        } else {
            af[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sa[u] = 0.f;
        }
    }
    const float *sbp = p.sB + (int64_t)(n0 >> 7) * p.sb_nb + (int64_t)kb0 * p.sb_kb;
    const float sbv = sbp[(int64_t)min(lane, NB - 1) * p.sb_kb];

    const uint8_t *brow = p.B + (int64_t)(n0 + l16) * p.ldb + (int64_t)kb0 * 128 + 16 * lg;
    v8i bf[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const uint8_t *src = brow + u * 128;
        bf[u] = join(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 64));
    }
    // Keep every load above this point: the scheduler would otherwise sink
    // later loads below earlier MFMAs to save registers, serialising latency.
    __builtin_amdgcn_sched_barrier(0);

    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const float sb = __shfl(sbv, u);
        const v4f part = mfma_e4m3_16x16x128(bf[u], af[u]);
        acc += part * (sa[u] * sb);
    }

    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        v4f v = red[0][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            v += red[w][lane];
        if (arow)
            *reinterpret_cast<uint2 *>(p.D + (int64_t)l16 * p.ldd + n0 + 4 * lg) = pack_bf16x4(v);
    }
}

// ---------------------------------------------------------------------------
// Small-M kernel, M <= MR (8 or 16), NB K blocks per wave (K = 8 * NB * 128).
// Each wave stages the LHS rows of its own K blocks (and their sA) in a
// wave-private LDS region with full-line LDS-DMA, issued first; then it loads
// sB and issues its B blocks (the HBM stream) straight into MFMA operand
// registers. No barrier precedes the math: a wave only reads its own LDS
// region, and each block's MFMA waits for that block's B alone.
template <int NB, int MR, bool BFULL, int MP = 1, bool ROT = false>
__global__ void __launch_bounds__(kDecodeThreads, 1) decode_dma_kernel(Params p)
{
    // MP passes of MR = 16 LHS rows each (M <= 16 MP): B is loaded and put
    // in operand layout once; each later pass restages the next 16 rows of
    // the wave's LHS blocks in the same LDS area.
    static_assert(MR == 8 || MR == 16, "LHS rows staged per block");
    static_assert(MP == 1 || MR == 16, "multi-pass stages 16 rows per pass");
    static_assert(MP >= 1 && MP <= kDecodeWaves, "one reducing wave per pass");
    constexpr int kBlk = MR * 128;                 // LDS bytes per K block of the LHS
    constexpr int kOps = NB * MR / 8;              // 1 KB DMA ops per wave for the LHS
    constexpr int kSaOps = (MR * NB + 63) / 64;    // dword DMA ops per wave for its sA
    __shared__ __attribute__((aligned(1024))) uint8_t a_lds[kDecodeWaves][NB * kBlk];
    __shared__ __attribute__((aligned(1024))) uint8_t b_ring[kDecodeWaves][BFULL ? 2 : 1][2048];
    __shared__ float sa_lds[kDecodeWaves][kSaOps * 64];
    // Each wave hands its partials to the reduction through its own LHS
    // staging area, which it has finished reading by then.
    static_assert(sizeof(v4f) * 64 * MP <= NB * kBlk, "reduction slot");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int kb0 = wave * NB;
    const int M = p.M;
    // ROT (chosen when B's row stride is a multiple of 4 KB): every row then
    // starts at the same HBM channel offset, and the loads issued together
    // would all sit at the same few 128-byte positions of a row, so
    // workgroup g walks its waves' blocks starting at block g % NB
    // (8x4096x4096: 6.25 -> 5.72 us). Without ROT the block indices stay
    // compile-time constants. Only the order of the fp32 sum over blocks
    // depends on it (fixed for a given shape).
    const int rot = ROT ? (int)(blockIdx.x % NB) : 0;

    // 1. LHS rows [16 pass, 16 pass + MR): op q covers rows 8(q%(MR/8))..+7 of
    // block q/(MR/8); lane i takes row +i/8, physical chunk i%8 = logical
    // chunk (i%8) ^ swz(row). Rows >= M read as zeros (offset past the buffer).
    const uint32_t a_base = lds_addr(&a_lds[wave][0]);
    const v4i rsrc_a = buffer_rsrc(p.A, (uint32_t)((int64_t)(M - 1) * p.lda + p.K));
    auto stage_lhs = [&](int pass) {
#pragma unroll
        for (int q = 0; q < kOps; ++q) {
            const int u = q / (MR / 8), r = (q % (MR / 8)) * 8 + (lane >> 3);
            const int ch = (lane & 7) ^ swz(r);
            const int row = MR * pass + r;
            const uint32_t voff = row < M ? (uint32_t)(row * p.lda + (kb0 + u) * 128 + ch * 16) : 0xffffffffu;
            dma_buf_b128(rsrc_a, voff, 0u, a_base + q * 1024);
        }
#pragma unroll
        for (int o = 0; o < kSaOps; ++o) {  // sA for (row, block) = (i % MR, i / MR), i = 64 o + lane
            const int i = 64 * o + lane;
            const int r = MR * pass + i % MR, u = min(i / MR, NB - 1);
            const int rr = r < M ? r : 0;
            dma_b32(p.sA, (uint32_t)((rr * p.sa_m + (int64_t)(kb0 + u) * p.sa_kb) * 4),
                    lds_addr(&sa_lds[wave][64 * o]));
        }
    };
    stage_lhs(0);
    // 2. sB for the wave's blocks, one per lane.
    const float *sbp = p.sB + (int64_t)(n0 >> 7) * p.sb_nb + (int64_t)kb0 * p.sb_kb;
    const float sbv = sbp[(int64_t)min(lane, NB - 1) * p.sb_kb];
    // 3. B blocks. BFULL: non-temporal full 128-byte lines (lane i: row
    // 8 j + i/8, chunk i%8 of instruction j), transposed to the MFMA layout
    // through a two-slot wave-private LDS ring; otherwise straight into MFMA
    // operand registers (16 rows x 64 bytes per instruction).
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    v4u bl[NB][2];
    v8i bf[NB];
    if constexpr (BFULL) {
        const uint8_t *bbase = p.B + (int64_t)(n0 + (lane >> 3)) * p.ldb + (int64_t)kb0 * 128 + 16 * (lane & 7);
#pragma unroll
        for (int v = 0; v < NB; ++v) {
            const int u = v + rot < NB ? v + rot : v + rot - NB;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bl[v][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u *>(bbase + (int64_t)(8 * j) * p.ldb + u * 128));
            __builtin_amdgcn_sched_barrier(0);  // keep block order: each block waits for itself only
        }
    } else {
        const uint8_t *brow = p.B + (int64_t)(n0 + l16) * p.ldb + (int64_t)kb0 * 128 + 16 * lg;
#pragma unroll
        for (int v = 0; v < NB; ++v) {
            const int u = v + rot < NB ? v + rot : v + rot - NB;
            const uint8_t *src = brow + u * 128;
            bf[v] = join(*reinterpret_cast<const uint4 *>(src), *reinterpret_cast<const uint4 *>(src + 64));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // The LHS DMA is older than sB and the B loads: it has landed once at most
    // 1 + 2 NB loads are outstanding.
    wait_vmcnt<1 + 2 * NB>();

    v4f acc[MP];
    const int fsw = swz(l16);
    const int fsw_a = swz(l16 & 7);
#pragma unroll
    for (int pass = 0; pass < MP; ++pass) {
        if (pass > 0) {
            // This wave's reads of the previous pass's LHS have returned (they
            // fed its MFMAs); restage its area and wait for the copies only
            // (every B load was consumed in pass 0).
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stage_lhs(pass);
            wait_vmcnt<0>();
        }
        acc[pass] = v4f{0.f, 0.f, 0.f, 0.f};
        const bool arow = MR * pass + l16 < M;
#pragma unroll
        for (int v = 0; v < NB; ++v) {
            const int u = v + rot < NB ? v + rot : v + rot - NB;  // block of the wave's range
            if constexpr (BFULL) {
                if (pass == 0) {
                    uint8_t *slot = &b_ring[wave][v & 1][0];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int r = 8 * j + (lane >> 3);
                        *reinterpret_cast<v4u *>(slot + r * 128 + (((lane & 7) ^ swz(r)) << 4)) = bl[v][j];
                    }
                    const uint8_t *t = slot + l16 * 128;
                    bf[v] = join(*reinterpret_cast<const uint4 *>(t + ((lg ^ fsw) << 4)),
                                 *reinterpret_cast<const uint4 *>(t + (((lg + 4) ^ fsw) << 4)));
                }
            }
            v8i af = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            float sa = 0.f;
            if (arow) {
                const uint8_t *t = &a_lds[wave][u * kBlk + l16 * 128];
                af = join(*reinterpret_cast<const uint4 *>(t + ((lg ^ fsw_a) << 4)),
                          *reinterpret_cast<const uint4 *>(t + (((lg + 4) ^ fsw_a) << 4)));
                sa = sa_lds[wave][u * MR + l16];
            }
            const float sb = __shfl(sbv, u);
            const v4f part = mfma_e4m3_16x16x128(bf[v], af);
            acc[pass] += part * (sa * sb);
        }
    }

    // Wave w's partials of pass q sit at its area + 1 KB q; wave q reduces pass q.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < MP; ++pass)
        reinterpret_cast<v4f *>(&a_lds[wave][1024 * pass])[lane] = acc[pass];
    __syncthreads();
    if (wave < MP) {
        const int pass = wave;
        v4f v = reinterpret_cast<const v4f *>(&a_lds[0][1024 * pass])[lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            v += reinterpret_cast<const v4f *>(&a_lds[w][1024 * pass])[lane];
        const int row = MR * pass + l16;
        if (row < M)
            *reinterpret_cast<uint2 *>(p.D + (int64_t)row * p.ldd + n0 + 4 * lg) = pack_bf16x4(v);
    }
}

}  // namespace dgk
