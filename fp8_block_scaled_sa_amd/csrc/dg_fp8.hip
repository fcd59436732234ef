// dg_fp8.hip -- C ABI of the gfx950 block-scaled FP8 GEMM (declared in
// include/dg_fp8.h): host-side validation, device check, kernel choice and
// launch. The library allocates no device memory and synchronises no stream:
// the scratch memory some paths use (split-K partial sums, segment offsets
// derived on the device) is the caller's workspace, passed to the *_ws entry
// points; without one those paths run unsplit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#include "dg_fp8.h"
#include "kernels.hpp"
#include "moe.hpp"
#include "quant.hpp"

namespace {

thread_local int g_last_hip_error = 0;

struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int cus = 0;
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mu;

// Scratch memory of dg_fp8_gemm_nt_noalloc, for callers that cannot
// allocate: a fixed array in the library's code object. Each GPU the library
// is loaded on holds its own copy until the process ends. Host code never
// names the array itself (on the host its name is only a stand-in for the
// device symbol): it takes each device's address once with
// hipGetSymbolAddress, with that device current, and passes that address to
// the kernels. 32 MiB holds the partial sums of every dense split-K launch on
// a 256-CU device (at most 256 work items of 256x128 fp32 partial tiles).
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
uint8_t *g_scratch_ptr[kMaxDevices];
bool g_scratch_known[kMaxDevices];

// The address of the current device's copy of `scratch`, resolved on the
// first call on that device; nullptr (with the HIP error recorded) on failure.
uint8_t *device_scratch(int &status)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        status = DG_ERR_HIP;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        status = DG_ERR_UNSUPPORTED;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_devices_mu);
    if (!g_scratch_known[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            g_last_hip_error = (int)e;
            status = DG_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = (uint8_t *)ptr;
        g_scratch_known[dev] = true;
    }
    status = DG_OK;
    return g_scratch_ptr[dev];
}

int fail_hip(hipError_t e)
{
    g_last_hip_error = (int)e;
    return DG_ERR_HIP;
}

// Checks that the current device is gfx950 and caches its CU count.
int current_device(DeviceInfo &out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail_hip(e);
    if (dev < 0 || dev >= kMaxDevices)
        return DG_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_devices_mu);
    DeviceInfo &d = g_devices[dev];
    if (!d.known) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail_hip(e);
        d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        d.known = true;
    }
    out = d;
    return d.gfx950 ? DG_OK : DG_ERR_UNSUPPORTED;
}

// One call's launch context: the device's CU count, the caller's stream and
// the caller's workspace. The library owns no device memory: every step that
// can use scratch (split-K partial sums, segment offsets derived on the
// device) takes a region of the workspace the caller passed, or runs its path
// without scratch when there is none or too little. A dry run launches
// nothing and only records how many workspace bytes the fastest path would
// take (what the *_workspace_bytes queries report).
struct Ctx {
    int cus = 0;
    hipStream_t stream = nullptr;
    uint8_t *ws = nullptr;  // caller's workspace (device), may be null
    size_t ws_bytes = 0;
    size_t need = 0;        // most workspace bytes any step asked for
    bool dry = false;

    // Bytes of the workspace available from offset `off` on.
    size_t avail(size_t off) const { return ws && ws_bytes > off ? ws_bytes - off : 0; }
    // Records that a step would take `want` bytes at `off`; returns the region
    // if the workspace holds it, else nullptr.
    void *take(size_t off, size_t want)
    {
        need = std::max(need, off + want);
        if (dry || want > avail(off))
            return nullptr;
        return ws + off;
    }
};

// Workspace regions start on 256-byte boundaries.
constexpr size_t kWsAlign = 256;
size_t ws_round(size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Most experts for which the contiguous call given only ids derives segment offsets.
constexpr int64_t kDeriveMaxExperts = 128;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [lo, hi) byte extent of a strided 2-D/3-D operand (all strides >= 0).
struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void *p, int64_t elem, int64_t last_index)
{
    const uintptr_t lo = (uintptr_t)p;
    return Extent{lo, lo + (uintptr_t)((last_index + 1) * elem)};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

constexpr int64_t kInt32Max = 0x7fffffff;

int check_common_shape(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K <= 0)
        return DG_ERR_BAD_SHAPE;
    if (K % 128 != 0 || N % 128 != 0)
        return DG_ERR_BAD_SHAPE;
    if (M > kInt32Max || N > kInt32Max || K > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    return DG_OK;
}

// sA extent for rows [0, rows) and nkb K blocks.
int64_t last_scale_index(int64_t rows, int64_t nkb, int64_t s_row, int64_t s_kb)
{
    return (rows - 1) * s_row + (nkb - 1) * s_kb;
}

// Tile configurations (BM, BN, waves M x N, LDS stages, tile-order group).
// 256x128 tiles split 4096- and 8192-row problems into whole waves of the
// 256 CUs; each holds 3 stages of 49 KB in LDS, one workgroup per CU, with
// 8 waves (2 per SIMD) so one wave's promotion FMAs overlap another's MFMAs.
using CfgDense = dgk::TileCfg<256, 128, 4, 2, 3, 4>;
using CfgDense4 = dgk::TileCfg<256, 128, 2, 2, 3, 4>;
using CfgBig = dgk::TileCfg<256, 256, 2, 4, 2, 4>;  // 2 stages of 66 KB; N % 256 == 0
// Masked layout: each group's B feeds one M tile, so B is streamed (non-temporal DMA).
using CfgBigStreamB = dgk::TileCfg<256, 256, 2, 4, 2, 4, true>;
// The same with the B copy of block k + 2 issued during block k (B half of a
// stage released after row 0 behind a second barrier). The whole tiles of
// the contiguous layout's segments use it: 8 experts x 8192 tokens measured
// 2% faster (260-261 against 265-266 us). Dense 4096^3 and prefill showed no
// change and the masked layout 1% slower, so those keep CfgBig.
using CfgBigE = dgk::TileCfg<256, 256, 2, 4, 2, 4, false, true>;
using CfgWide = dgk::TileCfg<128, 256, 2, 2, 3, 8>;
using CfgNarrow = dgk::TileCfg<128, 128, 2, 2, 4, 8>;
// Segment tails next to CfgBig: 8 waves and 3 stages of 50 KB. 8 waves were
// 8% faster there than CfgWide's 4, and 3 stages another 2% (5 us) than 2.
using CfgTail = dgk::TileCfg<128, 256, 2, 4, 3, 4>;

// Optional override of the kernel choice, read once: DG_TILE=<index>, for
// measurements. 1, 2, 4: dense on 256x128 (4 waves), 128x128 or 256x128 tiles
// without split-K; 6: decode with B loaded in operand layout; 7, 8, 9: older
// decode kernels; 12: masked B loaded without the non-temporal hint; 13 / 14:
// decode kernels up to M = 16 / all older decode kernels up to 64; 15:
// split-K always on 256-wide tiles;
// 16: no split-K; 18: no cut of a partly filled last round of 256x256 tiles;
// 23: segment tails not split over K; 24: the contiguous call without
// segment offsets stays on the uniform grid (no offsets derived on the device);
// 27: segment whole tiles without the early B copies;
// 2, 3, 4 also pick the contiguous layout's tile shape.
int tile_override()
{
    static int v = [] {
        const char *e = getenv("DG_TILE");
        return e ? atoi(e) : -1;
    }();
    return v;
}

template <int L, class C, int F = 0, bool SCATTER = false>
int launch_tiles(dgk::Params &p, int groups, Ctx &c)
{
    if (p.N % C::kBN != 0)
        return DG_ERR_UNSUPPORTED;  // every config is chosen so that its BN divides N
    p.tiles_m = (int)((p.M + C::kBM - 1) / C::kBM);
    p.tiles_n = p.N / C::kBN;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n * groups;
    if (tiles > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    p.num_tiles = (int)tiles;
    if (p.num_tiles == 0 || c.dry)
        return DG_OK;
    const int grid = p.num_tiles < c.cus ? p.num_tiles : c.cus;  // persistent: one workgroup per CU
    hipLaunchKernelGGL((dgk::tile_kernel<L, C, F, SCATTER>), dim3(grid), dim3(C::kThreads), 0, c.stream, p);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : fail_hip(e);
}

// Contiguous layout on segment-aligned tiles (tile_kernel's SEG mode). The
// real tile count depends on the device-side layout; each grid covers a bound
// and the kernel skips the rest. With workspace for it (from byte `ws_off`
// on), the whole 256-row tiles run first (they fill whole rounds when the
// segments are long), then the 128-row tails split over K (their rows are
// few, but each would otherwise take about as long as a whole tile), then a
// reduction adds the tails' slices in order. Without it the tails run
// unsplit in the same launch as the whole tiles.
template <class C, class CT, bool SCATTER>
int launch_contiguous_seg(dgk::Params &p, Ctx &c, size_t ws_off)
{
    static_assert(C::kBM == 256 && CT::kBM == 128, "whole tiles 256 rows, tails 128");
    if (p.N % C::kBN != 0 || p.N % CT::kBN != 0)
        return DG_ERR_UNSUPPORTED;
    p.tiles_n = p.N / C::kBN;
    p.tiles_m = (p.M + 255) / 256 + p.G;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    p.num_tiles = (int)tiles;
    p.seg_mode = 0;
    p.ksplit = 1;
    // At most this many K slices per tail, at least four K blocks each; the
    // kernels pick the count from the number of tails they find. No split
    // when the tails alone would fill two rounds of the CUs. A workspace too
    // small for every slice takes as many slices as it holds.
    const int64_t tail_tiles = (int64_t)p.G * (p.N / CT::kBN);
    int ks = tail_tiles >= 2 * (int64_t)c.cus || tile_override() == 23 ? 1 : std::min(dgk::kMaxTailSplit, (p.K / 128) / 4);
    const size_t slice_bytes = (size_t)p.G * 128 * p.N * sizeof(float);
    float *ws = nullptr;
    if (ks >= 2) {
        ws = (float *)c.take(ws_off, ks * slice_bytes);
        if (!ws && !c.dry) {
            ks = (int)std::min<size_t>(ks, c.avail(ws_off) / slice_bytes);
            ws = ks >= 2 ? (float *)(c.ws + ws_off) : nullptr;
        }
    }
    if (c.dry)
        return DG_OK;
    if (ws)
        p.seg_mode = 1;
    hipLaunchKernelGGL((dgk::tile_kernel<dgk::kContiguous, C, 0, SCATTER, true>),
                       dim3(p.num_tiles < c.cus ? p.num_tiles : c.cus), dim3(C::kThreads), 0, c.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail_hip(e);
    if (!ws)
        return DG_OK;
    dgk::Params q = p;
    q.seg_mode = 2;
    q.ksplit = ks;
    q.ws = ws;
    q.ws_rows = p.G * 128;
    q.tiles_n = p.N / CT::kBN;
    q.num_tiles = p.G * q.tiles_n * ks;
    q.tail_slots = q.num_tiles < c.cus ? q.num_tiles : c.cus;
    hipLaunchKernelGGL((dgk::tile_kernel<dgk::kContiguous, CT, 0, SCATTER, true>), dim3(q.tail_slots),
                       dim3(CT::kThreads), 0, c.stream, q);
    if ((e = hipGetLastError()) != hipSuccess)
        return fail_hip(e);
    hipLaunchKernelGGL(dgk::seg_tail_reduce_kernel, dim3(128, (unsigned)p.G), dim3(256), 0, c.stream, q);
    e = hipGetLastError();
    return e == hipSuccess ? DG_OK : fail_hip(e);
}

// launch_tiles with the operand formats chosen at run time (bit 0: A is e5m2,
// bit 1: B is e5m2); the formats only set the MFMA's format selectors.
template <int L, class C>
int launch_tiles_fmt(dgk::Params &p, int groups, Ctx &c, int f)
{
    switch (f) {
    case 1: return launch_tiles<L, C, 1>(p, groups, c);
    case 2: return launch_tiles<L, C, 2>(p, groups, c);
    case 3: return launch_tiles<L, C, 3>(p, groups, c);
    default: return launch_tiles<L, C, 0>(p, groups, c);
    }
}

int format_bits(int a_fmt, int b_fmt)
{
    if ((a_fmt != DG_FP8_E4M3 && a_fmt != DG_FP8_E5M2) || (b_fmt != DG_FP8_E4M3 && b_fmt != DG_FP8_E5M2))
        return -1;
    return (a_fmt == DG_FP8_E5M2 ? 1 : 0) | (b_fmt == DG_FP8_E5M2 ? 2 : 0);
}

// Dense GEMM on configuration C. When the tiles fill at most half of the CUs
// (small M, or small M x N), each tile's K blocks are split over ks work items
// (tiles * ks <= CUs, one round) that write fp32 partials; a second kernel
// adds the slices in order and writes D.
template <class C, int F = 0>
int launch_dense(dgk::Params &p, Ctx &c)
{
    if (p.N % C::kBN != 0)
        return DG_ERR_UNSUPPORTED;
    const int64_t tiles = (int64_t)((p.M + C::kBM - 1) / C::kBM) * (p.N / C::kBN);
    const int nk = p.K / 128;
    int ks = 1;
    if (tile_override() != 16 && tiles * 2 <= c.cus && nk >= 2)
        ks = (int)std::min<int64_t>(std::min<int64_t>(nk, c.cus / tiles), 8);
    if (ks > 1) {
        // A workspace too small for every slice takes as many as it holds.
        const size_t slice_bytes = (size_t)p.M * p.N * sizeof(float);
        p.ws = (float *)c.take(0, ks * slice_bytes);
        if (!p.ws && !c.dry) {
            ks = (int)std::min<size_t>(ks, c.avail(0) / slice_bytes);
            p.ws = ks >= 2 ? (float *)c.ws : nullptr;
        }
        if (!p.ws)
            ks = 1;
    }
    p.ksplit = ks;
    int st = launch_tiles<dgk::kDense, C, F>(p, ks, c);
    if (st != DG_OK || ks == 1 || c.dry)
        return st;
    const int64_t quads = (int64_t)p.M * (p.N / 4);
    hipLaunchKernelGGL(dgk::splitk_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, c.stream,
                       p.ws, ks, p.M, p.N, p.D, p.ldd);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : fail_hip(e);
}

// Rounds of 256x256 tiles: when the last round of a tiles_m x tiles_n grid
// would be at most half full, the grid can be cut into a part of whole
// rounds and a strip that a second launch covers with smaller tiles (the
// per-element arithmetic does not depend on the tile shape). Returns the
// number of leading n-tiles (cut_n) or else m-tiles (cut_m) of the
// whole-round part, or 0 for no cut. Only dense grids are cut: on the
// contiguous layout a row cut measured slower than the partly filled round.
struct TileCut {
    int64_t cut_n = 0, cut_m = 0;
};
TileCut round_cut(int64_t tiles_m, int64_t tiles_n, int cus)
{
    TileCut c;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t tail = tiles % cus;
    if (tile_override() == 18 || tiles < cus || tail == 0 || tail * 2 > cus)
        return c;
    for (int64_t n1 = tiles_n - 1; n1 > 0; --n1)
        if ((tiles_m * n1) % cus == 0) {
            c.cut_n = n1;
            return c;
        }
    for (int64_t m1 = tiles_m - 1; m1 > 0; --m1)
        if ((m1 * tiles_n) % cus == 0) {
            c.cut_m = m1;
            return c;
        }
    return c;
}

// Dense GEMM, configuration chosen from the shape: 256x256 tiles while they
// fill the CUs (a last round at most half full is cut off and run with
// smaller tiles); below that, smaller tiles split over K.
template <int F = 0>
int launch_dense_auto(dgk::Params &p, Ctx &cx)
{
    const bool wide_n = p.N % 256 == 0;
    const int64_t tiles_m = (p.M + 255) / 256, tiles_n = p.N / 256;
    if (wide_n && tiles_m * tiles_n * 2 > cx.cus) {
        const TileCut c = round_cut(tiles_m, tiles_n, cx.cus);
        if (c.cut_n == 0 && c.cut_m == 0)
            return launch_dense<CfgBig, F>(p, cx);
        dgk::Params main = p, rest = p;
        if (c.cut_n) {  // columns [0, N1) whole rounds; the rest on 256x128 tiles
            const int64_t N1 = 256 * c.cut_n;
            main.N = (int)N1;
            rest.B += N1 * p.ldb;
            rest.sB += (N1 / 128) * p.sb_nb;
            rest.D += N1;
            rest.N = p.N - (int)N1;
        } else {        // rows [0, M1) whole rounds
            const int64_t M1 = 256 * c.cut_m;
            main.M = (int)M1;
            rest.A += M1 * p.lda;
            rest.sA += M1 * p.sa_m;
            rest.D += M1 * p.ldd;
            rest.M = p.M - (int)M1;
        }
        // the two launches run in stream order, so the strip may reuse the workspace
        const int st = launch_dense<CfgBig, F>(main, cx);
        if (st != DG_OK)
            return st;
        return c.cut_n ? launch_dense<CfgDense, F>(rest, cx) : launch_dense_auto<F>(rest, cx);
    }
    if (p.M <= 128)
        return launch_dense<CfgNarrow, F>(p, cx);
    return launch_dense<CfgDense, F>(p, cx);
}

// Per-lane DMA offsets are 32-bit: a tile's rows of A, B and sA must span < 2^32 bytes.
bool offsets_fit(int64_t lda, int64_t ldb, int64_t sa_stride_m)
{
    return lda <= (1 << 22) && ldb <= (1 << 22) && sa_stride_m <= (1 << 20);
}

// LDS bytes of decode_dma_kernel<NB, MR, true>: LHS staging, B ring, sA.
constexpr int decode_dma_lds(int nb, int mr)
{
    return dgk::kDecodeWaves * (nb * mr * 128 + 2 * 2048 + ((mr * nb + 63) / 64) * 64 * 4);
}

// decode_dma_kernel for NB K blocks per wave and MR staged LHS rows; false if
// that instantiation does not fit the LDS.
template <int MR, int MP = 1>
bool launch_decode_dma(const dgk::Params &p, int nb, bool full, const Ctx &c)
{
    hipStream_t stream = c.stream;
    const dim3 g(p.N / 16), b(dgk::kDecodeThreads);
    bool done = false;
    auto one = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        // more than 8 blocks per wave only in one pass (B fragments are not
        // kept in registers across passes then)
        if constexpr (decode_dma_lds(NB, MR) <= 160 * 1024 && MP * 1024 <= NB * MR * 128 && (MP == 1 || NB <= 8)) {
            if (nb != NB)
                return;
            done = true;
            if (c.dry)
                return;
            if (full && (p.ldb & 4095) == 0)   // rotated block order (see the kernel)
                hipLaunchKernelGGL((dgk::decode_dma_kernel<NB, MR, true, MP, true>), g, b, 0, stream, p);
            else if (full)
                hipLaunchKernelGGL((dgk::decode_dma_kernel<NB, MR, true, MP>), g, b, 0, stream, p);
            else
                hipLaunchKernelGGL((dgk::decode_dma_kernel<NB, MR, false, MP>), g, b, 0, stream, p);
        }
    };
    one(std::integral_constant<int, 1>{});
    one(std::integral_constant<int, 2>{});
    one(std::integral_constant<int, 3>{});
    one(std::integral_constant<int, 4>{});
    one(std::integral_constant<int, 5>{});
    one(std::integral_constant<int, 6>{});
    one(std::integral_constant<int, 7>{});
    one(std::integral_constant<int, 8>{});
    one(std::integral_constant<int, 9>{});
    one(std::integral_constant<int, 10>{});
    one(std::integral_constant<int, 11>{});
    one(std::integral_constant<int, 12>{});
    one(std::integral_constant<int, 13>{});
    one(std::integral_constant<int, 14>{});
    one(std::integral_constant<int, 15>{});
    return done;
}

// Returned by launch_decode when it leaves the problem to the tile kernel.
constexpr int kDecodeDeclined = -1;

// Small-M kernels. The LHS-staging kernel (up to 4 passes of 16 rows) is
// tried first; when its LDS does not fit the shape, the older decode kernels
// run if `fallback` (M <= 24 or short K), else kDecodeDeclined.
int launch_decode(dgk::Params &p, const Ctx &c, bool fallback)
{
    hipStream_t stream = c.stream;
    const int grid = p.N / 16;
    hipError_t e;
    const int64_t nkb = p.K / 128;
    const bool dma_ok = nkb % dgk::kDecodeWaves == 0 && nkb / dgk::kDecodeWaves <= 15 &&
                        (tile_override() < 7 || tile_override() > 9) &&
                        (int64_t)(p.M - 1) * p.lda + p.K < ((int64_t)1 << 31) &&
                        ((int64_t)(p.M - 1) * p.sa_m + (nkb - 1) * p.sa_kb) * 4 < ((int64_t)1 << 31);
    const int nb = (int)(nkb / dgk::kDecodeWaves);
    const bool full = tile_override() != 6;
    if (dma_ok && p.M <= 8 && launch_decode_dma<8>(p, nb, full, c)) {
    } else if (dma_ok && p.M <= 16 && launch_decode_dma<16>(p, nb, full, c)) {
    } else if (dma_ok && p.M <= 32 && launch_decode_dma<16, 2>(p, nb, full, c)) {
    } else if (dma_ok && p.M <= 48 && launch_decode_dma<16, 3>(p, nb, full, c)) {
    } else if (dma_ok && p.M <= 64 && launch_decode_dma<16, 4>(p, nb, full, c)) {
    } else if (!fallback) {
        return kDecodeDeclined;
    } else if (c.dry) {
        return DG_OK;   // one of the older decode kernels below; they take no workspace
    } else if (p.M <= 16 && nkb % dgk::kDecodeWaves == 0 && nkb / dgk::kDecodeWaves <= 8 && tile_override() != 7 &&
        tile_override() != 8) {
        const dim3 g(grid), b(dgk::kDecodeThreads);
        switch (nkb / dgk::kDecodeWaves) {
        case 1: hipLaunchKernelGGL(dgk::decode_static_kernel<1>, g, b, 0, stream, p); break;
        case 2: hipLaunchKernelGGL(dgk::decode_static_kernel<2>, g, b, 0, stream, p); break;
        case 3: hipLaunchKernelGGL(dgk::decode_static_kernel<3>, g, b, 0, stream, p); break;
        case 4: hipLaunchKernelGGL(dgk::decode_static_kernel<4>, g, b, 0, stream, p); break;
        case 5: hipLaunchKernelGGL(dgk::decode_static_kernel<5>, g, b, 0, stream, p); break;
        case 6: hipLaunchKernelGGL(dgk::decode_static_kernel<6>, g, b, 0, stream, p); break;
        case 7: hipLaunchKernelGGL(dgk::decode_static_kernel<7>, g, b, 0, stream, p); break;
        default: hipLaunchKernelGGL(dgk::decode_static_kernel<8>, g, b, 0, stream, p); break;
        }
    } else if (p.M <= 16 && (int64_t)p.M * p.K <= dgk::kDecodeLdsA && (int64_t)p.M * nkb <= dgk::kDecodeLdsSa &&
        ((int64_t)p.M * p.K) % 1024 == 0 && (int64_t)(p.M - 1) * p.lda + p.K < ((int64_t)1 << 31) &&
        ((int64_t)(p.M - 1) * p.sa_m + (nkb - 1) * p.sa_kb) * 4 < ((int64_t)1 << 31) && tile_override() != 7)
        hipLaunchKernelGGL(dgk::decode_lds_kernel, dim3(grid), dim3(dgk::kDecodeThreads), 0, stream, p);
    else if (p.M <= 16)
        hipLaunchKernelGGL(dgk::decode_kernel<1>, dim3(grid), dim3(dgk::kDecodeThreads), 0, stream, p);
    else if (p.M <= 32)
        hipLaunchKernelGGL(dgk::decode_kernel<2>, dim3(grid), dim3(dgk::kDecodeThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(dgk::decode_kernel<4>, dim3(grid), dim3(dgk::kDecodeThreads), 0, stream, p);
    if (c.dry)
        return DG_OK;
    e = hipGetLastError();
    return e == hipSuccess ? DG_OK : fail_hip(e);
}

// The quantiser; src_rows (optional) names the row of X that each output row
// reads (a gathered layout), x_rows the rows of X.
int quantize_impl(const void *X, int x_dtype, int64_t ldx, int64_t x_rows, const int32_t *src_rows, void *Q,
                  int64_t ldq, float *S, int64_t s_stride_m, int64_t s_stride_kb, int64_t M, int64_t K,
                  void *stream)
{
    if (M < 0 || K <= 0 || K % 128 != 0)
        return DG_ERR_BAD_SHAPE;
    if (x_dtype != DG_DTYPE_F32 && x_dtype != DG_DTYPE_BF16)
        return DG_ERR_UNSUPPORTED;
    if (M > kInt32Max || K > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (M == 0)
        return DG_OK;
    if ((x_rows > 0 && !X) || !Q || !S)
        return DG_ERR_NULL_POINTER;
    const int64_t nkb = K / 128;
    // Every (m, kb) must own its scale: a row-major-like or an M-major-like
    // layout (a dimension of extent 1 may take any stride).
    const bool rows_distinct = M == 1 || s_stride_m >= 1;
    const bool blocks_distinct = nkb == 1 || s_stride_kb >= 1;
    const bool row_major = s_stride_m >= (nkb - 1) * s_stride_kb + 1 || M == 1;
    const bool m_major = s_stride_kb >= (M - 1) * s_stride_m + 1 || nkb == 1;
    if (ldx < K || ldq < K || s_stride_m < 0 || s_stride_kb < 0 || !rows_distinct || !blocks_distinct ||
        !(row_major || m_major))
        return DG_ERR_BAD_STRIDE;
    const int64_t esize = x_dtype == DG_DTYPE_F32 ? 4 : 2;
    if (!aligned(X, 16) || !aligned(Q, 16) || (ldx * esize) % 16 || ldq % 16 || !aligned(S, 4))
        return DG_ERR_MISALIGNED;
    const Extent eq = extent(Q, 1, (M - 1) * ldq + K - 1);
    const Extent es = extent(S, 4, last_scale_index(M, nkb, s_stride_m, s_stride_kb));
    if (overlaps(eq, es))
        return DG_ERR_ALIASING;
    if (x_rows > 0) {
        const Extent ex = extent(X, esize, (x_rows - 1) * ldx + K - 1);
        if (overlaps(eq, ex) || overlaps(es, ex))
            return DG_ERR_ALIASING;
    }
    if (src_rows) {
        const Extent ei = extent(src_rows, 4, M - 1);
        if (overlaps(eq, ei) || overlaps(es, ei))
            return DG_ERR_ALIASING;
    }
    const int64_t span_len = 1024 * (x_dtype == DG_DTYPE_BF16 ? dgq::groups_per_wave<true>()
                                                             : dgq::groups_per_wave<false>());
    const int64_t spans = (K + span_len - 1) / span_len;
    const int64_t units = M * spans;
    const int64_t groups = (units + dgq::kWavesPerGroup - 1) / dgq::kWavesPerGroup;
    if (groups > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    DeviceInfo dev;
    int st = current_device(dev);
    if (st != DG_OK)
        return st;

    dgq::QuantParams p = {};
    p.X = X; p.ldx = ldx; p.src_rows = src_rows; p.x_rows = x_rows;
    p.Q = (uint8_t *)Q; p.ldq = ldq;
    p.S = S; p.s_m = s_stride_m; p.s_kb = s_stride_kb;
    p.M = (int)M; p.K = (int)K; p.spans = (int)spans; p.units = units;
    const dim3 grid((unsigned)groups), block(64 * dgq::kWavesPerGroup);
    if (x_dtype == DG_DTYPE_BF16)
        hipLaunchKernelGGL(dgq::quantize_1x128_kernel<true>, grid, block, 0, (hipStream_t)stream, p);
    else
        hipLaunchKernelGGL(dgq::quantize_1x128_kernel<false>, grid, block, 0, (hipStream_t)stream, p);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : fail_hip(e);
}

// A caller workspace must be 16-byte aligned, have a non-negative size and
// lie apart from the call's output and inputs.
int check_workspace(const void *ws, int64_t ws_bytes, std::initializer_list<Extent> others)
{
    if (ws_bytes < 0)
        return DG_ERR_BAD_SHAPE;
    if (!ws || ws_bytes == 0)
        return DG_OK;
    if (!aligned(ws, 16))
        return DG_ERR_MISALIGNED;
    const Extent ew = extent(ws, 1, ws_bytes - 1);
    for (const Extent &e : others)
        if (e.hi > e.lo && overlaps(ew, e))
            return DG_ERR_ALIASING;
    return DG_OK;
}

// Validation and kernel arguments of a dense call. Returns DG_OK with `p`
// and `dev` filled, kEmptyProblem for an empty problem, or an error.
constexpr int kEmptyProblem = -2;

int dense_setup(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                const void *B, int64_t ldb, const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                void *D, int64_t ldd, int64_t M, int64_t N, int64_t K, dgk::Params &p, DeviceInfo &dev,
                const void *workspace = nullptr, int64_t ws_bytes = 0)
{
    if (ws_bytes < 0)
        return DG_ERR_BAD_SHAPE;
    int st = check_common_shape(M, N, K);
    if (st != DG_OK)
        return st;
    if (M == 0 || N == 0)
        return kEmptyProblem;
    if (!A || !sA || !B || !sB || !D)
        return DG_ERR_NULL_POINTER;
    if (lda < K || ldb < K || ldd < N || sa_stride_m < 0 || sa_stride_kb < 0 || sb_stride_nb < 0 ||
        sb_stride_kb < 0)
        return DG_ERR_BAD_STRIDE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || lda % 16 || ldb % 16 || ldd % 8 ||
        !aligned(sA, 4) || !aligned(sB, 4))
        return DG_ERR_MISALIGNED;
    const int64_t nkb = K / 128;
    const Extent ed = extent(D, 2, (M - 1) * ldd + N - 1);
    const Extent ea = extent(A, 1, (M - 1) * lda + K - 1), eb = extent(B, 1, (N - 1) * ldb + K - 1);
    const Extent esa = extent(sA, 4, last_scale_index(M, nkb, sa_stride_m, sa_stride_kb));
    const Extent esb = extent(sB, 4, last_scale_index(N / 128, nkb, sb_stride_nb, sb_stride_kb));
    if (overlaps(ed, ea) || overlaps(ed, eb) || overlaps(ed, esa) || overlaps(ed, esb))
        return DG_ERR_ALIASING;
    if ((st = check_workspace(workspace, ws_bytes, {ed, ea, eb, esa, esb})) != DG_OK)
        return st;
    if ((st = current_device(dev)) != DG_OK)
        return st;

    p = dgk::Params{};
    p.A = (const uint8_t *)A; p.lda = lda;
    p.sA = sA; p.sa_m = sa_stride_m; p.sa_kb = sa_stride_kb;
    p.B = (const uint8_t *)B; p.ldb = ldb;
    p.sB = sB; p.sb_nb = sb_stride_nb; p.sb_kb = sb_stride_kb;
    p.D = (uint16_t *)D; p.ldd = ldd;
    p.M = (int)M; p.N = (int)N; p.K = (int)K; p.G = 1;
    return DG_OK;
}

// Kernel choice and launches of the contiguous grouped GEMM (arguments
// already validated; in a dry run only the workspace need is recorded).
// scatter: rows go to token order (p.row_dst); fmt as for launch_tiles_fmt.
int contiguous_dispatch(dgk::Params &p, Ctx &c, bool scatter, int fmt)
{
    const int64_t N = p.N, G = p.G;
    const int ov = tile_override();  // 24: no derivation; 2, 3, 4 force the uniform grid's tile shape
    if (p.layout) {
        const bool wide = N % 256 == 0;
        if (scatter)
            return wide ? launch_contiguous_seg<CfgBig, CfgTail, true>(p, c, 0)
                        : launch_contiguous_seg<CfgDense, CfgNarrow, true>(p, c, 0);
        return wide ? (ov == 27 ? launch_contiguous_seg<CfgBig, CfgTail, false>(p, c, 0)
                                : launch_contiguous_seg<CfgBigE, CfgTail, false>(p, c, 0))
                    : launch_contiguous_seg<CfgDense, CfgNarrow, false>(p, c, 0);
    }
    // Only the ids given: with workspace for the offsets, derive the segment
    // offsets on the device and tile along them (e4m3, 256-wide tiles, at
    // most 4096 blocks of 128 rows). If the ids' experts are not in ascending
    // order, the derivation flags it and the segment launch of whole tiles
    // covers the rows on the uniform grid instead. Up to 128 experts: at 8192
    // tokens, N 4096, K 7168 this measured 9-31% faster than the uniform grid
    // for 8-64 experts and 2% faster at 128; at 256 (every segment one
    // 128-row block) it was 2% slower, the per-tile segment search then
    // outweighing the saved two-expert passes. Workspace: the offsets first
    // (G + 2 int32), then the split tails' partial sums.
    if (!fmt && N % 256 == 0 && G <= kDeriveMaxExperts && p.M / 128 <= dgm::kDeriveMaxBlocks && ov != 24 &&
        ov != 2 && ov != 3 && ov != 4) {
        const size_t aux_bytes = ws_round((size_t)(G + 2) * sizeof(int32_t));
        int32_t *aux = (int32_t *)c.take(0, aux_bytes);
        if (aux || c.dry) {
            if (!c.dry) {
                dgm::DeriveParams dp = {p.ids, p.M, p.G, aux, aux + G + 1};
                hipLaunchKernelGGL(dgm::derive_layout_kernel, dim3(1), dim3(dgm::kRouteThreads), 0, c.stream, dp);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return fail_hip(e);
            }
            dgk::Params q = p;
            q.layout = aux;
            q.gate = aux ? aux + G + 1 : nullptr;
            return scatter ? launch_contiguous_seg<CfgBig, CfgTail, true>(q, c, aux_bytes)
                 : ov == 27 ? launch_contiguous_seg<CfgBig, CfgTail, false>(q, c, aux_bytes)
                            : launch_contiguous_seg<CfgBigE, CfgTail, false>(q, c, aux_bytes);
        }
    }
    if (scatter) {
        if (N % 256 == 0)
            return launch_tiles<dgk::kContiguous, CfgBig, 0, true>(p, 1, c);
        return launch_tiles<dgk::kContiguous, CfgDense, 0, true>(p, 1, c);
    }
    if (fmt) {
        if (N % 256 == 0)
            return launch_tiles_fmt<dgk::kContiguous, CfgBig>(p, 1, c, fmt);
        return launch_tiles_fmt<dgk::kContiguous, CfgDense>(p, 1, c, fmt);
    }
    switch (ov) {
    case 2: return launch_tiles<dgk::kContiguous, CfgNarrow>(p, 1, c);
    case 3: return launch_tiles<dgk::kContiguous, CfgWide>(p, 1, c);
    case 4: return launch_tiles<dgk::kContiguous, CfgDense>(p, 1, c);
    default:
        if (N % 256 == 0)
            return launch_tiles<dgk::kContiguous, CfgBig>(p, 1, c);
        return launch_tiles<dgk::kContiguous, CfgDense>(p, 1, c);
    }
}

// The contiguous grouped GEMM. With token_of_row, row r of the result is
// written to row token_of_row[r] of D (D has d_rows rows); without it, to row r
// (d_rows = M_total). workspace / ws_bytes: the caller's scratch memory (may
// be null / 0).
int contiguous_impl(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                    const void *B, int64_t ldb, int64_t b_stride_g, const float *sB, int64_t sb_stride_g,
                    int64_t sb_stride_nb, int64_t sb_stride_kb, const int32_t *expert_ids,
                    const int32_t *token_of_row, void *D, int64_t ldd, int64_t d_rows, int64_t M_total, int64_t N,
                    int64_t K, int64_t G, void *stream, int fmt = 0, const int32_t *layout = nullptr,
                    void *workspace = nullptr, int64_t ws_bytes = 0)
{
    int st = check_common_shape(M_total, N, K);
    if (st != DG_OK)
        return st;
    if (G < 0 || M_total % 128 != 0)
        return DG_ERR_BAD_SHAPE;
    if (G > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (d_rows < 0 || ws_bytes < 0)
        return DG_ERR_BAD_SHAPE;
    if (d_rows > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (M_total == 0 || N == 0 || G == 0 || d_rows == 0)
        return DG_OK;
    if (!A || !sA || !B || !sB || !expert_ids || !D)
        return DG_ERR_NULL_POINTER;
    if ((token_of_row && !aligned(token_of_row, 4)) || (layout && !aligned(layout, 4)))
        return DG_ERR_MISALIGNED;
    if (layout && G > dgm::kMaxExperts)
        return DG_ERR_UNSUPPORTED;
    if (lda < K || ldb < K || ldd < N || sa_stride_m < 0 || sa_stride_kb < 0 || sb_stride_nb < 0 ||
        sb_stride_kb < 0 || sb_stride_g < 0 || (G > 1 && b_stride_g < (N - 1) * ldb + K))
        return DG_ERR_BAD_STRIDE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || lda % 16 || ldb % 16 || b_stride_g % 16 ||
        ldd % 8 || !aligned(sA, 4) || !aligned(sB, 4) || !aligned(expert_ids, 4))
        return DG_ERR_MISALIGNED;
    const int64_t nkb = K / 128;
    const Extent ed = extent(D, 2, (d_rows - 1) * ldd + N - 1);
    if ((token_of_row && overlaps(ed, extent(token_of_row, 4, M_total - 1))) ||
        (layout && overlaps(ed, extent(layout, 4, G))))
        return DG_ERR_ALIASING;
    const Extent ea = extent(A, 1, (M_total - 1) * lda + K - 1);
    const Extent eb = extent(B, 1, (G - 1) * b_stride_g + (N - 1) * ldb + K - 1);
    const Extent esa = extent(sA, 4, last_scale_index(M_total, nkb, sa_stride_m, sa_stride_kb));
    const Extent esb = extent(sB, 4, (G - 1) * sb_stride_g + last_scale_index(N / 128, nkb, sb_stride_nb, sb_stride_kb));
    const Extent eid = extent(expert_ids, 4, M_total - 1);
    if (overlaps(ed, ea) || overlaps(ed, eb) || overlaps(ed, esa) || overlaps(ed, esb) || overlaps(ed, eid))
        return DG_ERR_ALIASING;
    const Extent none{0, 0};
    st = check_workspace(workspace, ws_bytes,
                         {ed, ea, eb, esa, esb, eid, token_of_row ? extent(token_of_row, 4, M_total - 1) : none,
                          layout ? extent(layout, 4, G) : none});
    if (st != DG_OK)
        return st;
    DeviceInfo dev;
    if ((st = current_device(dev)) != DG_OK)
        return st;

    dgk::Params p = {};
    p.A = (const uint8_t *)A; p.lda = lda;
    p.sA = sA; p.sa_m = sa_stride_m; p.sa_kb = sa_stride_kb;
    p.B = (const uint8_t *)B; p.ldb = ldb; p.b_stride_g = b_stride_g;
    p.sB = sB; p.sb_nb = sb_stride_nb; p.sb_kb = sb_stride_kb; p.sb_g = sb_stride_g;
    p.D = (uint16_t *)D; p.ldd = ldd;
    p.ids = expert_ids;
    p.row_dst = token_of_row; p.dst_rows = (int)d_rows;
    p.layout = layout;
    p.M = (int)M_total; p.N = (int)N; p.K = (int)K; p.G = (int)G;
    if (!offsets_fit(lda, ldb, sa_stride_m))
        return DG_ERR_UNSUPPORTED;
    Ctx c;
    c.cus = dev.cus;
    c.stream = (hipStream_t)stream;
    c.ws = (uint8_t *)workspace;
    c.ws_bytes = workspace ? (size_t)ws_bytes : 0;
    return contiguous_dispatch(p, c, token_of_row != nullptr, fmt);
}

// The masked grouped GEMM; fmt as for launch_tiles_fmt.
int masked_impl(const void *A, int64_t lda, int64_t a_stride_g, const float *sA, int64_t sa_stride_g,
                int64_t sa_stride_m, int64_t sa_stride_kb, const void *B, int64_t ldb, int64_t b_stride_g,
                const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb, int64_t sb_stride_kb,
                const int32_t *masked_m, void *D, int64_t ldd, int64_t d_stride_g, int64_t G, int64_t M_max,
                int64_t N, int64_t K, void *stream, int fmt)
{
    int st = check_common_shape(M_max, N, K);
    if (st != DG_OK)
        return st;
    if (G < 0)
        return DG_ERR_BAD_SHAPE;
    if (G > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0)
        return DG_OK;
    if (!A || !sA || !B || !sB || !masked_m || !D)
        return DG_ERR_NULL_POINTER;
    if (lda < K || ldb < K || ldd < N || sa_stride_m < 0 || sa_stride_kb < 0 || sa_stride_g < 0 ||
        sb_stride_nb < 0 || sb_stride_kb < 0 || sb_stride_g < 0 ||
        (G > 1 && (a_stride_g < (M_max - 1) * lda + K || b_stride_g < (N - 1) * ldb + K ||
                   d_stride_g < (M_max - 1) * ldd + N)))
        return DG_ERR_BAD_STRIDE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || lda % 16 || ldb % 16 || a_stride_g % 16 ||
        b_stride_g % 16 || ldd % 8 || d_stride_g % 8 || !aligned(sA, 4) || !aligned(sB, 4) ||
        !aligned(masked_m, 4))
        return DG_ERR_MISALIGNED;
    const int64_t nkb = K / 128;
    const Extent ed = extent(D, 2, (G - 1) * d_stride_g + (M_max - 1) * ldd + N - 1);
    if (overlaps(ed, extent(A, 1, (G - 1) * a_stride_g + (M_max - 1) * lda + K - 1)) ||
        overlaps(ed, extent(B, 1, (G - 1) * b_stride_g + (N - 1) * ldb + K - 1)) ||
        overlaps(ed, extent(sA, 4, (G - 1) * sa_stride_g + last_scale_index(M_max, nkb, sa_stride_m, sa_stride_kb))) ||
        overlaps(ed, extent(sB, 4, (G - 1) * sb_stride_g + last_scale_index(N / 128, nkb, sb_stride_nb, sb_stride_kb))) ||
        overlaps(ed, extent(masked_m, 4, G - 1)))
        return DG_ERR_ALIASING;
    DeviceInfo dev;
    if ((st = current_device(dev)) != DG_OK)
        return st;

    dgk::Params p = {};
    p.A = (const uint8_t *)A; p.lda = lda; p.a_stride_g = a_stride_g;
    p.sA = sA; p.sa_m = sa_stride_m; p.sa_kb = sa_stride_kb; p.sa_g = sa_stride_g;
    p.B = (const uint8_t *)B; p.ldb = ldb; p.b_stride_g = b_stride_g;
    p.sB = sB; p.sb_nb = sb_stride_nb; p.sb_kb = sb_stride_kb; p.sb_g = sb_stride_g;
    p.D = (uint16_t *)D; p.ldd = ldd; p.d_stride_g = d_stride_g;
    p.masked_m = masked_m;
    p.M = (int)M_max; p.N = (int)N; p.K = (int)K; p.G = (int)G;
    if (!offsets_fit(lda, ldb, sa_stride_m))
        return DG_ERR_UNSUPPORTED;
    Ctx c;
    c.cus = dev.cus;
    c.stream = (hipStream_t)stream;
    if (fmt) {
        if (N % 256 == 0)
            return launch_tiles_fmt<dgk::kMasked, CfgBigStreamB>(p, (int)G, c, fmt);
        return launch_tiles_fmt<dgk::kMasked, CfgDense>(p, (int)G, c, fmt);
    }
    switch (tile_override()) {
    case 1: return launch_tiles<dgk::kMasked, CfgDense4>(p, (int)G, c);
    case 2: return launch_tiles<dgk::kMasked, CfgNarrow>(p, (int)G, c);
    case 4: return launch_tiles<dgk::kMasked, CfgDense>(p, (int)G, c);
    case 12: return N % 256 == 0 ? launch_tiles<dgk::kMasked, CfgBig>(p, (int)G, c)
                                 : DG_ERR_UNSUPPORTED;
    default:
        if (N % 256 == 0)
            return launch_tiles<dgk::kMasked, CfgBigStreamB>(p, (int)G, c);
        return launch_tiles<dgk::kMasked, CfgDense>(p, (int)G, c);
    }
}

// Kernel choice and launches of the dense e4m3 GEMM (arguments validated;
// in a dry run only the workspace need is recorded).
int dense_dispatch(dgk::Params &p, Ctx &c)
{
    const int64_t M = p.M, nkb = p.K / 128;
    // M <= 64: the decode kernels (B streamed once per launch, the LHS staged
    // per wave 16 rows at a time). Where their LDS staging does not fit the
    // shape, the older decode kernels keep M <= 24 and short K (< 16 blocks:
    // a split-K launch pair costs more than it saves); the rest, and all
    // larger M, go to the tile kernel, split over K when its tiles are few
    // and the workspace holds the partial sums.
    const bool forced_tiles = tile_override() == 1 || tile_override() == 2 || tile_override() == 4;
    const int64_t decode_max_m = tile_override() == 13 ? 16 : 64;
    if (M <= decode_max_m && !forced_tiles) {
        const int st = launch_decode(p, c, M <= 24 || nkb < 16 || tile_override() == 14);
        if (st != kDecodeDeclined)
            return st;
    }
    if (!offsets_fit(p.lda, p.ldb, p.sa_m))
        return DG_ERR_UNSUPPORTED;
    const bool wide_n = p.N % 256 == 0;
    switch (tile_override()) {
    case 1: return launch_tiles<dgk::kDense, CfgDense4>(p, 1, c);
    case 2: return launch_tiles<dgk::kDense, CfgNarrow>(p, 1, c);
    case 4: return launch_tiles<dgk::kDense, CfgDense>(p, 1, c);
    case 15: return wide_n ? launch_dense<CfgBig>(p, c) : launch_dense<CfgDense>(p, c);
    default:
        return launch_dense_auto(p, c);
    }
}

}  // namespace

extern "C" {

int dg_abi_version(void) { return DG_ABI_VERSION; }

const char *dg_status_string(dg_status status)
{
    switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_NULL_POINTER: return "a required pointer is NULL";
    case DG_ERR_BAD_SHAPE: return "bad shape (need K > 0, K % 128 == 0, N % 128 == 0, M_total % 128 == 0, dims >= 0)";
    case DG_ERR_MISALIGNED: return "misaligned pointer or stride (16-byte operands/strides, 4-byte scales)";
    case DG_ERR_BAD_STRIDE: return "bad stride (lda/ldb >= K, ldd >= N, non-negative, group strides cover a group)";
    case DG_ERR_UNSUPPORTED: return "unsupported device (gfx950 required) or size beyond int32";
    case DG_ERR_HIP: return "HIP runtime error (see dg_last_hip_error)";
    case DG_ERR_ALIASING: return "output (or workspace) overlaps an input or the output";
    case DG_ERR_SCRATCH: return "the problem needs more scratch than the library's static buffer holds (use the _ws call)";
    default: return "unknown status";
    }
}

int dg_last_hip_error(void) { return g_last_hip_error; }

dg_status dg_fp8_gemm_nt(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                         const void *B, int64_t ldb, const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                         void *D, int64_t ldd, int64_t M, int64_t N, int64_t K, void *stream)
{
    return dg_fp8_gemm_nt_ws(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, sB, sb_stride_nb, sb_stride_kb, D, ldd,
                             M, N, K, nullptr, 0, stream);
}

dg_status dg_fp8_gemm_nt_ws(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m, int64_t sa_stride_kb,
                            const void *B, int64_t ldb, const float *sB, int64_t sb_stride_nb, int64_t sb_stride_kb,
                            void *D, int64_t ldd, int64_t M, int64_t N, int64_t K, void *workspace,
                            int64_t workspace_bytes, void *stream)
{
    dgk::Params p;
    DeviceInfo dev;
    int st = dense_setup(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, sB, sb_stride_nb, sb_stride_kb, D, ldd,
                         M, N, K, p, dev, workspace, workspace_bytes);
    if (st != DG_OK)
        return (dg_status)(st == kEmptyProblem ? DG_OK : st);
    Ctx c;
    c.cus = dev.cus;
    c.stream = (hipStream_t)stream;
    c.ws = (uint8_t *)workspace;
    c.ws_bytes = workspace ? (size_t)workspace_bytes : 0;
    return (dg_status)dense_dispatch(p, c);
}

int64_t dg_fp8_gemm_nt_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    int st = check_common_shape(M, N, K);
    if (st != DG_OK)
        return -st;
    if (M == 0 || N == 0)
        return 0;
    DeviceInfo dev;
    if ((st = current_device(dev)) != DG_OK)
        return -st;
    dgk::Params p = {};
    p.lda = K; p.ldb = K; p.ldd = N;
    p.sa_m = 1; p.sa_kb = M; p.sb_nb = K / 128; p.sb_kb = 1;  // the generator's (contiguous) layouts
    p.M = (int)M; p.N = (int)N; p.K = (int)K; p.G = 1;
    Ctx c;
    c.cus = dev.cus;
    c.dry = true;
    st = dense_dispatch(p, c);
    return st == DG_OK ? (int64_t)c.need : -st;
}

dg_status dg_fp8_grouped_gemm_contiguous(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m,
                                   int64_t sa_stride_kb, const void *B, int64_t ldb, int64_t b_stride_g,
                                   const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb, int64_t sb_stride_kb,
                                   const int32_t *expert_ids, void *D, int64_t ldd, int64_t M_total, int64_t N,
                                   int64_t K, int64_t G, void *stream)
{
    return (dg_status)contiguous_impl(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB, sb_stride_g,
                           sb_stride_nb, sb_stride_kb, expert_ids, nullptr, D, ldd, M_total, M_total, N, K, G,
                           stream);
}

dg_status dg_fp8_grouped_gemm_contiguous_to_tokens(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m,
                                             int64_t sa_stride_kb, const void *B, int64_t ldb, int64_t b_stride_g,
                                             const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                             int64_t sb_stride_kb, const int32_t *expert_ids,
                                             const int32_t *token_of_row, const int32_t *layout, void *out,
                                             int64_t ldo, int64_t T, int64_t M_total, int64_t N, int64_t K,
                                             int64_t G, void *stream)
{
    if (M_total > 0 && N > 0 && G > 0 && T > 0 && !token_of_row)
        return DG_ERR_NULL_POINTER;
    return (dg_status)contiguous_impl(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB, sb_stride_g,
                           sb_stride_nb, sb_stride_kb, expert_ids, token_of_row, out, ldo, T, M_total, N, K, G,
                           stream, 0, layout);
}

dg_status dg_fp8_grouped_gemm_contiguous_layout(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m,
                                          int64_t sa_stride_kb, const void *B, int64_t ldb, int64_t b_stride_g,
                                          const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                          int64_t sb_stride_kb, const int32_t *expert_ids, const int32_t *layout,
                                          void *D, int64_t ldd, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                          void *stream)
{
    if (M_total > 0 && N > 0 && G > 0 && !layout)
        return DG_ERR_NULL_POINTER;
    return (dg_status)contiguous_impl(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB, sb_stride_g,
                           sb_stride_nb, sb_stride_kb, expert_ids, nullptr, D, ldd, M_total, M_total, N, K, G,
                           stream, 0, layout);
}

dg_status dg_fp8_gemm_nt_noalloc(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m,
                                 int64_t sa_stride_kb, const void *B, int64_t ldb, const float *sB,
                                 int64_t sb_stride_nb, int64_t sb_stride_kb, void *D, int64_t ldd, int64_t M,
                                 int64_t N, int64_t K, void *stream)
{
    dgk::Params p;
    DeviceInfo dev;
    int st = dense_setup(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, sB, sb_stride_nb, sb_stride_kb, D, ldd,
                         M, N, K, p, dev);
    if (st != DG_OK)
        return (dg_status)(st == kEmptyProblem ? DG_OK : st);
    // What the fastest path takes, for these exact arguments (a dry run).
    Ctx q;
    q.cus = dev.cus;
    q.dry = true;
    dgk::Params pq = p;
    if ((st = dense_dispatch(pq, q)) != DG_OK)
        return (dg_status)st;
    if (q.need > kScratchBytes)
        return DG_ERR_SCRATCH;
    uint8_t *ws = nullptr;
    if (q.need > 0 && !(ws = device_scratch(st)))
        return (dg_status)st;
    // The split-K partial sums are written before they are read, so nothing
    // in the array needs clearing between calls.
    Ctx c;
    c.cus = dev.cus;
    c.stream = (hipStream_t)stream;
    c.ws = ws;
    c.ws_bytes = ws ? kScratchBytes : 0;
    return (dg_status)dense_dispatch(p, c);
}

dg_status dg_fp8_grouped_gemm_contiguous_ws(const void *A, int64_t lda, const float *sA, int64_t sa_stride_m,
                                             int64_t sa_stride_kb, const void *B, int64_t ldb, int64_t b_stride_g,
                                             const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                                             int64_t sb_stride_kb, const int32_t *expert_ids,
                                             const int32_t *token_of_row, const int32_t *layout, void *D,
                                             int64_t ldd, int64_t T, int64_t M_total, int64_t N, int64_t K,
                                             int64_t G, void *workspace, int64_t workspace_bytes, void *stream)
{
    return (dg_status)contiguous_impl(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB, sb_stride_g,
                                      sb_stride_nb, sb_stride_kb, expert_ids, token_of_row, D, ldd,
                                      token_of_row ? T : M_total, M_total, N, K, G, stream, 0, layout, workspace,
                                      workspace_bytes);
}

int64_t dg_fp8_grouped_gemm_contiguous_workspace_bytes(int64_t M_total, int64_t N, int64_t K, int64_t G)
{
    int st = check_common_shape(M_total, N, K);
    if (st != DG_OK)
        return -st;
    if (G < 0 || M_total % 128 != 0)
        return -DG_ERR_BAD_SHAPE;
    if (G > kInt32Max)
        return -DG_ERR_UNSUPPORTED;
    if (M_total == 0 || N == 0 || G == 0)
        return 0;
    DeviceInfo dev;
    if ((st = current_device(dev)) != DG_OK)
        return -st;
    dgk::Params p = {};
    p.lda = K; p.ldb = K; p.ldd = N; p.b_stride_g = N * K;
    p.sa_m = 1; p.sa_kb = M_total; p.sb_nb = K / 128; p.sb_kb = 1; p.sb_g = (N / 128) * (K / 128);
    p.M = (int)M_total; p.N = (int)N; p.K = (int)K; p.G = (int)G;
    Ctx c;
    c.cus = dev.cus;
    c.dry = true;
    st = contiguous_dispatch(p, c, false, 0);
    return st == DG_OK ? (int64_t)c.need : -st;
}

dg_status dg_fp8_grouped_gemm_masked(const void *A, int64_t lda, int64_t a_stride_g, const float *sA, int64_t sa_stride_g,
                               int64_t sa_stride_m, int64_t sa_stride_kb, const void *B, int64_t ldb,
                               int64_t b_stride_g, const float *sB, int64_t sb_stride_g, int64_t sb_stride_nb,
                               int64_t sb_stride_kb, const int32_t *masked_m, void *D, int64_t ldd,
                               int64_t d_stride_g, int64_t G, int64_t M_max, int64_t N, int64_t K, void *stream)
{
    return (dg_status)masked_impl(A, lda, a_stride_g, sA, sa_stride_g, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB,
                       sb_stride_g, sb_stride_nb, sb_stride_kb, masked_m, D, ldd, d_stride_g, G, M_max, N, K, stream,
                       0);
}

dg_status dg_fp8_grouped_gemm_masked_fmt(const void *A, int a_fmt, int64_t lda, int64_t a_stride_g, const float *sA,
                                   int64_t sa_stride_g, int64_t sa_stride_m, int64_t sa_stride_kb, const void *B,
                                   int b_fmt, int64_t ldb, int64_t b_stride_g, const float *sB, int64_t sb_stride_g,
                                   int64_t sb_stride_nb, int64_t sb_stride_kb, const int32_t *masked_m, void *D,
                                   int64_t ldd, int64_t d_stride_g, int64_t G, int64_t M_max, int64_t N, int64_t K,
                                   void *stream)
{
    const int f = format_bits(a_fmt, b_fmt);
    if (f < 0)
        return DG_ERR_UNSUPPORTED;
    return (dg_status)masked_impl(A, lda, a_stride_g, sA, sa_stride_g, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB,
                       sb_stride_g, sb_stride_nb, sb_stride_kb, masked_m, D, ldd, d_stride_g, G, M_max, N, K, stream,
                       f);
}

dg_status dg_fp8_grouped_gemm_contiguous_fmt(const void *A, int a_fmt, int64_t lda, const float *sA, int64_t sa_stride_m,
                                       int64_t sa_stride_kb, const void *B, int b_fmt, int64_t ldb,
                                       int64_t b_stride_g, const float *sB, int64_t sb_stride_g,
                                       int64_t sb_stride_nb, int64_t sb_stride_kb, const int32_t *expert_ids,
                                       void *D, int64_t ldd, int64_t M_total, int64_t N, int64_t K, int64_t G,
                                       void *stream)
{
    const int f = format_bits(a_fmt, b_fmt);
    if (f < 0)
        return DG_ERR_UNSUPPORTED;
    return (dg_status)contiguous_impl(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, b_stride_g, sB, sb_stride_g,
                           sb_stride_nb, sb_stride_kb, expert_ids, nullptr, D, ldd, M_total, M_total, N, K, G,
                           stream, f);
}

dg_status dg_fp8_gemm_nt_fmt(const void *A, int a_fmt, int64_t lda, const float *sA, int64_t sa_stride_m,
                       int64_t sa_stride_kb, const void *B, int b_fmt, int64_t ldb, const float *sB,
                       int64_t sb_stride_nb, int64_t sb_stride_kb, void *D, int64_t ldd, int64_t M, int64_t N,
                       int64_t K, void *stream)
{
    if ((a_fmt != DG_FP8_E4M3 && a_fmt != DG_FP8_E5M2) || (b_fmt != DG_FP8_E4M3 && b_fmt != DG_FP8_E5M2))
        return DG_ERR_UNSUPPORTED;
    if (a_fmt == DG_FP8_E4M3 && b_fmt == DG_FP8_E4M3)
        return (dg_status)dg_fp8_gemm_nt(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, sB, sb_stride_nb, sb_stride_kb, D,
                              ldd, M, N, K, stream);
    dgk::Params p;
    DeviceInfo dev;
    int st = dense_setup(A, lda, sA, sa_stride_m, sa_stride_kb, B, ldb, sB, sb_stride_nb, sb_stride_kb, D, ldd,
                         M, N, K, p, dev);
    if (st != DG_OK)
        return (dg_status)(st == kEmptyProblem ? DG_OK : st);
    if (!offsets_fit(lda, ldb, sa_stride_m))
        return DG_ERR_UNSUPPORTED;
    Ctx c;  // no workspace: never split over K
    c.cus = dev.cus;
    c.stream = (hipStream_t)stream;
    // Formats other than e4m3 x e4m3 run on the tile kernel at every M.
    switch ((a_fmt == DG_FP8_E5M2 ? 1 : 0) | (b_fmt == DG_FP8_E5M2 ? 2 : 0)) {
    case 1: return (dg_status)launch_dense_auto<1>(p, c);
    case 2: return (dg_status)launch_dense_auto<2>(p, c);
    default: return (dg_status)launch_dense_auto<3>(p, c);
    }
}

dg_status dg_fp8_quantize_1x128(const void *X, int x_dtype, int64_t ldx, void *Q, int64_t ldq, float *S,
                          int64_t s_stride_m, int64_t s_stride_kb, int64_t M, int64_t K, void *stream)
{
    return (dg_status)(quantize_impl(X, x_dtype, ldx, M, nullptr, Q, ldq, S, s_stride_m, s_stride_kb, M, K, stream));
}

dg_status dg_fp8_quantize_1x128_gather(const void *X, int x_dtype, int64_t ldx, int64_t x_rows,
                                 const int32_t *src_rows, void *Q, int64_t ldq, float *S, int64_t s_stride_m,
                                 int64_t s_stride_kb, int64_t M, int64_t K, void *stream)
{
    if (x_rows < 0)
        return DG_ERR_BAD_SHAPE;
    if (M > 0 && !src_rows)
        return DG_ERR_NULL_POINTER;
    if (src_rows && !aligned(src_rows, 4))
        return DG_ERR_MISALIGNED;
    return (dg_status)(quantize_impl(X, x_dtype, ldx, x_rows, src_rows, Q, ldq, S, s_stride_m, s_stride_kb, M, K, stream));
}

int64_t dg_moe_contiguous_max_rows(int64_t T, int64_t G)
{
    if (T < 0 || G < 0)
        return -1;
    return 128 * ((T + 127) / 128 + std::min(G, T));
}

dg_status dg_moe_route_contiguous(const int32_t *expert_of_token, int64_t T, int64_t G, int32_t *row_of_token,
                            int32_t *expert_ids, int32_t *token_of_row, int32_t *layout, int64_t M_cap,
                            void *stream)
{
    if (T < 0 || G <= 0 || M_cap < 0 || M_cap % 128 != 0)
        return DG_ERR_BAD_SHAPE;
    if (G > dgm::kMaxExperts || T > kInt32Max || M_cap > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (M_cap < dg_moe_contiguous_max_rows(T, G))
        return DG_ERR_BAD_SHAPE;
    if (!layout || (T > 0 && (!expert_of_token || !row_of_token)) || (M_cap > 0 && (!expert_ids || !token_of_row)))
        return DG_ERR_NULL_POINTER;
    if (!aligned(expert_of_token, 4) || !aligned(row_of_token, 4) || !aligned(expert_ids, 4) ||
        !aligned(token_of_row, 4) || !aligned(layout, 4))
        return DG_ERR_MISALIGNED;
    const Extent outs[4] = {extent(row_of_token, 4, T - 1), extent(expert_ids, 4, M_cap - 1),
                            extent(token_of_row, 4, M_cap - 1), extent(layout, 4, G)};
    const int64_t sizes[4] = {T, M_cap, M_cap, G + 1};
    const Extent ein = extent(expert_of_token, 4, T - 1);
    for (int i = 0; i < 4; ++i) {
        if (!sizes[i])
            continue;
        if (T > 0 && overlaps(outs[i], ein))
            return DG_ERR_ALIASING;
        for (int j = i + 1; j < 4; ++j)
            if (sizes[j] && overlaps(outs[i], outs[j]))
                return DG_ERR_ALIASING;
    }
    DeviceInfo dev;
    int st = current_device(dev);
    if (st != DG_OK)
        return (dg_status)(st);
    dgm::RouteParams p = {};
    p.expert_of_token = expert_of_token;
    p.T = (int)T; p.G = (int)G; p.M_cap = (int)M_cap;
    p.row_of_token = row_of_token; p.expert_ids = expert_ids; p.token_of_row = token_of_row; p.layout = layout;
    hipLaunchKernelGGL(dgm::route_contiguous_kernel, dim3(1), dim3(dgm::kRouteThreads), 0, (hipStream_t)stream, p);
    const hipError_t e = hipGetLastError();
    return (dg_status)(e == hipSuccess ? DG_OK : fail_hip(e));
}

dg_status dg_moe_unpermute(const void *D, int64_t ldd, int64_t d_rows, const int32_t *row_of_token, int64_t T,
                     int64_t N, void *out, int64_t ldo, void *stream)
{
    if (T < 0 || N < 0 || d_rows < 0 || N % 8 != 0)
        return DG_ERR_BAD_SHAPE;
    if (T > kInt32Max || N > kInt32Max || d_rows > kInt32Max)
        return DG_ERR_UNSUPPORTED;
    if (T == 0 || N == 0)
        return DG_OK;
    if ((d_rows > 0 && !D) || !row_of_token || !out)
        return DG_ERR_NULL_POINTER;
    if (ldo < N || (d_rows > 0 && ldd < N))
        return DG_ERR_BAD_STRIDE;
    if (!aligned(D, 16) || !aligned(out, 16) || ldd % 8 || ldo % 8 || !aligned(row_of_token, 4))
        return DG_ERR_MISALIGNED;
    const Extent eo = extent(out, 2, (T - 1) * ldo + N - 1);
    if ((d_rows > 0 && overlaps(eo, extent(D, 2, (d_rows - 1) * ldd + N - 1))) ||
        overlaps(eo, extent(row_of_token, 4, T - 1)))
        return DG_ERR_ALIASING;
    DeviceInfo dev;
    int st = current_device(dev);
    if (st != DG_OK)
        return (dg_status)(st);
    dgm::UnpermuteParams p = {};
    p.D = (const uint16_t *)D; p.ldd = ldd; p.d_rows = (int)d_rows;
    p.row_of_token = row_of_token; p.T = (int)T; p.N = (int)N;
    p.out = (uint16_t *)out; p.ldo = ldo;
    const unsigned groups = (unsigned)((T + dgm::kUnpermuteWaves - 1) / dgm::kUnpermuteWaves);
    hipLaunchKernelGGL(dgm::unpermute_kernel, dim3(groups), dim3(64 * dgm::kUnpermuteWaves), 0,
                       (hipStream_t)stream, p);
    const hipError_t e = hipGetLastError();
    return (dg_status)(e == hipSuccess ? DG_OK : fail_hip(e));
}

}  // extern "C"
