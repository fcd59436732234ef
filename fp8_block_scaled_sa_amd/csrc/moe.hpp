// moe.hpp -- gfx950 kernels around the contiguous grouped GEMM: routing of
// tokens into the padded contiguous layout, and the gather of the GEMM's rows
// back into token order.
//
// Layout (regrouping tokens by expert: lpnh.cn article, §5.3; padding to
// aligned shapes: bhfrc.com article, §4.2; group id and token offsets passed
// to the GEMM: rkmt.cn walkthrough, §5.3): experts one after another in
// ascending id order, each expert's tokens in ascending token order, each
// segment padded to a multiple of 128 rows. Padding rows, and every row from
// the last segment's end to the capacity, carry expert id -1 and token -1. A
// token whose expert id is outside [0, G) is dropped (row -1).
//
// Routing is a stable counting sort in one workgroup of 16 waves. Each wave
// owns a contiguous range of tokens, loads up to 16 chunks of 64 at once and
// takes the chunks one after another. Inside a chunk, every lane finds the
// lanes that hold its own expert with one ballot per bit of the expert id (a
// multisplit by key bits: Ashkiani et al., "GPU Multisplit", PPoPP 2016), so
// a chunk costs ceil(log2 G) ballots whatever its mix of experts; a lane's
// rank among them is the count of such lanes below it. Pass 1 counts per
// (wave, expert) in LDS; an exclusive prefix over the waves and a scan over
// the padded segment sizes give every token's row in pass 2. No atomics: the
// result is the same on every run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgm {

constexpr int kRouteWaves = 16;
constexpr int kRouteThreads = 64 * kRouteWaves;
constexpr int kMaxExperts = 1024;

struct RouteParams {
    const int32_t *expert_of_token;  // [T]
    int T, G, M_cap;
    int32_t *row_of_token;           // [T]
    int32_t *expert_ids;             // [M_cap]
    int32_t *token_of_row;           // [M_cap]
    int32_t *layout;                 // [G + 1]: first row of each expert, then the rows used
};

// Chunks of 64 tokens a wave loads at once. The loads are unconditional (the
// index is clamped into [0, T), and tokens outside the wave's range are
// masked afterwards), so all of them are in flight before the first wait; a
// load per chunk inside the loop cost one memory latency per chunk.
constexpr int kChunks = 16;

__device__ __forceinline__ void load_experts(const RouteParams &p, int base, int t_end, int lane, int (&e)[kChunks])
{
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int t = base + 64 * c + lane;
        const int v = p.expert_of_token[min(t, p.T - 1)];
        e[c] = (t < t_end && v >= 0 && v < p.G) ? v : -1;
    }
}

// Lanes of the wave whose expert equals this lane's (e >= 0; only lanes with
// e >= 0 take part): ANDs the ballot of each id bit, or of its complement,
// over the `bits` bits that ids in [0, G) use. Uniform over the wave.
__device__ __forceinline__ uint64_t same_expert(int e, int bits)
{
    uint64_t same = __ballot(e >= 0);
    for (int b = 0; b < bits; ++b) {
        const bool set = (e >> b) & 1;
        const uint64_t m = __ballot(set);
        same &= set ? m : ~m;
    }
    return same;
}

__global__ __launch_bounds__(kRouteThreads) void route_contiguous_kernel(RouteParams p)
{
    __shared__ int cnt[kRouteWaves][kMaxExperts];  // per-wave counts, then per-wave running offsets
    __shared__ int seg[kMaxExperts + 1];           // first row of each expert's segment
    __shared__ int tot[kMaxExperts];               // tokens per expert
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    for (int e = lane; e < p.G; e += 64)
        cnt[w][e] = 0;
    __syncthreads();

    const int chunk = (p.T + kRouteWaves - 1) / kRouteWaves;
    const int t0 = min(p.T, w * chunk), t1 = min(p.T, t0 + chunk);
    const int bits = p.G > 1 ? 32 - __clz(p.G - 1) : 0;
    const uint64_t below = (1ull << lane) - 1;  // lanes under this one
    for (int sc = t0; sc < t1; sc += 64 * kChunks) {
        int ex[kChunks];
        load_experts(p, sc, t1, lane, ex);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (sc + 64 * c >= t1)
                break;
            const int e = ex[c];
            const uint64_t same = same_expert(e, bits);
            // the lowest lane of each expert adds the chunk's count (distinct
            // addresses within the chunk; this wave's LDS operations stay in order)
            if (e >= 0 && (same & below) == 0)
                cnt[w][e] += __popcll(same);
        }
    }
    __syncthreads();

    const int e = threadIdx.x;  // G <= kMaxExperts == kRouteThreads: one expert per thread
    if (e < p.G) {
        int run = 0;
        for (int v = 0; v < kRouteWaves; ++v) {
            const int c = cnt[v][e];
            cnt[v][e] = run;
            run += c;
        }
        tot[e] = run;
        seg[e + 1] = (run + 127) / 128 * 128;
    }
    if (threadIdx.x == 0)
        seg[0] = 0;
    __syncthreads();
    for (int off = 1; off < p.G; off <<= 1) {  // inclusive scan of seg[1..G]
        const int i = threadIdx.x + 1;
        const int v = (i <= p.G && i - off >= 1) ? seg[i - off] : 0;
        __syncthreads();
        if (i <= p.G)
            seg[i] += v;
        __syncthreads();
    }
    if (threadIdx.x < p.G)
        p.layout[threadIdx.x] = seg[threadIdx.x];
    if (threadIdx.x == 0)
        p.layout[p.G] = seg[p.G];

    // Rows that hold no token: the tail of each expert's segment (wave w takes
    // experts w, w + 16, ...) and everything past the last segment.
    for (int g = w; g < p.G; g += kRouteWaves)
        for (int r = seg[g] + tot[g] + lane; r < seg[g + 1]; r += 64) {
            p.expert_ids[r] = -1;
            p.token_of_row[r] = -1;
        }
    for (int r = seg[p.G] + threadIdx.x; r < p.M_cap; r += kRouteThreads) {
        p.expert_ids[r] = -1;
        p.token_of_row[r] = -1;
    }

    for (int sc = t0; sc < t1; sc += 64 * kChunks) {
        int ex[kChunks];
        load_experts(p, sc, t1, lane, ex);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (sc + 64 * c >= t1)
                break;
            const int t = sc + 64 * c + lane;
            const int e = ex[c];
            const uint64_t same = same_expert(e, bits);
            int row = -1;
            if (e >= 0) {
                // cnt holds this wave's running offset within expert e's
                // segment; the chunk's lanes of e take the next rows in lane
                // order, and the lowest of them moves the offset on
                const int off = cnt[w][e];
                row = seg[e] + off + __popcll(same & below);
                if ((same & below) == 0)
                    cnt[w][e] = off + __popcll(same);
            }
            if (t < t1) {
                p.row_of_token[t] = row;
                if (row >= 0) {
                    p.token_of_row[row] = t;
                    p.expert_ids[row] = e;
                }
            }
        }
    }
}

struct UnpermuteParams {
    const uint16_t *D;   // bf16 [d_rows, N], row stride ldd
    int64_t ldd;
    int d_rows;
    const int32_t *row_of_token;
    int T, N;
    uint16_t *out;       // bf16 [T, N], row stride ldo
    int64_t ldo;
};

typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));
constexpr int kUnpermuteWaves = 4;

// out[t, :] = D[row_of_token[t], :]; a row index outside [0, d_rows) gives
// zeros. One wave per token, 16 bytes per lane and step.
__global__ __launch_bounds__(64 * kUnpermuteWaves) void unpermute_kernel(UnpermuteParams p)
{
    const int t = blockIdx.x * kUnpermuteWaves + (threadIdx.x >> 6);
    if (t >= p.T)
        return;
    const int lane = threadIdx.x & 63;
    const int r = p.row_of_token[t];
    uint16_t *dst = p.out + (int64_t)t * p.ldo;
    if (r < 0 || r >= p.d_rows) {
        for (int n = 8 * lane; n < p.N; n += 512)
            *(u32x4m *)(dst + n) = u32x4m{0, 0, 0, 0};
        return;
    }
    const uint16_t *src = p.D + (int64_t)r * p.ldd;
#pragma unroll 4
    for (int n = 8 * lane; n < p.N; n += 512)
        *(u32x4m *)(dst + n) = *(const u32x4m *)(src + n);
}

// Segment offsets for the contiguous grouped GEMM derived from its expert ids
// alone, so that a call given only the ids can tile along the segments. A
// 128-row block's expert is the largest id in [0, G) among its rows (-1 for a
// block of padding only), as the GEMM itself defines it. When the non-padding
// block experts never decrease, layout[e] is the first row of the first block
// whose expert is >= e and layout[G] the end of the last non-padding block:
// each segment then holds its expert's blocks and the padding blocks after
// them, and the GEMM writes exactly the rows it writes on the uniform grid.
// Otherwise every offset is 0 (no segment tiles) and *use_grid = 1, which
// gates the uniform-grid launch that follows; else *use_grid = 0.
// One workgroup of 16 waves; nb = M / 128 <= kDeriveMaxBlocks.
constexpr int kDeriveMaxBlocks = 4096;

struct DeriveParams {
    const int32_t *ids;  // [M]
    int M, G;
    int32_t *layout;     // [G + 1]
    int32_t *use_grid;   // [1]
};

__global__ __launch_bounds__(kRouteThreads) void derive_layout_kernel(DeriveParams p)
{
    __shared__ int bexp[kDeriveMaxBlocks];  // block experts, then their prefix maximum
    __shared__ int s_ok, s_end;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nb = p.M >> 7;
    // Each thread takes whole 128-row blocks (block b: thread b, b + 1024, ...)
    // and reads its 128 ids with all loads in flight together (32 16-byte
    // loads when the ids are 16-byte aligned, else four rounds of 32 4-byte
    // loads): the block's expert is a maximum in registers, with no
    // cross-lane steps.
    const bool aligned16 = ((uintptr_t)p.ids & 15) == 0;
    for (int b = threadIdx.x; b < nb; b += kRouteThreads) {
        const int32_t *blk = p.ids + 128 * b;
        int e = -1;
        auto take = [&](int x) { e = max(e, (x >= 0 && x < p.G) ? x : -1); };
        if (aligned16) {
            int4 v[32];
#pragma unroll
            for (int j = 0; j < 32; ++j)
                v[j] = reinterpret_cast<const int4 *>(blk)[j];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                take(v[j].x), take(v[j].y), take(v[j].z), take(v[j].w);
            }
        } else {
            for (int r = 0; r < 128; r += 32) {
                int v[32];
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    v[j] = blk[r + j];
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    take(v[j]);
            }
        }
        bexp[b] = e;
    }
    __syncthreads();
    if (w == 0) {
        // lane l takes blocks [l * chunk, (l + 1) * chunk)
        const int chunk = (nb + 63) / 64;
        const int b0 = min(nb, lane * chunk), b1 = min(nb, b0 + chunk);
        int run = -1, first = -1, last = -1;
        bool ok = true;
        for (int b = b0; b < b1; ++b) {
            const int e = bexp[b];
            if (e >= 0) {
                ok = ok && e >= run;
                if (first < 0)
                    first = e;
                last = b;
            }
            run = max(run, e);
        }
        // maximum over the lanes below (exclusive prefix maximum)
        int below = run;
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(below, o);
            if (lane >= o)
                below = max(below, v);
        }
        below = __shfl_up(below, 1);
        if (lane == 0)
            below = -1;
        ok = ok && (first < 0 || first >= below);
        int end = last;
        for (int o = 32; o > 0; o >>= 1)
            end = max(end, __shfl_xor(end, o));
        const bool all_ok = __ballot(!ok) == 0;
        // prefix maximum in place
        int m = below;
        for (int b = b0; b < b1; ++b) {
            m = max(m, bexp[b]);
            bexp[b] = m;
        }
        if (lane == 0) {
            s_ok = all_ok ? 1 : 0;
            s_end = end + 1;  // blocks up to the last non-padding one
        }
    }
    __syncthreads();
    const bool ok = s_ok != 0;
    for (int e = threadIdx.x; e <= p.G; e += kRouteThreads) {
        int v = 0;
        if (ok) {
            // first block whose prefix maximum is >= e (the prefix maximum
            // never decreases), capped at the end of the last non-padding block
            int lo = 0, hi = nb;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (bexp[mid] >= e)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            v = 128 * min(e == p.G ? s_end : lo, s_end);
        }
        p.layout[e] = v;
    }
    if (threadIdx.x == 0)
        *p.use_grid = ok ? 0 : 1;
}

}  // namespace dgm
