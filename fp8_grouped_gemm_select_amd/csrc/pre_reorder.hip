// Stage 2: permutation of (token, slot) pairs into expert-contiguous rows and
// dynamic FP8 quantisation of the token rows into those rows.
//
// Follows "Support token-level quantization for EP MoE" (sglang PR #6782),
// change summary of pre_reorder_triton_kernel and EPMoELayer: per-token maxima
// give per-token scales, and the scales travel with the rows through src2dst.
// Here the scale reorder is fused into the scatter.
//
// A deterministic stable counting sort over the (token, slot) pairs
// f = t * topk + slot, in chunks of 64 consecutive pairs (one wave each):
//   count    a pair's stable rank among the chunk's earlier pairs of the same
//            local expert (one ballot per distinct expert, kept in src2dst) and the
//            chunk's count per expert, stored expert-major [E_l][nchunks];
//   scan     one block per local expert: an exclusive scan of its chunk
//            counts (entry (e, c) = expert e's pairs in chunks before c) and its
//            total; block 0 also reduces the per-tensor amax partials;
//   scatter  one wave per token: its row loads are issued as soon as its ids
//            are known; the experts' first rows (seg_indptr) come from a wave
//            prefix sum of the totals, block 0 writes them out; final rows,
//            dst2src, and the quantised row written to each of the token's
//            local rows; the grid clears dst2src[M..m_cap).
// Batches of up to 4096 pairs count and scan in one block; up to 2048 pairs,
// every scatter block counts and scans for itself and the stage is one launch.
#include "common.h"

#include <mutex>

namespace moe {
namespace {

constexpr int kChunkPairs = 64;
constexpr int kRegIters = 7;   // rows up to 7168 wide stay in registers
constexpr int kAmaxBlocks = 1024;

struct PreWs {
    int32_t* counts;   // [num_local][nchunks]
    int32_t* offs;     // [num_local][nchunks], exclusive scan of counts within each expert
    int32_t* tot;      // [num_local], pairs per local expert
    float* amax_part;  // [kAmaxBlocks]
    float* tscale;     // [2]: per-tensor scale, inverse
};

__host__ __device__ inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

inline int64_t n_chunks(int64_t T, int32_t topk) { return ceil_div(T * (int64_t)topk, kChunkPairs); }

// counts / offs entries (padded to a multiple of 32, plus 32)
inline int64_t n_entries(int64_t T, int32_t topk, int32_t num_local) {
    return (n_chunks(T, topk) * num_local + 31) / 32 * 32 + 32;
}

inline size_t pre_ws_bytes(int64_t T, int32_t topk, int32_t num_local) {
    const int64_t ne = n_entries(T, topk, num_local);
    size_t b = 0;
    b += align256(sizeof(int32_t) * (size_t)ne);
    b += align256(sizeof(int32_t) * (size_t)ne);
    b += align256(sizeof(int32_t) * (size_t)(num_local > 0 ? num_local : 1));
    b += align256(sizeof(float) * kAmaxBlocks);
    b += align256(sizeof(float) * 2);
    return b;
}

inline PreWs pre_ws_carve(void* ws, int64_t T, int32_t topk, int32_t num_local) {
    const int64_t ne = n_entries(T, topk, num_local);
    char* p = (char*)ws;
    PreWs w;
    w.counts = (int32_t*)p;
    p += align256(sizeof(int32_t) * (size_t)ne);
    w.offs = (int32_t*)p;
    p += align256(sizeof(int32_t) * (size_t)ne);
    w.tot = (int32_t*)p;
    p += align256(sizeof(int32_t) * (size_t)(num_local > 0 ? num_local : 1));
    w.amax_part = (float*)p;
    p += align256(sizeof(float) * kAmaxBlocks);
    w.tscale = (float*)p;
    return w;
}

// Local expert index of a global id: the routed local range [expert_start,
// expert_start + num_routed) maps to 0.., the shared ids [shared_base,
// shared_base + n_shared) to num_routed.., anything else is not local (-1).
struct LocalMap {
    int expert_start, num_routed, shared_base, n_shared;
};
__device__ __forceinline__ int local_of(int id, const LocalMap& m) {
    const int r = id - m.expert_start;
    if (r >= 0 && r < m.num_routed) return r;
    const int q = id - m.shared_base;
    if (q >= 0 && q < m.n_shared) return m.num_routed + q;
    return -1;
}

// A local pair's stable rank among the lower lanes of its wave that hold the same
// local expert (below) and how many lanes hold it (all); one ballot round per
// distinct local expert present (a chunk of 64 pairs holds a few), lanes that
// are not local (e < 0) get 0.
__device__ __forceinline__ void chunk_rank(int e, int lane, int& below, int& all) {
    uint64_t rem = __ballot(e >= 0);
    while (rem) {
        const int x = __builtin_amdgcn_readlane(e, __builtin_ctzll(rem));
        const uint64_t m = __ballot(e == x);
        if (e == x) {
            below = __popcll(m & lanemask_lt(lane));
            all = __popcll(m);
        }
        rem &= ~m;
    }
}

// ---- count: chunk-local stable ranks -----------------------------------------
// One 64-thread block per chunk of 64 pairs; lane l holds pair 64 c + l. Its
// rank is the number of lower lanes holding the same local expert
// (chunk_rank); the lane holding an expert's last occurrence in the chunk
// records the count. cnt[] (dynamic LDS, num_local
// ints) gives every (expert, chunk) entry exactly one writer.
__global__ __launch_bounds__(64) void pr_count_kernel(const int32_t* __restrict__ ids, int64_t F,
                                                      LocalMap map, int num_local, int64_t nch,
                                                      int32_t* __restrict__ src2dst,
                                                      int32_t* __restrict__ counts) {
    extern __shared__ int32_t cnt[];
    const int lane = threadIdx.x;
    const int64_t chunk = blockIdx.x;
    for (int e = lane; e < num_local; e += 64) cnt[e] = 0;
    const int64_t f = chunk * kChunkPairs + lane;
    const int e = f < F ? local_of(ids[f], map) : -1;
    const bool local = e >= 0;
    int below = 0, all = 0;
    chunk_rank(e, lane, below, all);
    __syncthreads();  // cnt[] cleared
    if (local && below == all - 1) cnt[e] = all;
    if (f < F) src2dst[f] = local ? below : -1;
    __syncthreads();
    for (int x = lane; x < num_local; x += 64) counts[(int64_t)x * nch + chunk] = cnt[x];
}

// ---- per-tensor amax partials over all of x ---------------------------------------
__global__ __launch_bounds__(256) void pr_amax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                      float* __restrict__ part) {
    __shared__ float red[4];
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
        const uint4 a = x[i * 2], b = x[i * 2 + 1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---- scan: per-expert exclusive scans of the chunk counts ------------------------------
// Block e scans row e of the expert-major counts in passes of 256 x 4 entries
// and stores the row total; the experts' first rows are prefix sums of those
// totals, formed where they are used (expert_base below). Block 0 also reduces
// the per-tensor amax partials into the scale and its inverse.
__global__ __launch_bounds__(256) void pr_scan_kernel(const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offs, int64_t nch,
                                                      int num_local, int32_t* __restrict__ tot,
                                                      const float* __restrict__ amax_part,
                                                      int n_part, int per_tensor,
                                                      float* __restrict__ a_scale,
                                                      float* __restrict__ tscale) {
    __shared__ int scratch[17];
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    if (e < num_local) {
        const int32_t* row = counts + (int64_t)e * nch;
        int32_t* orow = offs + (int64_t)e * nch;
        int carry = 0;
        for (int64_t c0 = 0; c0 < nch; c0 += 256 * 4) {
            int v[4];
            int mine = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t c = c0 + tid * 4 + q;
                v[q] = c < nch ? row[c] : 0;
                mine += v[q];
            }
            int total = 0;
            int run = carry + block_exclusive_scan(mine, scratch, &total);
            carry += total;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t c = c0 + tid * 4 + q;
                if (c < nch) orow[c] = run;
                run += v[q];
            }
        }
        if (tid == 0) tot[e] = carry;
    }
    if (e == 0 && per_tensor) {
        float m = 0.0f;
        for (int i = tid; i < n_part; i += 256) m = fmaxf(m, amax_part[i]);
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            float sc, inv;
            dyn_scale(a, sc, inv);
            a_scale[0] = sc;
            tscale[0] = sc;
            tscale[1] = inv;
        }
    }
}

// ---- count + scan in one block (few pairs) ---------------------------------------
// The results of pr_count_kernel followed by pr_scan_kernel, in one launch, when
// there are at most kFusedChunks chunks and the expert x chunk count table fits
// in LDS (a decode batch): wave w ranks chunks w, w + 16, ... exactly as the
// count kernel does, the table stays in LDS, and thread e then scans expert e's
// row of it. The per-tensor amax partials (written by an earlier launch) are
// reduced by the whole block.
constexpr int kFusedChunks = 64;
constexpr int kFusedTable = 8192;

__global__ __launch_bounds__(1024) void pr_count_scan_kernel(const int32_t* __restrict__ ids, int64_t F,
                                                             LocalMap map, int num_local, int nch,
                                                             int32_t* __restrict__ src2dst,
                                                             int32_t* __restrict__ offs,
                                                             int32_t* __restrict__ tot,
                                                             const float* __restrict__ amax_part,
                                                             int n_part, int per_tensor,
                                                             float* __restrict__ a_scale,
                                                             float* __restrict__ tscale) {
    __shared__ int32_t cnt[kFusedTable];
    __shared__ float red[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < num_local * nch; i += 1024) cnt[i] = 0;
    __syncthreads();
    for (int c = w; c < nch; c += 16) {
        const int64_t f = (int64_t)c * kChunkPairs + lane;
        const int e = f < F ? local_of(ids[f], map) : -1;
        int below = 0, all = 0;
        chunk_rank(e, lane, below, all);
        if (e >= 0 && below == all - 1) cnt[e * nch + c] = all;
        if (f < F) src2dst[f] = e >= 0 ? below : -1;
    }
    __syncthreads();
    for (int e = tid; e < num_local; e += 1024) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            offs[(int64_t)e * nch + c] = run;
            run += cnt[e * nch + c];
        }
        tot[e] = run;
    }
    if (per_tensor) {
        float m = 0.0f;
        for (int i = tid; i < n_part; i += 1024) m = fmaxf(m, amax_part[i]);
        m = wave_max(m);
        if (lane == 0) red[w] = m;
        __syncthreads();
        if (tid == 0) {
            float a = red[0];
            for (int q = 1; q < 16; ++q) a = fmaxf(a, red[q]);
            float sc, inv;
            dyn_scale(a, sc, inv);
            a_scale[0] = sc;
            tscale[0] = sc;
            tscale[1] = inv;
        }
    }
}

// First row of local expert e (exclusive prefix sum of the totals, for each
// lane's own e; lanes with e < 0 get 0) and, in `total`, M = all local pairs.
// Wave-uniform loop over the totals in groups of 64.
__device__ __forceinline__ int expert_base(const int32_t* __restrict__ tot, int num_local, int e, int lane,
                                           int& total) {
    int base = 0, carry = 0;
    for (int q0 = 0; q0 < num_local; q0 += 64) {
        const int v = q0 + lane < num_local ? tot[q0 + lane] : 0;
        const int incl = wave_inclusive_scan(v, lane);
        const int excl = incl - v + carry;
        const int src = e - q0;
        const bool here = src >= 0 && src < 64;
        const int b = __shfl(excl, here ? src : 0, MOE_WAVE);
        if (here) base = b;
        carry += __shfl(incl, 63, MOE_WAVE);
    }
    total = carry;
    return base;
}

// ---- scatter + quantise ------------------------------------------------------------------
__device__ __forceinline__ float amax16(const uint4& a, const uint4& b) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
    return m;
}

__device__ __forceinline__ uint4 quant16(const uint4& a, const uint4& b, float inv) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = quant4(bf16_lo(w[2 * q]), bf16_hi(w[2 * q]), bf16_lo(w[2 * q + 1]), bf16_hi(w[2 * q + 1]), inv);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One token (one wave): lanes < topk hold its pairs. rank[f] is pair f's stable
// rank among its chunk's earlier pairs of the same expert (src2dst itself, as
// the count pass left it, or the small-batch kernel's LDS copy).
template <int MODE>
__device__ __forceinline__ void scatter_token(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, int64_t t, int H, int topk,
    const LocalMap& map, int num_local, int64_t nch, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ tot, const int32_t* rank,
    int32_t* __restrict__ src2dst, int32_t* __restrict__ dst2src, uint8_t* __restrict__ a_q,
    float* __restrict__ a_scale, const float* __restrict__ tscale, int64_t m_cap, int lane) {
    const int64_t f = t * topk + lane;
    int e = -1;
    if (lane < topk) e = local_of(ids[f], map);
    if (__ballot(e >= 0) == 0) {
        if (lane < topk) src2dst[f] = -1;
        return;
    }

    const int G = (H + MOE_QB - 1) / MOE_QB;
    const int nit = (H + 1023) / 1024;  // iterations of 1024 columns (16 per lane)
    const uint4* xr = x + (t * H) / 8;   // 8 bf16 per uint4
    // Columns past H read column 0 (a valid address) and are masked to zero with
    // an AND, not a branch: a branch around the loads makes the compiler wait
    // for each load before issuing the next.
    auto load16 = [&](int it, uint4& a, uint4& b) {
        const int c = it * 1024 + lane * 16;
        const int cc = c < H ? c : 0;
        const uint32_t m = c < H ? 0xFFFFFFFFu : 0u;
        const uint4 a0 = xr[cc / 8], b0 = xr[cc / 8 + 1];
        a = make_uint4(a0.x & m, a0.y & m, a0.z & m, a0.w & m);
        b = make_uint4(b0.x & m, b0.y & m, b0.z & m, b0.w & m);
    };

    // the row's first kRegIters iterations go to registers now (every mode), in
    // flight while the destination rows are looked up
    uint4 buf[kRegIters][2];
#pragma unroll
    for (int it = 0; it < kRegIters; ++it) load16(it, buf[it][0], buf[it][1]);

    int m_all = 0;
    const int base = expert_base(tot, num_local, e, lane, m_all);
    int dst = -1;
    if (e >= 0) {
        dst = base + offs[(int64_t)e * nch + f / kChunkPairs] + rank[f];
        // rows past m_cap exist only if a token repeats an expert; drop them
        if (dst >= m_cap) dst = -1;
        else dst2src[dst] = (int32_t)f;
    }
    if (lane < topk) src2dst[f] = dst;
    const uint64_t local_mask = __ballot(dst >= 0);
    if (local_mask == 0) return;

    auto store_rows = [&](int it, const uint4& codes) {
        const int c = it * 1024 + lane * 16;
        for (int j = 0; j < topk; ++j) {
            if ((local_mask >> j) & 1ull) {
                const int r = __builtin_amdgcn_readlane(dst, j);
                if (c < H) *(uint4*)(a_q + (int64_t)r * H + c) = codes;
            }
        }
    };

    if (MODE == MOE_ACT_PER_GROUP) {
#pragma unroll
        for (int it = 0; it < kRegIters; ++it) {
            if (it >= nit) break;
            const uint4 a = buf[it][0], b = buf[it][1];
            const float gm = group8_max(amax16(a, b));
            float s, inv;
            dyn_scale(gm, s, inv);
            store_rows(it, quant16(a, b, inv));
            const int g = it * 8 + (lane >> 3);
            for (int j = 0; j < topk; ++j) {
                if ((local_mask >> j) & 1ull) {
                    const int r = __builtin_amdgcn_readlane(dst, j);
                    if ((lane & 7) == 0 && g < G) a_scale[(int64_t)r * G + g] = s;
                }
            }
        }
        for (int it = kRegIters; it < nit; ++it) {
            uint4 a, b;
            load16(it, a, b);
            const float gm = group8_max(amax16(a, b));
            float s, inv;
            dyn_scale(gm, s, inv);
            store_rows(it, quant16(a, b, inv));
            const int g = it * 8 + (lane >> 3);
            for (int j = 0; j < topk; ++j) {
                if ((local_mask >> j) & 1ull) {
                    const int r = __builtin_amdgcn_readlane(dst, j);
                    if ((lane & 7) == 0 && g < G) a_scale[(int64_t)r * G + g] = s;
                }
            }
        }
        return;
    }

    float s, inv;
    if (MODE == MOE_ACT_PER_TENSOR) {
        s = tscale[0];
        inv = tscale[1];
#pragma unroll
        for (int it = 0; it < kRegIters; ++it)
            if (it < nit) store_rows(it, quant16(buf[it][0], buf[it][1], inv));
        for (int it = kRegIters; it < nit; ++it) {
            uint4 a, b;
            load16(it, a, b);
            store_rows(it, quant16(a, b, inv));
        }
        return;
    }

    // per token: amax over the row, then the codes
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < kRegIters; ++it)
        if (it < nit) amax = fmaxf(amax, amax16(buf[it][0], buf[it][1]));
    for (int it = kRegIters; it < nit; ++it) {
        uint4 a, b;
        load16(it, a, b);
        amax = fmaxf(amax, amax16(a, b));
    }
    amax = wave_max(amax);
    dyn_scale(amax, s, inv);
#pragma unroll
    for (int it = 0; it < kRegIters; ++it)
        if (it < nit) store_rows(it, quant16(buf[it][0], buf[it][1], inv));
    for (int it = kRegIters; it < nit; ++it) {
        uint4 a, b;
        load16(it, a, b);
        store_rows(it, quant16(a, b, inv));
    }
    if (lane < topk && dst >= 0) a_scale[dst] = s;
}

template <int MODE>
// five waves per SIMD: the row buffer (7 x 32 bytes per lane) and the rest fit 96 VGPRs
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void pr_scatter_quant_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, int64_t T, int H, int topk,
    LocalMap map, int num_local, int64_t nch, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ tot, int32_t* __restrict__ seg, int32_t* __restrict__ src2dst,
    int32_t* __restrict__ dst2src,
    uint8_t* __restrict__ a_q, float* __restrict__ a_scale, const float* __restrict__ tscale,
    int64_t m_cap) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    int m_all = 0;
    expert_base(tot, num_local, -1, lane, m_all);  // M, for the tail below
    const int64_t M = m_all;
    if (blockIdx.x == 0 && wid == 0) {  // seg_indptr = [first rows..., M]
        int carry = 0;
        for (int q0 = 0; q0 < num_local; q0 += 64) {
            const int v = q0 + lane < num_local ? tot[q0 + lane] : 0;
            const int incl = wave_inclusive_scan(v, lane);
            if (q0 + lane < num_local) seg[q0 + lane] = incl - v + carry;
            carry += __shfl(incl, 63, MOE_WAVE);
        }
        if (lane == 0) seg[num_local] = carry;
    }
    if (t < T)
        scatter_token<MODE>(x, ids, t, H, topk, map, num_local, nch, offs, tot, src2dst, src2dst, dst2src,
                            a_q, a_scale, tscale, m_cap, lane);
    // rows M .. m_cap-1 of dst2src are -1 (grid-stride over the whole grid)
    for (int64_t r = M + (int64_t)blockIdx.x * 256 + threadIdx.x; r < m_cap; r += (int64_t)gridDim.x * 256)
        dst2src[r] = -1;
}

// ---- small batches: count, scan and scatter in one launch --------------------------
// When the pairs fill at most kSmallChunks chunks and the expert x chunk table
// fits LDS (a decode batch), every scatter block derives the permutation
// itself: its four waves rank the chunks exactly as the count pass does, thread
// e scans expert e's row of the table as the scan pass does, the per-tensor
// amax partials are reduced, and the block then scatters its four tokens as the
// scatter kernel does. The blocks repeat the same small computation instead of
// waiting for two earlier launches; the results are the same bits.
constexpr int kSmallChunks = 32;    // up to 2048 pairs
constexpr int kSmallTable = 4096;   // expert x chunk entries
constexpr int kSmallLocal = 1024;   // local experts

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void pr_scatter_small_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, int64_t T, int H, int topk,
    LocalMap map, int num_local, int nch, int32_t* __restrict__ seg, int32_t* __restrict__ src2dst,
    int32_t* __restrict__ dst2src, uint8_t* __restrict__ a_q, float* __restrict__ a_scale,
    const float* __restrict__ amax_part, int n_part, int64_t m_cap) {
    __shared__ int32_t s_offs[kSmallTable];                // counts, then their scan per expert
    __shared__ int32_t s_rank[kSmallChunks * kChunkPairs];  // within-chunk ranks
    __shared__ int32_t s_tot[kSmallLocal];
    __shared__ float s_ts[2], s_red[4];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int64_t F = T * topk;
    for (int i = tid; i < num_local * nch; i += 256) s_offs[i] = 0;
    __syncthreads();
    for (int c = wid; c < nch; c += 4) {
        const int f = c * kChunkPairs + lane;
        const int e = f < F ? local_of(ids[f], map) : -1;
        int below = 0, all = 0;
        chunk_rank(e, lane, below, all);
        if (e >= 0 && below == all - 1) s_offs[e * nch + c] = all;
        s_rank[f] = below;
    }
    __syncthreads();
    for (int e = tid; e < num_local; e += 256) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            const int v = s_offs[e * nch + c];
            s_offs[e * nch + c] = run;
            run += v;
        }
        s_tot[e] = run;
    }
    if (MODE == MOE_ACT_PER_TENSOR) {
        float m = 0.0f;
        for (int i = tid; i < n_part; i += 256) m = fmaxf(m, amax_part[i]);
        m = wave_max(m);
        if (lane == 0) s_red[wid] = m;
    }
    __syncthreads();
    if (MODE == MOE_ACT_PER_TENSOR && tid == 0) {
        const float a = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        float sc, inv;
        dyn_scale(a, sc, inv);
        s_ts[0] = sc;
        s_ts[1] = inv;
        if (blockIdx.x == 0) a_scale[0] = sc;
    }
    __syncthreads();

    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    int m_all = 0;
    expert_base(s_tot, num_local, -1, lane, m_all);  // M, for the tail below
    const int64_t M = m_all;
    if (blockIdx.x == 0 && wid == 0) {  // seg_indptr = [first rows..., M]
        int carry = 0;
        for (int q0 = 0; q0 < num_local; q0 += 64) {
            const int v = q0 + lane < num_local ? s_tot[q0 + lane] : 0;
            const int incl = wave_inclusive_scan(v, lane);
            if (q0 + lane < num_local) seg[q0 + lane] = incl - v + carry;
            carry += __shfl(incl, 63, MOE_WAVE);
        }
        if (lane == 0) seg[num_local] = carry;
    }
    if (t < T)
        scatter_token<MODE>(x, ids, t, H, topk, map, num_local, nch, s_offs, s_tot, s_rank, src2dst, dst2src,
                            a_q, a_scale, s_ts, m_cap, lane);
    for (int64_t r = M + (int64_t)blockIdx.x * 256 + threadIdx.x; r < m_cap; r += (int64_t)gridDim.x * 256)
        dst2src[r] = -1;
}

}  // namespace

size_t pre_reorder_ws_bytes(int64_t T, int32_t topk, int32_t num_local) {
    return pre_ws_bytes(T, topk, num_local);
}

}  // namespace moe

namespace moe {
// Shared by moe_pre_reorder_quant (no shared experts) and
// moe_pre_reorder_quant_shared; num_local = num_routed + n_shared local experts.
static int pre_reorder_impl(const void* x_bf16, const int32_t* topk_ids, int64_t T, int32_t H,
                            int32_t topk, int32_t expert_start, int32_t num_routed,
                            int32_t shared_base, int32_t n_shared, int32_t act_quant, int64_t m_cap,
                            uint8_t* a_q, float* a_scale, int64_t a_scale_numel, int32_t* src2dst,
                            int32_t* dst2src, int32_t* seg_indptr, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (num_routed < 0 || n_shared < 0 || n_shared > 64 || shared_base < 0) return MOE_ERR_INVALID_ARG;
    if (n_shared > 0 && (int64_t)shared_base < (int64_t)expert_start + num_routed &&
        (int64_t)shared_base + n_shared > expert_start)
        return MOE_ERR_INVALID_ARG;  // shared ids must not overlap the routed local range
    const int32_t num_local = num_routed + n_shared;
    const LocalMap map{expert_start, num_routed, shared_base, n_shared};
    if (T < 0 || H <= 0 || topk <= 0 || num_local < 0 || m_cap < 0) return MOE_ERR_INVALID_ARG;
    if (act_quant < MOE_ACT_PER_TENSOR || act_quant > MOE_ACT_PER_GROUP) return MOE_ERR_INVALID_ARG;
    if (H % 16 != 0 || topk > 32 || num_local > 8192) return MOE_ERR_UNSUPPORTED;
    if (T * (int64_t)topk > INT32_MAX || m_cap > INT32_MAX || m_cap * (int64_t)H > ((int64_t)1 << 40))
        return MOE_ERR_UNSUPPORTED;
    const int64_t need_rows = T * (int64_t)(topk < num_local ? topk : num_local);
    if (m_cap < need_rows) return MOE_ERR_SHAPE;
    const int64_t G = ceil_div(H, MOE_QB);
    const int64_t want_scales = act_quant == MOE_ACT_PER_TENSOR ? 1
                              : act_quant == MOE_ACT_PER_TOKEN  ? m_cap
                                                                : m_cap * G;
    if (a_scale_numel != want_scales) return MOE_ERR_SHAPE;
    if (!seg_indptr) return MOE_ERR_NULL;
    if (T > 0 && (!x_bf16 || !topk_ids || !src2dst)) return MOE_ERR_NULL;
    if (m_cap > 0 && (!a_q || !dst2src)) return MOE_ERR_NULL;
    if (want_scales > 0 && !a_scale && (m_cap > 0 || act_quant == MOE_ACT_PER_TENSOR)) return MOE_ERR_NULL;
    if ((x_bf16 && !aligned16(x_bf16)) || (a_q && !aligned16(a_q))) return MOE_ERR_INVALID_ARG;
    const size_t need_ws = pre_ws_bytes(T, topk, num_local);
    if (!workspace || workspace_bytes < need_ws) return MOE_ERR_WORKSPACE;

    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const int64_t nch = n_chunks(T, topk);
    PreWs ws = pre_ws_carve(workspace, T, topk, num_local);
    const int per_tensor = act_quant == MOE_ACT_PER_TENSOR;
    const int64_t n16 = T * (int64_t)H / 16;
    int n_part = 0;
    if (per_tensor) {
        n_part = (int)(n16 / 256 + 1 < kAmaxBlocks ? n16 / 256 + 1 : kAmaxBlocks);
        hipLaunchKernelGGL(pr_amax_kernel, dim3(n_part), dim3(256), 0, s, (const uint4*)x_bf16,
                           n16, ws.amax_part);
    }
    const int64_t nblk = ceil_div(T, 4) > 0 ? ceil_div(T, 4) : 1;
    if (nch <= kSmallChunks && (int64_t)num_local * nch <= kSmallTable && num_local <= kSmallLocal) {
#define MOE_LAUNCH_SMALL(MODE)                                                                    \
    hipLaunchKernelGGL(pr_scatter_small_kernel<MODE>, dim3((unsigned)nblk), dim3(256), 0, s,     \
                       (const uint4*)x_bf16, topk_ids, T, H, topk, map, num_local, (int)nch,      \
                       seg_indptr, src2dst, dst2src, a_q, a_scale, ws.amax_part, n_part, m_cap)
        if (act_quant == MOE_ACT_PER_TENSOR) MOE_LAUNCH_SMALL(MOE_ACT_PER_TENSOR);
        else if (act_quant == MOE_ACT_PER_TOKEN) MOE_LAUNCH_SMALL(MOE_ACT_PER_TOKEN);
        else MOE_LAUNCH_SMALL(MOE_ACT_PER_GROUP);
#undef MOE_LAUNCH_SMALL
        return launch_status();
    }
    if (nch <= kFusedChunks && (int64_t)num_local * nch <= kFusedTable) {
        hipLaunchKernelGGL(pr_count_scan_kernel, dim3(1), dim3(1024), 0, s, topk_ids, T * (int64_t)topk, map,
                           num_local, (int)nch, src2dst, ws.offs, ws.tot, ws.amax_part, n_part, per_tensor,
                           a_scale, ws.tscale);
    } else {
        if (nch > 0 && num_local > 0)
            hipLaunchKernelGGL(pr_count_kernel, dim3((unsigned)nch), dim3(64),
                               sizeof(int32_t) * num_local, s, topk_ids, T * (int64_t)topk, map,
                               num_local, nch, src2dst, ws.counts);
        hipLaunchKernelGGL(pr_scan_kernel, dim3((unsigned)(num_local > 0 ? num_local : 1)), dim3(256), 0, s,
                           ws.counts, ws.offs, nch, num_local, ws.tot, ws.amax_part, n_part, per_tensor,
                           a_scale, ws.tscale);
    }
    // The scatter grid also writes seg_indptr and clears dst2src[M..m_cap); it
    // always runs, with at least one block.
    {
#define MOE_LAUNCH_SCATTER(MODE)                                                                  \
    hipLaunchKernelGGL(pr_scatter_quant_kernel<MODE>, dim3((unsigned)nblk), dim3(256), 0, s,     \
                       (const uint4*)x_bf16, topk_ids, T, H, topk, map, num_local, nch,          \
                       ws.offs, ws.tot, seg_indptr, src2dst, dst2src, a_q, a_scale, ws.tscale, m_cap)
        if (act_quant == MOE_ACT_PER_TENSOR) MOE_LAUNCH_SCATTER(MOE_ACT_PER_TENSOR);
        else if (act_quant == MOE_ACT_PER_TOKEN) MOE_LAUNCH_SCATTER(MOE_ACT_PER_TOKEN);
        else MOE_LAUNCH_SCATTER(MOE_ACT_PER_GROUP);
#undef MOE_LAUNCH_SCATTER
    }
    return launch_status();
}
}  // namespace moe

extern "C" int moe_pre_reorder_quant(const void* x_bf16, const int32_t* topk_ids, int64_t T,
                                     int32_t H, int32_t topk, int32_t expert_start,
                                     int32_t num_local, int32_t act_quant, int64_t m_cap,
                                     uint8_t* a_q, float* a_scale, int64_t a_scale_numel,
                                     int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return moe::pre_reorder_impl(x_bf16, topk_ids, T, H, topk, expert_start, num_local, 0, 0,
                                 act_quant, m_cap, a_q, a_scale, a_scale_numel, src2dst, dst2src,
                                 seg_indptr, workspace, workspace_bytes, stream);
}

extern "C" int moe_pre_reorder_quant_shared(const void* x_bf16, const int32_t* topk_ids, int64_t T,
                                            int32_t H, int32_t topk, int32_t expert_start,
                                            int32_t num_routed, int32_t shared_base,
                                            int32_t n_shared, int32_t act_quant, int64_t m_cap,
                                            uint8_t* a_q, float* a_scale, int64_t a_scale_numel,
                                            int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr,
                                            void* workspace, size_t workspace_bytes, void* stream) {
    return moe::pre_reorder_impl(x_bf16, topk_ids, T, H, topk, expert_start, num_routed, shared_base,
                                 n_shared, act_quant, m_cap, a_q, a_scale, a_scale_numel, src2dst,
                                 dst2src, seg_indptr, workspace, workspace_bytes, stream);
}

// ---- the variant that allocates nothing ------------------------------------------
//
// moe_pre_reorder_quant_noalloc runs the same three kernels with their scratch
// (chunk counts, offsets, per-expert totals, amax partials, the per-tensor
// scale) in `scratch`, a static device array that every GPU the library runs
// on holds until the process ends. In host code the array's name is only a
// host-side stand-in: the device address is taken with hipGetSymbolAddress on
// the first call on each device (with that device current) and kept per device;
// only that address reaches the kernels. The kernels write every scratch entry
// they later read, so nothing needs clearing between calls; calls that overlap
// on one GPU share the array and race.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" int moe_pre_reorder_quant_noalloc(const void* x_bf16, const int32_t* topk_ids, int64_t T,
                                             int32_t H, int32_t topk, int32_t expert_start,
                                             int32_t num_local, int32_t act_quant, int64_t m_cap,
                                             uint8_t* a_q, float* a_scale, int64_t a_scale_numel,
                                             int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr,
                                             void* stream) {
    using namespace moe;
    if (T < 0 || topk <= 0 || num_local < 0) return MOE_ERR_INVALID_ARG;
    if (topk > 32 || num_local > 8192 || T * (int64_t)topk > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (pre_ws_bytes(T, topk, num_local) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != MOE_OK) return rc;
    return pre_reorder_impl(x_bf16, topk_ids, T, H, topk, expert_start, num_local, 0, 0, act_quant,
                            m_cap, a_q, a_scale, a_scale_numel, src2dst, dst2src, seg_indptr, ws,
                            (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
