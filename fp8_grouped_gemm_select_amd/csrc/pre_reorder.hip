// Stage 2: permutation of (token, slot) pairs into expert-contiguous rows and
// dynamic FP8 quantisation of the token rows into those rows.
//
// Follows "Support token-level quantization for EP MoE" (sglang PR #6782),
// change summary of pre_reorder_triton_kernel and EPMoELayer: per-token maxima
// give per-token scales, and the scales travel with the rows through src2dst.
// Here the scale reorder is fused into the scatter.
//
// A deterministic stable counting sort in three launches (plus one amax pass in
// the per-tensor mode):
//   count    one wave per chunk of kChunkTok tokens: chunk-local stable rank of
//            every local pair (kept in src2dst) and per-expert chunk counts;
//   scan     one block: per-expert exclusive scan over chunks, then over
//            experts -> seg_indptr; per-tensor amax partials -> one scale;
//   scatter  one wave per token: final rows, dst2src, and the quantised row
//            written to each of the token's local rows.
#include "common.h"

namespace moe {
namespace {

constexpr int kChunkTok = 64;
constexpr int kRegIters = 8;   // rows up to 8192 wide stay in registers
constexpr int kAmaxBlocks = 1024;

struct PreWs {
    int32_t* counts;   // [nchunks][num_local]
    int32_t* offs;     // [nchunks][num_local]
    float* amax_part;  // [kAmaxBlocks]
    float* tscale;     // [2]: per-tensor scale, inverse
};

__host__ __device__ inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

inline size_t pre_ws_bytes(int64_t T, int32_t num_local) {
    const int64_t nch = ceil_div(T, kChunkTok);
    size_t b = 0;
    b += align256(sizeof(int32_t) * (size_t)(nch * num_local));
    b += align256(sizeof(int32_t) * (size_t)(nch * num_local));
    b += align256(sizeof(float) * kAmaxBlocks);
    b += align256(sizeof(float) * 2);
    return b;
}

inline PreWs pre_ws_carve(void* ws, int64_t T, int32_t num_local) {
    const int64_t nch = ceil_div(T, kChunkTok);
    char* p = (char*)ws;
    PreWs w;
    w.counts = (int32_t*)p;
    p += align256(sizeof(int32_t) * (size_t)(nch * num_local));
    w.offs = (int32_t*)p;
    p += align256(sizeof(int32_t) * (size_t)(nch * num_local));
    w.amax_part = (float*)p;
    p += align256(sizeof(float) * kAmaxBlocks);
    w.tscale = (float*)p;
    return w;
}

// ---- count: chunk-local stable ranks -----------------------------------------
__global__ __launch_bounds__(64) void pr_count_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int topk, int expert_start, int num_local,
                                                      int32_t* __restrict__ src2dst,
                                                      int32_t* __restrict__ counts) {
    extern __shared__ int32_t cnt[];
    const int lane = threadIdx.x;
    const int64_t chunk = blockIdx.x;
    for (int e = lane; e < num_local; e += 64) cnt[e] = 0;
    __syncthreads();
    const int64_t f0 = chunk * kChunkTok * topk;
    const int64_t t1 = (chunk + 1) * kChunkTok < T ? (chunk + 1) * kChunkTok : T;
    const int64_t f1 = t1 * topk;
    for (int64_t base = f0; base < f1; base += 64) {
        const int64_t f = base + lane;
        const int e = f < f1 ? ids[f] - expert_start : -1;
        const bool local = e >= 0 && e < num_local;
        bool pending = local;
        int rank = -1;
        // Resolve one expert value per round: lanes holding it take consecutive
        // ranks in lane (= pair) order after the chunk's running count.
        while (true) {
            const uint64_t m = __ballot(pending);
            if (m == 0) break;
            const int leader = __ffsll((unsigned long long)m) - 1;
            const int v = __shfl(e, leader, MOE_WAVE);
            const uint64_t same = __ballot(pending && e == v);
            const int base_cnt = cnt[v];
            if (pending && e == v) {
                rank = base_cnt + __popcll(same & lanemask_lt(lane));
                pending = false;
            }
            if (lane == leader) cnt[v] = base_cnt + __popcll(same);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS write done before the next read
        }
        if (f < f1) src2dst[f] = local ? rank : -1;
    }
    __syncthreads();
    for (int e = lane; e < num_local; e += 64) counts[chunk * num_local + e] = cnt[e];
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

// ---- scan: segment starts and per-chunk offsets ------------------------------------
__global__ __launch_bounds__(1024) void pr_scan_kernel(const int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offs, int64_t nchunks,
                                                       int num_local, int32_t* __restrict__ seg,
                                                       const float* __restrict__ amax_part,
                                                       int n_part, int per_tensor,
                                                       float* __restrict__ a_scale,
                                                       float* __restrict__ tscale) {
    __shared__ int scratch[17];
    __shared__ float red[16];
    const int tid = threadIdx.x;
    // experts handled by this thread: a contiguous run
    const int per = (num_local + 1023) / 1024;
    const int e0 = tid * per;
    int mine = 0;
    for (int q = 0; q < per; ++q) {
        const int e = e0 + q;
        if (e >= num_local) break;
        int run = 0;
        int64_t c = 0;
        for (; c + 8 <= nchunks; c += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = counts[(c + u) * num_local + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) { offs[(c + u) * num_local + e] = run; run += v[u]; }
        }
        for (; c < nchunks; ++c) {
            const int v = counts[c * num_local + e];
            offs[c * num_local + e] = run;
            run += v;
        }
        mine += run;
    }
    int total = 0;
    const int excl = block_exclusive_scan(mine, scratch, &total);
    // second pass: write segment starts
    int run = excl;
    for (int q = 0; q < per; ++q) {
        const int e = e0 + q;
        if (e >= num_local) break;
        seg[e] = run;
        int tot_e = 0;
        // total of expert e = offs[last] + counts[last]
        if (nchunks > 0) tot_e = offs[(nchunks - 1) * num_local + e] + counts[(nchunks - 1) * num_local + e];
        run += tot_e;
    }
    if (tid == 0) seg[num_local] = total;
    if (per_tensor) {
        float m = 0.0f;
        for (int i = tid; i < n_part; i += 1024) m = fmaxf(m, amax_part[i]);
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        if (tid == 0) {
            float a = 0.0f;
            for (int i = 0; i < 16; ++i) a = fmaxf(a, red[i]);
            float s, inv;
            dyn_scale(a, s, inv);
            a_scale[0] = s;
            tscale[0] = s;
            tscale[1] = inv;
        }
    }
}

// ---- scatter + quantise ------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void pr_scatter_quant_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ ids, int64_t T, int H, int topk,
    int expert_start, int num_local, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ seg, int32_t* __restrict__ src2dst, int32_t* __restrict__ dst2src,
    uint8_t* __restrict__ a_q, float* __restrict__ a_scale, const float* __restrict__ tscale,
    int64_t m_cap) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;

    // rows M .. m_cap-1 of dst2src are -1 (grid-stride over the whole grid)
    {
        const int64_t M = seg[num_local];
        for (int64_t r = M + (int64_t)blockIdx.x * 256 + threadIdx.x; r < m_cap;
             r += (int64_t)gridDim.x * 256)
            dst2src[r] = -1;
    }
    if (t >= T) return;

    int dst = -1;
    if (lane < topk) {
        const int64_t f = t * topk + lane;
        const int e = ids[f] - expert_start;
        if (e >= 0 && e < num_local) {
            const int64_t chunk = t / kChunkTok;
            dst = seg[e] + offs[chunk * num_local + e] + src2dst[f];
            // rows past m_cap exist only if a token repeats an expert; drop them
            if (dst >= m_cap) dst = -1;
            else dst2src[dst] = (int32_t)f;
        }
        src2dst[f] = dst;
    }
    uint64_t local_mask = __ballot(dst >= 0);
    if (local_mask == 0) return;

    const int G = (H + MOE_QB - 1) / MOE_QB;
    const int nit = (H + 1023) / 1024;  // iterations of 1024 columns (16 per lane)
    const uint4* xr = x + (t * H) / 8;   // 8 bf16 per uint4
    float amax = 0.0f;

    auto load16 = [&](int it, uint4& a, uint4& b) {
        const int c = it * 1024 + lane * 16;
        if (c < H) {
            a = xr[c / 8];
            b = xr[c / 8 + 1];
        } else {
            a = make_uint4(0, 0, 0, 0);
            b = a;
        }
    };
    auto amax16 = [](const uint4& a, const uint4& b) {
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
        return m;
    };
    auto quant16 = [](const uint4& a, const uint4& b, float inv) {
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = quant4(bf16_lo(w[2 * q]), bf16_hi(w[2 * q]), bf16_lo(w[2 * q + 1]),
                          bf16_hi(w[2 * q + 1]), inv);
        return make_uint4(o[0], o[1], o[2], o[3]);
    };
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
        for (int it = 0; it < nit; ++it) {
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
        for (int it = 0; it < nit; ++it) {
            uint4 a, b;
            load16(it, a, b);
            store_rows(it, quant16(a, b, inv));
        }
        return;
    }

    // per token: pass 1 (amax), pass 2 (codes)
    uint4 buf[kRegIters][2];
#pragma unroll
    for (int it = 0; it < kRegIters; ++it) buf[it][0] = buf[it][1] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int it = 0; it < kRegIters; ++it) {
        if (it < nit) {
            load16(it, buf[it][0], buf[it][1]);
            amax = fmaxf(amax, amax16(buf[it][0], buf[it][1]));
        }
    }
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

}  // namespace

size_t pre_reorder_ws_bytes(int64_t T, int32_t num_local) { return pre_ws_bytes(T, num_local); }

}  // namespace moe

extern "C" int moe_pre_reorder_quant(const void* x_bf16, const int32_t* topk_ids, int64_t T,
                                     int32_t H, int32_t topk, int32_t expert_start,
                                     int32_t num_local, int32_t act_quant, int64_t m_cap,
                                     uint8_t* a_q, float* a_scale, int64_t a_scale_numel,
                                     int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    using namespace moe;
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
    const size_t need_ws = pre_ws_bytes(T, num_local);
    if (!workspace || workspace_bytes < need_ws) return MOE_ERR_WORKSPACE;

    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const int64_t nch = ceil_div(T, kChunkTok);
    PreWs ws = pre_ws_carve(workspace, T, num_local);
    if (nch > 0 && num_local > 0)
        hipLaunchKernelGGL(pr_count_kernel, dim3((unsigned)nch), dim3(64),
                           sizeof(int32_t) * num_local, s, topk_ids, T, topk, expert_start,
                           num_local, src2dst, ws.counts);
    const int per_tensor = act_quant == MOE_ACT_PER_TENSOR;
    const int64_t n16 = T * (int64_t)H / 16;
    int n_part = 0;
    if (per_tensor) {
        n_part = (int)(n16 / 256 + 1 < kAmaxBlocks ? n16 / 256 + 1 : kAmaxBlocks);
        hipLaunchKernelGGL(pr_amax_kernel, dim3(n_part), dim3(256), 0, s, (const uint4*)x_bf16,
                           n16, ws.amax_part);
    }
    hipLaunchKernelGGL(pr_scan_kernel, dim3(1), dim3(1024), 0, s, ws.counts, ws.offs, nch,
                       num_local, seg_indptr, ws.amax_part, n_part, per_tensor, a_scale, ws.tscale);
    // The scatter grid also clears dst2src[M..m_cap); give it at least one block.
    const int64_t nblk = ceil_div(T, 4) > 0 ? ceil_div(T, 4) : 1;
    if (m_cap > 0 || T > 0) {
#define MOE_LAUNCH_SCATTER(MODE)                                                                  \
    hipLaunchKernelGGL(pr_scatter_quant_kernel<MODE>, dim3((unsigned)nblk), dim3(256), 0, s,     \
                       (const uint4*)x_bf16, topk_ids, T, H, topk, expert_start, num_local,      \
                       ws.offs, seg_indptr, src2dst, dst2src, a_q, a_scale, ws.tscale, m_cap)
        if (act_quant == MOE_ACT_PER_TENSOR) MOE_LAUNCH_SCATTER(MOE_ACT_PER_TENSOR);
        else if (act_quant == MOE_ACT_PER_TOKEN) MOE_LAUNCH_SCATTER(MOE_ACT_PER_TOKEN);
        else MOE_LAUNCH_SCATTER(MOE_ACT_PER_GROUP);
#undef MOE_LAUNCH_SCATTER
    }
    return launch_status();
}
