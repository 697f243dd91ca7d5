// Stage 4: SiLU(gate) * up rounded to bf16, then dynamic FP8 requantisation of
// the w2 input, one wavefront per row over the M rows that exist on the device.
//
// Follows "Support token-level quantization for EP MoE" (sglang PR #6782),
// change summary of layer.py: down_input comes out of the activation in the
// activation dtype and is then quantised per token, giving w2_input_scale.
//
// Per row and per 128-column group the whole step is one pass (h stays in
// registers between the amax and the encode for rows up to 8192 wide; all of
// a row's loads are issued before the first is used). The
// per-tensor mode needs the maximum over all M*I values first: pass 1 writes a
// partial maximum per block, evaluating SiLU only for values whose cheap upper
// bound could raise the maximum; pass 2 reduces the partials in every block and
// computes h while encoding (re-reading gate/up costs the same bytes as storing
// and re-reading h).
#include "common.h"

namespace moe {
namespace {

constexpr int kActBlocks = 2048;  // fixed grid of the per-tensor passes (partials buffer)

struct ActWs {
    float* part;  // [kActBlocks]
};

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ __forceinline__ int64_t rows_present(const int32_t* seg, int num_local, int64_t m_cap) {
    int64_t M = seg[num_local];
    return M < 0 ? 0 : (M > m_cap ? m_cap : M);
}

// h for 16 consecutive columns [c, c+16) of `row` (packed bf16 pairs), zeros past I.
__device__ __forceinline__ void silu_mul16(const uint16_t* __restrict__ gu, int64_t row, int I, int c,
                                           uint4& h0, uint4& h1) {
    if (c >= I) {
        h0 = make_uint4(0, 0, 0, 0);
        h1 = h0;
        return;
    }
    const uint4* g4 = (const uint4*)(gu + row * 2 * (int64_t)I + c);
    const uint4* u4 = (const uint4*)(gu + row * 2 * (int64_t)I + I + c);
    const uint4 ga = g4[0], gb = g4[1], ua = u4[0], ub = u4[1];
    const uint32_t g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
    const uint32_t u[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
    uint32_t h[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float g0 = bf16_lo(g[q]), g1 = bf16_hi(g[q]);
        const float u0 = bf16_lo(u[q]), u1 = bf16_hi(u[q]);
        h[q] = bf16x2_rne(silu_fixed(g0) * u0, silu_fixed(g1) * u1);
    }
    h0 = make_uint4(h[0], h[1], h[2], h[3]);
    h1 = make_uint4(h[4], h[5], h[6], h[7]);
}

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

// gate / up bf16 of 16 consecutive columns [c, c+16) of `row`; columns past I
// read column 0 (a valid address) and are zeroed later by silu_mul16_from.
struct GU16 {
    uint4 ga, gb, ua, ub;
};
__device__ __forceinline__ GU16 load_gu16(const uint16_t* __restrict__ gu, int64_t row, int I, int c) {
    const int cc = c < I ? c : 0;
    const uint4* g4 = (const uint4*)(gu + row * 2 * (int64_t)I + cc);
    const uint4* u4 = (const uint4*)(gu + row * 2 * (int64_t)I + I + cc);
    GU16 v;
    v.ga = g4[0];
    v.gb = g4[1];
    v.ua = u4[0];
    v.ub = u4[1];
    return v;
}
__device__ __forceinline__ void silu_mul16_from(const GU16& v, int I, int c, uint4& h0, uint4& h1) {
    if (c >= I) {
        h0 = make_uint4(0, 0, 0, 0);
        h1 = h0;
        return;
    }
    const uint32_t g[8] = {v.ga.x, v.ga.y, v.ga.z, v.ga.w, v.gb.x, v.gb.y, v.gb.z, v.gb.w};
    const uint32_t u[8] = {v.ua.x, v.ua.y, v.ua.z, v.ua.w, v.ub.x, v.ub.y, v.ub.z, v.ub.w};
    uint32_t h[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float g0 = bf16_lo(g[q]), g1 = bf16_hi(g[q]);
        const float u0 = bf16_lo(u[q]), u1 = bf16_hi(u[q]);
        h[q] = bf16x2_rne(silu_fixed(g0) * u0, silu_fixed(g1) * u1);
    }
    h0 = make_uint4(h[0], h[1], h[2], h[3]);
    h1 = make_uint4(h[4], h[5], h[6], h[7]);
}

// One wave per row, rows up to NIT * 1024 columns: all of a row's gate / up
// loads are issued before any of them is used.
template <int MODE, int NIT>  // MODE: MOE_ACT_PER_TOKEN or MOE_ACT_PER_GROUP
__global__ __launch_bounds__(256) void act_requant_kernel(const uint16_t* __restrict__ gu,
                                                          const int32_t* __restrict__ seg,
                                                          int num_local, int64_t m_cap, int I,
                                                          uint8_t* __restrict__ a_q,
                                                          float* __restrict__ a_scale) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t M = rows_present(seg, num_local, m_cap);
    const int G = (I + MOE_QB - 1) / MOE_QB;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wid; row < M; row += (int64_t)gridDim.x * 4) {
        uint8_t* out = a_q + row * I;
        GU16 v[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) v[it] = load_gu16(gu, row, I, it * 1024 + lane * 16);
        uint4 hb[NIT][2];
#pragma unroll
        for (int it = 0; it < NIT; ++it) silu_mul16_from(v[it], I, it * 1024 + lane * 16, hb[it][0], hb[it][1]);
        if (MODE == MOE_ACT_PER_GROUP) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int c = it * 1024 + lane * 16;
                float s, inv;
                dyn_scale(group8_max(amax16(hb[it][0], hb[it][1])), s, inv);
                if (c < I) *(uint4*)(out + c) = quant16(hb[it][0], hb[it][1], inv);
                const int g = it * 8 + (lane >> 3);
                if ((lane & 7) == 0 && g < G) a_scale[row * G + g] = s;
            }
            continue;
        }
        float amax = 0.0f;
#pragma unroll
        for (int it = 0; it < NIT; ++it) amax = fmaxf(amax, amax16(hb[it][0], hb[it][1]));
        float s, inv;
        dyn_scale(wave_max(amax), s, inv);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int c = it * 1024 + lane * 16;
            if (c < I) *(uint4*)(out + c) = quant16(hb[it][0], hb[it][1], inv);
        }
        if (lane == 0) a_scale[row] = s;
    }
}

// Per-group mode when a row's 16-column chunks do not fill whole waves (I / 16
// not a multiple of 64, e.g. I = 768, where one wave per row leaves a quarter of
// its lanes idle): the chunks of all rows are numbered row-major and each wave
// takes 64 consecutive ones, so no lane idles. A 128-column group is 8
// consecutive chunks of one row (I is a multiple of 128 here), so the group
// maximum stays an 8-lane reduction; lanes past the last chunk form whole
// groups of their own. Same values and scales as act_requant_kernel.
__global__ __launch_bounds__(256) void act_requant_group_flat_kernel(const uint16_t* __restrict__ gu,
                                                                     const int32_t* __restrict__ seg,
                                                                     int num_local, int64_t m_cap, int I,
                                                                     uint8_t* __restrict__ a_q,
                                                                     float* __restrict__ a_scale) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t M = rows_present(seg, num_local, m_cap);
    const int cpr = I / 16;  // chunks per row, a multiple of 8
    const int G = I / MOE_QB;
    const int64_t total = M * cpr;
    for (int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 64; base < total; base += (int64_t)gridDim.x * 256) {
        const int64_t t = base + lane;
        const bool ok = t < total;
        const int64_t row = ok ? t / cpr : 0;
        const int c = ok ? (int)(t - row * cpr) * 16 : I;  // c = I: no columns (zeros)
        const GU16 v = load_gu16(gu, row, I, c);
        uint4 h0, h1;
        silu_mul16_from(v, I, c, h0, h1);
        float s, inv;
        dyn_scale(group8_max(amax16(h0, h1)), s, inv);
        if (ok) {
            *(uint4*)(a_q + row * I + c) = quant16(h0, h1, inv);
            if ((lane & 7) == 0) a_scale[row * G + c / MOE_QB] = s;
        }
    }
}

// Rows wider than 8192 columns (per token / per group): streamed, two passes
// over the row for the per-token maximum.
template <int MODE>
__global__ __launch_bounds__(256) void act_requant_wide_kernel(const uint16_t* __restrict__ gu,
                                                               const int32_t* __restrict__ seg,
                                                               int num_local, int64_t m_cap, int I,
                                                               uint8_t* __restrict__ a_q,
                                                               float* __restrict__ a_scale) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t M = rows_present(seg, num_local, m_cap);
    const int nit = (I + 1023) / 1024;
    const int G = (I + MOE_QB - 1) / MOE_QB;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wid; row < M; row += (int64_t)gridDim.x * 4) {
        uint8_t* out = a_q + row * I;
        float s = 0.0f, inv = 0.0f;
        if (MODE == MOE_ACT_PER_TOKEN) {
            float amax = 0.0f;
            for (int it = 0; it < nit; ++it) {
                uint4 h0, h1;
                silu_mul16(gu, row, I, it * 1024 + lane * 16, h0, h1);
                amax = fmaxf(amax, amax16(h0, h1));
            }
            dyn_scale(wave_max(amax), s, inv);
        }
        for (int it = 0; it < nit; ++it) {
            const int c = it * 1024 + lane * 16;
            uint4 h0, h1;
            silu_mul16(gu, row, I, c, h0, h1);
            if (MODE == MOE_ACT_PER_GROUP) {
                dyn_scale(group8_max(amax16(h0, h1)), s, inv);
                const int g = it * 8 + (lane >> 3);
                if ((lane & 7) == 0 && g < G) a_scale[row * G + g] = s;
            }
            if (c < I) *(uint4*)(out + c) = quant16(h0, h1, inv);
        }
        if (MODE == MOE_ACT_PER_TOKEN && lane == 0) a_scale[row] = s;
    }
}

// per tensor, pass 1: partial maxima of |h|, with SiLU evaluated only where it
// can matter. For every value, |h| = |bf16(silu(g) * u)| <= max(g, 0.28) * |u|
// * (1 + 2^-7): silu(g) = g / (1 + exp(-g)) divides by at least 1, so it never
// exceeds g, and for g < 0 its magnitude stays below 0.2785; the fp32 product
// and the bf16 rounding add less than 2^-7. A group of 1024 values (16 per lane)
// is evaluated exactly only if some value's bound times 1.01 reaches the wave's
// running maximum of exact |h| values; otherwise none of them can raise it. The
// value that attains the maximum is always evaluated exactly, so the result is
// the same maximum as evaluating every value (fmaxf ignores NaN either way).
__global__ __launch_bounds__(256) void act_amax_kernel(const uint16_t* __restrict__ gu,
                                                       const int32_t* __restrict__ seg, int num_local,
                                                       int64_t m_cap, int I, float* __restrict__ part) {
    __shared__ float red[4];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t M = rows_present(seg, num_local, m_cap);
    const int nit = (I + 1023) / 1024;
    float amax = 0.0f;  // wave-uniform: maximum of the exact |h| seen so far
    for (int64_t row = (int64_t)blockIdx.x * 4 + wid; row < M; row += (int64_t)gridDim.x * 4)
        for (int it = 0; it < nit; ++it) {
            const int c = it * 1024 + lane * 16;
            const GU16 v = load_gu16(gu, row, I, c);
            const uint32_t g[8] = {v.ga.x, v.ga.y, v.ga.z, v.ga.w, v.gb.x, v.gb.y, v.gb.z, v.gb.w};
            const uint32_t u[8] = {v.ua.x, v.ua.y, v.ua.z, v.ua.w, v.ub.x, v.ub.y, v.ub.z, v.ub.w};
            float bound = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                bound = fmaxf(bound, fmaxf(bf16_lo(g[q]), 0.28f) * fabsf(bf16_lo(u[q])));
                bound = fmaxf(bound, fmaxf(bf16_hi(g[q]), 0.28f) * fabsf(bf16_hi(u[q])));
            }
            const bool cand = c < I && !(bound * 1.01f < amax);  // NaN bounds count as candidates
            if (__builtin_amdgcn_ballot_w64(cand) == 0) continue;
            uint4 h0, h1;
            silu_mul16_from(v, I, c, h0, h1);
            amax = wave_max(fmaxf(amax, amax16(h0, h1)));
        }
    if (lane == 0) red[wid] = amax;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// per tensor, pass 2: every block reduces the partials, then encodes its rows
__global__ __launch_bounds__(256) void act_quant_tensor_kernel(const uint16_t* __restrict__ gu,
                                                               const int32_t* __restrict__ seg,
                                                               int num_local, int64_t m_cap, int I,
                                                               const float* __restrict__ part,
                                                               int n_part, uint8_t* __restrict__ a_q,
                                                               float* __restrict__ a_scale) {
    __shared__ float red[4];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float m = 0.0f;
    for (int i = threadIdx.x; i < n_part; i += 256) m = fmaxf(m, part[i]);
    m = wave_max(m);
    if (lane == 0) red[wid] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float s, inv;
    dyn_scale(amax, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) a_scale[0] = s;
    const int64_t M = rows_present(seg, num_local, m_cap);
    const int nit = (I + 1023) / 1024;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wid; row < M; row += (int64_t)gridDim.x * 4)
        for (int it = 0; it < nit; ++it) {
            const int c = it * 1024 + lane * 16;
            uint4 h0, h1;
            silu_mul16(gu, row, I, c, h0, h1);
            if (c < I) *(uint4*)(a_q + row * I + c) = quant16(h0, h1, inv);
        }
}

}  // namespace

size_t act_requant_ws_bytes() { return align256(sizeof(float) * kActBlocks); }

}  // namespace moe

extern "C" int moe_act_requant(const void* gateup_bf16, const int32_t* seg_indptr, int32_t num_local,
                               int64_t m_cap, int32_t I, int32_t act_quant, uint8_t* a_q,
                               float* a_scale, int64_t a_scale_numel, void* workspace,
                               size_t workspace_bytes, void* stream) {
    using namespace moe;
    if (num_local < 0 || m_cap < 0 || I <= 0) return MOE_ERR_INVALID_ARG;
    if (act_quant < MOE_ACT_PER_TENSOR || act_quant > MOE_ACT_PER_GROUP) return MOE_ERR_INVALID_ARG;
    if (I % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (m_cap * (int64_t)I > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    const int64_t G = ceil_div(I, MOE_QB);
    const int64_t want = act_quant == MOE_ACT_PER_TENSOR ? 1 : act_quant == MOE_ACT_PER_TOKEN ? m_cap : m_cap * G;
    if (a_scale_numel != want) return MOE_ERR_SHAPE;
    if (!seg_indptr) return MOE_ERR_NULL;
    if (act_quant == MOE_ACT_PER_TENSOR && (!workspace || workspace_bytes < act_requant_ws_bytes()))
        return MOE_ERR_WORKSPACE;
    if (m_cap == 0 && act_quant != MOE_ACT_PER_TENSOR) return MOE_OK;
    if (!a_scale || (m_cap > 0 && (!gateup_bf16 || !a_q))) return MOE_ERR_NULL;
    if ((gateup_bf16 && !aligned16(gateup_bf16)) || (a_q && !aligned16(a_q))) return MOE_ERR_INVALID_ARG;

    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const uint16_t* gu = (const uint16_t*)gateup_bf16;
    if (act_quant == MOE_ACT_PER_TENSOR) {
        float* part = (float*)workspace;
        hipLaunchKernelGGL(act_amax_kernel, dim3(kActBlocks), dim3(256), 0, s, gu, seg_indptr,
                           num_local, m_cap, I, part);
        hipLaunchKernelGGL(act_quant_tensor_kernel, dim3(kActBlocks), dim3(256), 0, s, gu,
                           seg_indptr, num_local, m_cap, I, part, kActBlocks, a_q, a_scale);
        return launch_status();
    }
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (act_quant == MOE_ACT_PER_GROUP && I % MOE_QB == 0 && (I / 16) % 64 != 0) {
        int64_t g = ceil_div(ceil_div(m_cap * (I / 16), 64), 4);  // blocks of four 64-chunk waves
        if (g > cap) g = cap;
        if (g < 1) g = 1;
        hipLaunchKernelGGL(act_requant_group_flat_kernel, dim3((unsigned)g), dim3(256), 0, s, gu, seg_indptr,
                           num_local, m_cap, I, a_q, a_scale);
        return launch_status();
    }
    int64_t grid = ceil_div(m_cap, 4);
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    const int nit = (int)ceil_div(I, 1024);
#define MOE_LAUNCH_ACT(MODE)                                                                        \
    do {                                                                                            \
        if (nit <= 1)                                                                               \
            hipLaunchKernelGGL((act_requant_kernel<MODE, 1>), dim3((unsigned)grid), dim3(256), 0, s, gu, \
                               seg_indptr, num_local, m_cap, I, a_q, a_scale);                     \
        else if (nit <= 2)                                                                          \
            hipLaunchKernelGGL((act_requant_kernel<MODE, 2>), dim3((unsigned)grid), dim3(256), 0, s, gu, \
                               seg_indptr, num_local, m_cap, I, a_q, a_scale);                     \
        else if (nit <= 4)                                                                          \
            hipLaunchKernelGGL((act_requant_kernel<MODE, 4>), dim3((unsigned)grid), dim3(256), 0, s, gu, \
                               seg_indptr, num_local, m_cap, I, a_q, a_scale);                     \
        else if (nit <= 8)                                                                          \
            hipLaunchKernelGGL((act_requant_kernel<MODE, 8>), dim3((unsigned)grid), dim3(256), 0, s, gu, \
                               seg_indptr, num_local, m_cap, I, a_q, a_scale);                     \
        else                                                                                        \
            hipLaunchKernelGGL((act_requant_wide_kernel<MODE>), dim3((unsigned)grid), dim3(256), 0, s, gu, \
                               seg_indptr, num_local, m_cap, I, a_q, a_scale);                     \
    } while (0)
    if (act_quant == MOE_ACT_PER_TOKEN) MOE_LAUNCH_ACT(MOE_ACT_PER_TOKEN);
    else MOE_LAUNCH_ACT(MOE_ACT_PER_GROUP);
#undef MOE_LAUNCH_ACT
    return launch_status();
}
