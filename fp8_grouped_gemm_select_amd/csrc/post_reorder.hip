// Stage 5: top-k weighted combine of the expert outputs back to token order,
// one wavefront per token.
//
// Follows "[1/2] sgl-kernel: Fuse routed scaling factor into select_experts"
// (sglang PR #8364), Motivation: moe_sum_reduce is the weighted sum of each
// token's selected expert outputs. The weights arrive from the gate with the
// routed scaling factor already folded in (or not, as the caller chose); this
// stage never applies it.
#include "common.h"

namespace moe {
namespace {

// topk <= 8 (or 16): the token's local slots are compacted in slot order (n of them,
// wave-uniform); each lane covers 16 columns (32 bytes) per iteration and the
// loads of U iterations of all n slots are issued together, then accumulated
// in slot order (the same fp32 order as the general kernel below). Fewer local
// slots leave room for more iterations in flight: U = 4 for n <= 2, 2 for
// n <= 4, else 1.
template <int S, int U>
__device__ __forceinline__ void combine_token(const uint16_t* __restrict__ down, const int (&rows)[S],
                                              const float (&wj)[S], int n, int H, int lane,
                                              uint16_t* __restrict__ orow) {
    for (int c0 = lane * 16; c0 < H; c0 += 1024 * U) {
        uint4 v[S][U][2];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s < n) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * 1024;
                    if (c < H) {
                        const uint4* p = (const uint4*)(down + (int64_t)rows[s] * H + c);
                        v[s][u][0] = p[0];
                        v[s][u][1] = p[1];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 1024;
            if (c >= H) break;
            float acc[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (s < n) {
                    const uint32_t d[8] = {v[s][u][0].x, v[s][u][0].y, v[s][u][0].z, v[s][u][0].w,
                                           v[s][u][1].x, v[s][u][1].y, v[s][u][1].z, v[s][u][1].w};
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        acc[2 * q] = acc[2 * q] + wj[s] * bf16_lo(d[q]);
                        acc[2 * q + 1] = acc[2 * q + 1] + wj[s] * bf16_hi(d[q]);
                    }
                }
            }
            uint32_t o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = bf16x2_rne(acc[2 * q], acc[2 * q + 1]);
            uint4* po = (uint4*)(orow + c);
            po[0] = make_uint4(o[0], o[1], o[2], o[3]);
            po[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

// KMAX = 8 (topk <= 8) or 16 (topk <= 16, e.g. eight routed slots and a shared
// expert's); the 16-slot instance adds a path for 9-16 local slots and is a
// separate kernel, so that its registers do not lower the 8-slot one's occupancy.
template <int KMAX>
__global__ __launch_bounds__(256) void post_reorder8_kernel(const uint16_t* __restrict__ down,
                                                            const int32_t* __restrict__ src2dst,
                                                            const float* __restrict__ w, int64_t T,
                                                            int H, int topk, int64_t m_cap,
                                                            uint16_t* __restrict__ out) {
    constexpr int K8 = KMAX;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    if (t >= T) return;
    int r = -1;
    float wt = 0.0f;
    if (lane < topk) {
        const int32_t v = src2dst[t * topk + lane];
        if (v >= 0 && v < m_cap) {
            r = v;
            wt = w[t * topk + lane];
        }
    }
    // local slots in ascending slot order: rows[q], wj[q] for q < n
    uint64_t m = __ballot(r >= 0);
    const int n = __builtin_popcountll(m);
    int rows[K8];
    float wj[K8];
#pragma unroll
    for (int q = 0; q < K8; ++q) {
        const int j = m ? __builtin_ctzll(m) : 0;
        m &= m - 1;
        rows[q] = __builtin_amdgcn_readlane(r, j);
        wj[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j));
    }
    uint16_t* orow = out + t * H;
    if (n <= 2) {
        const int r2[2] = {rows[0], rows[1]};
        const float w2[2] = {wj[0], wj[1]};
        combine_token<2, 4>(down, r2, w2, n, H, lane, orow);
    } else if (n <= 4) {
        const int r4[4] = {rows[0], rows[1], rows[2], rows[3]};
        const float w4[4] = {wj[0], wj[1], wj[2], wj[3]};
        combine_token<4, 2>(down, r4, w4, n, H, lane, orow);
    } else if (KMAX == 8 || n <= 8) {
        int r8[8];
        float w8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            r8[q] = rows[q];
            w8[q] = wj[q];
        }
        combine_token<8, 1>(down, r8, w8, n, H, lane, orow);
    } else {
        combine_token<K8, 1>(down, rows, wj, n, H, lane, orow);
    }
}

// any topk: one 16-byte column group per lane per iteration, slots one by one
__global__ __launch_bounds__(256) void post_reorder_kernel(const uint16_t* __restrict__ down,
                                                           const int32_t* __restrict__ src2dst,
                                                           const float* __restrict__ w, int64_t T,
                                                           int H, int topk, int64_t m_cap,
                                                           uint16_t* __restrict__ out) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wid;
    if (t >= T) return;
    int r = -1;
    float wt = 0.0f;
    if (lane < topk) {
        const int32_t v = src2dst[t * topk + lane];
        if (v >= 0 && v < m_cap) {
            r = v;
            wt = w[t * topk + lane];
        }
    }
    const uint64_t mask = __ballot(r >= 0);
    for (int c = lane * 8; c < H; c += 512) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        uint64_t m = mask;
        while (m) {
            const int j = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            const int rj = __builtin_amdgcn_readlane(r, j);
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), j));
            const uint4 v = *(const uint4*)(down + (int64_t)rj * H + c);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = acc[2 * q] + wj * bf16_lo(d[q]);
                acc[2 * q + 1] = acc[2 * q + 1] + wj * bf16_hi(d[q]);
            }
        }
        uint4 o;
        o.x = bf16x2_rne(acc[0], acc[1]);
        o.y = bf16x2_rne(acc[2], acc[3]);
        o.z = bf16x2_rne(acc[4], acc[5]);
        o.w = bf16x2_rne(acc[6], acc[7]);
        *(uint4*)(out + t * H + c) = o;
    }
}

}  // namespace
}  // namespace moe

extern "C" int moe_post_reorder(const void* down_bf16, const int32_t* src2dst,
                                const float* topk_weights, int64_t T, int32_t H, int32_t topk,
                                int64_t m_cap, void* out_bf16, void* stream) {
    using namespace moe;
    if (T < 0 || H <= 0 || topk <= 0 || m_cap < 0) return MOE_ERR_INVALID_ARG;
    if (H % 16 != 0 || topk > 64) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!src2dst || !topk_weights || !out_bf16 || (m_cap > 0 && !down_bf16)) return MOE_ERR_NULL;
    if ((down_bf16 && !aligned16(down_bf16)) || !aligned16(out_bf16)) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    if (topk <= 8)
        hipLaunchKernelGGL(post_reorder8_kernel<8>, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0,
                           (hipStream_t)stream, (const uint16_t*)down_bf16, src2dst, topk_weights, T,
                           H, topk, m_cap, (uint16_t*)out_bf16);
    else if (topk <= 16)
        hipLaunchKernelGGL(post_reorder8_kernel<16>, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0,
                           (hipStream_t)stream, (const uint16_t*)down_bf16, src2dst, topk_weights, T,
                           H, topk, m_cap, (uint16_t*)out_bf16);
    else
        hipLaunchKernelGGL(post_reorder_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0,
                           (hipStream_t)stream, (const uint16_t*)down_bf16, src2dst, topk_weights, T,
                           H, topk, m_cap, (uint16_t*)out_bf16);
    return launch_status();
}
