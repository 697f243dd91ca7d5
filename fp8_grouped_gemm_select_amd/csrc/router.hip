// Router projection before the gate: logits[t, e] = sum_h x[t, h] * wg[e, h]
// (bf16 inputs, fp32 accumulation on the CDNA4 bf16 MFMA), then stage 1 on
// those logits. The pages' fused gate starts from the router's logits ("[1/2]
// sgl-kernel: Fuse routed scaling factor into select_experts", sglang PR #8364,
// Motivation); this completes the layer from the hidden states.
//
// Tiles of 64 tokens x 128 experts, one 256-thread block each (4 waves, a wave
// owns 32 experts x 64 tokens = 2 x 4 MFMA 16x16x32 blocks, issued as W x X so
// that a lane holds four adjacent experts of one token). K advances by 64 bf16
// (128 bytes); x and wg rows are staged through registers into two LDS buffers
// (step k+1 in flight while step k's MFMAs run), 16-byte chunk c of row r at
// c ^ perm(r), which keeps the row stores and the 16-row operand reads free of
// bank conflicts. K past H, tokens past T and experts past E read as zeros.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int RBM = 64, RBN = 128, RBK = 64;  // tokens, experts, bf16 per K step
constexpr int kRThreads = 256;
constexpr int kRRow = RBK * 2;                 // 128 bytes per staged row

__device__ __forceinline__ int rperm(int r) { return (r & 6) | ((r ^ (r >> 3)) & 1); }
__device__ __forceinline__ int rswz(int r, int c) { return r * kRRow + ((c ^ rperm(r)) << 4); }

__global__ __launch_bounds__(kRThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wg,
                                                                  int64_t T, int H, int E,
                                                                  float* __restrict__ logits) {
    __shared__ __align__(16) uint8_t lds[2][(RBM + RBN) * kRRow];  // 2 x 24 KB
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RBM;
    const int e0 = blockIdx.y * RBN;
    const int lr = tid >> 3, lc = tid & 7;  // staged row (+32 i), 16-byte chunk

    uint4 rx[2], rw[4];
    auto gload = [&](int kk) {  // kk: first bf16 column of the step
        const int col = kk + lc * 8;
        const bool kin = col < H;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t t = t0 + lr + 32 * i;
            rx[i] = (kin && t < T) ? *(const uint4*)(x + t * H + col) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e0 + lr + 32 * i;
            rw[i] = (kin && e < E) ? *(const uint4*)(wg + (int64_t)e * H + col) : make_uint4(0, 0, 0, 0);
        }
    };
    auto operand = [&](const uint8_t* base, int row, int c) {
        return __builtin_bit_cast(v8bf, *(const uint4*)(base + rswz(row, c)));
    };

    v4f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (H + RBK - 1) / RBK;
    gload(0);
    for (int k = 0; k < nk; ++k) {
        uint8_t* lx = lds[k & 1];
        uint8_t* lw = lx + RBM * kRRow;
#pragma unroll
        for (int i = 0; i < 2; ++i) *(uint4*)(lx + rswz(lr + 32 * i, lc)) = rx[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4*)(lw + rswz(lr + 32 * i, lc)) = rw[i];
        __syncthreads();  // buffer k & 1 complete; it was last read two steps ago
        if (k + 1 < nk) gload((k + 1) * RBK);
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // two MFMA K slices of 32 bf16
            const int c = 4 * s + (lane >> 4);
            v8bf wf[2], xf[4];
#pragma unroll
            for (int j = 0; j < 2; ++j) wf[j] = operand(lw, wid * 32 + j * 16 + (lane & 15), c);
#pragma unroll
            for (int i = 0; i < 4; ++i) xf[i] = operand(lx, i * 16 + (lane & 15), c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        }
    }
    // acc[i][j][v]: token t0 + 16 i + lane % 16, expert e0 + 32 wid + 16 j + 4 (lane / 16) + v
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = e0 + wid * 32 + j * 16 + (lane >> 4) * 4;
            if (t < T && e < E) *(float4*)(logits + t * E + e) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

}  // namespace
}  // namespace moe

extern "C" int moe_router_select(const void* x_bf16, const void* wg_bf16, const float* correction_bias,
                                 int64_t T, int32_t H, int32_t E, int32_t topk, int32_t n_group,
                                 int32_t topk_group, int32_t score_fn, int32_t renormalize,
                                 float routed_scaling_factor, int32_t apply_rsf, float* logits,
                                 int32_t* topk_ids, float* topk_weights, void* stream) {
    using namespace moe;
    if (T < 0 || H <= 0 || E <= 0) return MOE_ERR_INVALID_ARG;
    if (H % 8 != 0 || E % 4 != 0) return MOE_ERR_UNSUPPORTED;
    if (T * (int64_t)E > ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !wg_bf16 || !logits) return MOE_ERR_NULL;
    if (!aligned16(x_bf16) || !aligned16(wg_bf16) || !aligned16(logits)) return MOE_ERR_INVALID_ARG;
    // stage-1 arguments are checked before anything is launched
    if (topk <= 0 || n_group <= 0 || topk_group <= 0 || topk > 32 || topk > E || E > 512 || n_group > 64 ||
        E % n_group != 0 || topk_group > n_group || (int64_t)topk_group * (E / n_group) < topk ||
        (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) ||
        (score_fn == MOE_SCORE_SOFTMAX && (correction_bias || n_group > 1)))
        return launch_select_experts(logits, correction_bias, T, E, topk, n_group, topk_group, score_fn,
                                     renormalize, routed_scaling_factor, apply_rsf, topk_ids,
                                     topk_weights, (hipStream_t)stream, 0, 0.0f);  // returns the precise error
    if (!topk_ids || !topk_weights) return MOE_ERR_NULL;
    if (!aligned16(topk_ids) || !aligned16(topk_weights)) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)ceil_div(T, RBM), (unsigned)ceil_div(E, RBN));
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kRThreads), 0, s, (const uint16_t*)x_bf16,
                       (const uint16_t*)wg_bf16, T, H, E, logits);
    const int st = launch_status();
    if (st != MOE_OK) return st;
    return launch_select_experts(logits, correction_bias, T, E, topk, n_group, topk_group, score_fn,
                                 renormalize, routed_scaling_factor, apply_rsf, topk_ids, topk_weights, s,
                                 0, 0.0f);
}
