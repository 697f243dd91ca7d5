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
// When H % 64 == 0 and E % 64 == 0 the split-K kernel below runs instead.
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

// ---- split-K router GEMM: 128 tokens x 256 experts per block, DMA ring ----
//
// The 64 x 128 tiling above gives every CU one tile and re-reads the router
// weight for every 64 tokens. This kernel takes 128 tokens x 256 experts per
// block and splits K among `nsplit` blocks so that the grid still fills the
// chip: a block's partial logits go to its own slice of the workspace, and
// router_reduce_kernel adds the slices in split order (deterministic). Eight
// waves (2 x 4) own 64 tokens x 64 experts each = 4 x 4 MFMA 16x16x32 bf16
// blocks per 32-deep slice, issued W x X as above. x and wg rows of one
// 64-element K step (128 bytes) go straight to LDS by global_load_lds_dwordx4
// into a three-stage ring (the perm8 layout), loads of step k+2 issued at step
// k after its MFMAs, with explicit waits. Requires H % 64 == 0; rows past T or E re-read the
// last valid row and are not stored.
constexpr int SRM = 128, SRN = 256, SRK = 64;
constexpr int kSRThreads = 512;
constexpr int kSRStages = 3;
constexpr int kSRStageA = SRM * kRRow;          // 16 KB
constexpr int kSRStage = (SRM + SRN) * kRRow;   // 48 KB
constexpr int kSRDmaA = SRM * kRRow / 1024 / 8;  // 2 per wave
constexpr int kSRDmaB = SRN * kRRow / 1024 / 8;  // 4 per wave
constexpr int kSRDma = kSRDmaA + kSRDmaB;

__global__ __launch_bounds__(kSRThreads, 1) void router_splitk_kernel(const uint16_t* __restrict__ x,
                                                                      const uint16_t* __restrict__ wg,
                                                                      int64_t T, int H, int E, int steps_per_split,
                                                                      float* __restrict__ part) {
    __shared__ __align__(16) uint8_t lds[kSRStages * kSRStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 2, wn = wid & 3;
    const int64_t t0 = (int64_t)blockIdx.x * SRM;
    const int e0 = blockIdx.y * SRN;
    const int split = blockIdx.z;
    const int nk_all = H / SRK;
    const int k_begin = split * steps_per_split;
    const int nk = (nk_all - k_begin < steps_per_split ? nk_all - k_begin : steps_per_split);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)lds;
    const int64_t rows_t = T - t0 < SRM ? T - t0 : SRM;
    const int rows_e = E - e0 < SRN ? E - e0 : SRN;

    // per-lane DMA offsets (bytes from the tile's first row at k = 0):
    // instruction i of wave w fills rows 8 (w * n + i) + lane / 8, chunk
    // position lane % 8, which holds global chunk (lane % 8) ^ rperm(row)
    uint32_t a_off[kSRDmaA], b_off[kSRDmaB];
#pragma unroll
    for (int i = 0; i < kSRDmaA; ++i) {
        const int r = (wid * kSRDmaA + i) * 8 + (lane >> 3);
        const int g = r < rows_t ? r : (int)rows_t - 1;
        a_off[i] = (uint32_t)g * (uint32_t)(H * 2) + (uint32_t)((((lane & 7) ^ rperm(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < kSRDmaB; ++i) {
        const int r = (wid * kSRDmaB + i) * 8 + (lane >> 3);
        const int g = r < rows_e ? r : rows_e - 1;
        b_off[i] = (uint32_t)g * (uint32_t)(H * 2) + (uint32_t)((((lane & 7) ^ rperm(r)) << 4));
    }
    const uint8_t* xa = (const uint8_t*)(x + t0 * H);
    const uint8_t* wb = (const uint8_t*)(wg + (int64_t)e0 * H);
    auto issue = [&](int k) {  // DMA of local step k (global step k_begin + k) into stage k % 3
        const uint32_t st = lds0 + (uint32_t)((k % kSRStages) * kSRStage);
        const int64_t kb = (int64_t)(k_begin + k) * kRRow;
        const uint8_t* ab = uniform_ptr(xa + kb);
        const uint8_t* bb = uniform_ptr(wb + kb);
        const uint32_t la = __builtin_amdgcn_readfirstlane(st + wid * kSRDmaA * 1024);
        const uint32_t lb = __builtin_amdgcn_readfirstlane(st + kSRStageA + wid * kSRDmaB * 1024);
#pragma unroll
        for (int i = 0; i < kSRDmaA; ++i) dma16(ab, a_off[i], la + i * 1024);
#pragma unroll
        for (int i = 0; i < kSRDmaB; ++i) dma16(bb, b_off[i], lb + i * 1024);
    };
    auto operand = [&](const uint8_t* base, int row, int c) {
        return __builtin_bit_cast(v8bf, *(const uint4*)(base + rswz(row, c)));
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) issue(0);
    if (nk > 1) issue(1);
    for (int k = 0; k < nk; ++k) {
        if (k + 1 < nk) wait_vmcnt<kSRDma>();  // DMA(k) done; DMA(k+1) may be in flight
        else wait_vmcnt<0>();
        __syncthreads();  // stage k complete; every wave is done with stage k-1
        const uint8_t* lx = lds + (k % kSRStages) * kSRStage;
        const uint8_t* lw = lx + kSRStageA;
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // two MFMA K slices of 32 bf16
            const int c = 4 * s + (lane >> 4);
            v8bf wf[4], xf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[j] = operand(lw, wn * 64 + j * 16 + (lane & 15), c);
#pragma unroll
            for (int i = 0; i < 4; ++i) xf[i] = operand(lx, wm * 64 + i * 16 + (lane & 15), c);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
        }
        // the DMA of step k+2 after this step's MFMAs (into the stage read at step
        // k-1, free since the barrier above)
        __builtin_amdgcn_sched_barrier(0);
        if (k + 2 < nk) issue(k + 2);
    }
    // acc[i][j][v]: token t0 + 64 wm + 16 i + lane % 16, expert e0 + 64 wn + 16 j + 4 (lane / 16) + v
    float* out = part + (int64_t)split * T * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + wm * 64 + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + wn * 64 + j * 16 + (lane >> 4) * 4;
            if (t < T && e < E) *(float4*)(out + t * E + e) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
    }
}

// logits = part[0] + part[1] + ... + part[nsplit-1], in that order (fp32).
__global__ __launch_bounds__(256) void router_reduce_kernel(const float4* __restrict__ part, int64_t n4,
                                                            int nsplit, float4* __restrict__ logits) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        float4 a = part[i];
        for (int s = 1; s < nsplit; ++s) {
            const float4 b = part[(int64_t)s * n4 + i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        logits[i] = a;
    }
}

}  // namespace

// K splits of the split-K router GEMM for this shape (0: not used, the 64 x 128
// kernel runs). Splits fill about one block per CU, whole 64-element steps each.
int router_splits(int64_t T, int H, int E, int* steps_per_split) {
    if (H % SRK != 0 || E % 64 != 0 || T <= 0) return 0;
    const int nk = H / SRK;
    const int64_t tiles = ceil_div(T, SRM) * ceil_div(E, SRN);
    int64_t s = ceil_div(256, tiles);
    if (s > 16) s = 16;
    if (s > nk) s = nk;
    if (s < 1) s = 1;
    const int per = (int)ceil_div(nk, s);
    if (steps_per_split) *steps_per_split = per;
    return (int)ceil_div(nk, per);
}

}  // namespace moe

extern "C" size_t moe_router_workspace_bytes(int64_t T, int32_t H, int32_t E) {
    if (T <= 0 || H <= 0 || E <= 0) return 0;
    const int s = moe::router_splits(T, H, E, nullptr);
    return (size_t)s * (size_t)T * (size_t)E * sizeof(float);
}

extern "C" int moe_router_select(const void* x_bf16, const void* wg_bf16, const float* correction_bias,
                                 int64_t T, int32_t H, int32_t E, int32_t topk, int32_t n_group,
                                 int32_t topk_group, int32_t score_fn, int32_t renormalize,
                                 float routed_scaling_factor, int32_t apply_rsf, float* logits,
                                 int32_t* topk_ids, float* topk_weights, void* workspace,
                                 size_t workspace_bytes, void* stream) {
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
    int per = 0;
    const int nsplit = router_splits(T, H, E, &per);
    if (nsplit > 0) {
        if (!workspace || workspace_bytes < moe_router_workspace_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
        if (!aligned16(workspace)) return MOE_ERR_INVALID_ARG;
        if ((int64_t)SRN * H * 2 >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    }
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    if (nsplit > 0) {
        float* part = (float*)workspace;
        const dim3 grid((unsigned)ceil_div(T, SRM), (unsigned)ceil_div(E, SRN), (unsigned)nsplit);
        hipLaunchKernelGGL(router_splitk_kernel, grid, dim3(kSRThreads), 0, s, (const uint16_t*)x_bf16,
                           (const uint16_t*)wg_bf16, T, H, E, per, part);
        const int64_t n4 = T * (int64_t)E / 4;
        int64_t rb = ceil_div(n4, 256);
        const int64_t cap = (int64_t)device_cu_count() * 8;
        if (rb > cap) rb = cap;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)rb), dim3(256), 0, s, (const float4*)part, n4,
                           nsplit, (float4*)logits);
    } else {
        const dim3 grid((unsigned)ceil_div(T, RBM), (unsigned)ceil_div(E, RBN));
        hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kRThreads), 0, s, (const uint16_t*)x_bf16,
                           (const uint16_t*)wg_bf16, T, H, E, logits);
    }
    const int st = launch_status();
    if (st != MOE_OK) return st;
    return launch_select_experts(logits, correction_bias, T, E, topk, n_group, topk_group, score_fn,
                                 renormalize, routed_scaling_factor, apply_rsf, topk_ids, topk_weights, s,
                                 0, 0.0f);
}
