// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_WAVE 64
#define MOE_E4M3_MAX 448.0f
#define MOE_QB 128  // block / group size of block quantisation

namespace moe {

// ---- host-side launch helpers ------------------------------------------------

static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static inline int launch_status() {
    hipError_t err = hipGetLastError();
    return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int device_cu_count();  // compute units of the current device (cached per device)

// select_experts.hip: argument checks + launch of stage 1 on given logits
int launch_select_experts(const float* logits, const float* correction_bias, int64_t T, int32_t E,
                          int32_t topk, int32_t n_group, int32_t topk_group, int32_t score_fn,
                          int32_t renormalize, float routed_scaling_factor, int32_t apply_rsf,
                          int32_t* topk_ids, float* topk_weights, hipStream_t s, int32_t n_shared,
                          float shared_weight);

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- exact-math helpers (the fp32 operation sequence is part of the contract) --

#pragma clang fp contract(off)

// exp(x) in fp32 with a fixed sequence: clamp to [-80, 80]; n = rint(x*log2 e);
// two-constant Cody-Waite reduction r = x - n*ln2 (one fma each); degree-7
// Taylor polynomial in Horner form (one fma per step); scale by 2^n.
__device__ __forceinline__ float exp_fixed(float x) {
    x = fminf(fmaxf(x, -80.0f), 80.0f);
    const float n = __builtin_rintf(x * 1.44269504088896341f);
    float r = __builtin_fmaf(-n, 0.693145751953125f, x);
    r = __builtin_fmaf(-n, 1.42860682030941723212e-6f, r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// n / d for d in [1, 2^116] and finite n: the reciprocal-and-corrections
// sequence of the compiler's IEEE division without its range scaling
// (v_div_scale / v_div_fmas / v_div_fixup), and the sign of n copied onto the
// result (the corrections turn -0 / d into +0). In that range the scaling is
// the identity unless |n| < 2^-103, so the quotient is the correctly rounded
// one; below, it may differ in the last place of a value under 2^-102 and
// keeps the sign of n.
__device__ __forceinline__ float div_by_ge1(float n, float d) {
    float r = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, r, 1.0f);
    r = __builtin_fmaf(e, r, r);
    float q = n * r;
    float rem = __builtin_fmaf(-d, q, n);
    q = __builtin_fmaf(rem, r, q);
    rem = __builtin_fmaf(-d, q, n);
    return __builtin_copysignf(__builtin_fmaf(rem, r, q), n);
}

// 1 / (1 + exp(-x)): the denominator lies in [1, 1 + e^80], the numerator is 1.
__device__ __forceinline__ float sigmoid_fixed(float x) { return div_by_ge1(1.0f, 1.0f + exp_fixed(-x)); }

// x * sigmoid(x) as x / (1 + exp(-x)).
__device__ __forceinline__ float silu_fixed(float x) { return div_by_ge1(x, 1.0f + exp_fixed(-x)); }

// bf16 <-> fp32 (round to nearest even for finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
// Two fp32 values rounded to nearest even bf16 by one v_cvt_pk_bf16_f32, packed
// (a in the low half); equal to f32_to_bf16_bits for finite values.
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const moe_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, moe_bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Dynamic FP8 scale: s = max(amax,1e-10)/448 (stored), inv = 448/max(amax,1e-10) (applied).
__device__ __forceinline__ void dyn_scale(float amax, float& scale, float& inv) {
    const float a = amax > 1e-10f ? amax : 1e-10f;
    scale = a / MOE_E4M3_MAX;
    inv = MOE_E4M3_MAX / a;
}

// Four fp32 values -> four OCP e4m3 codes packed little-endian, after x*inv and
// saturation to +-448 (the conversion rounds to nearest even).
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv) {
    a = fminf(fmaxf(a * inv, -MOE_E4M3_MAX), MOE_E4M3_MAX);
    b = fminf(fmaxf(b * inv, -MOE_E4M3_MAX), MOE_E4M3_MAX);
    c = fminf(fmaxf(c * inv, -MOE_E4M3_MAX), MOE_E4M3_MAX);
    d = fminf(fmaxf(d * inv, -MOE_E4M3_MAX), MOE_E4M3_MAX);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// ---- wave-level reductions ------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

// max over aligned groups of 8 lanes
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1, MOE_WAVE));
    v = fmaxf(v, __shfl_xor(v, 2, MOE_WAVE));
    v = fmaxf(v, __shfl_xor(v, 4, MOE_WAVE));
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

// inclusive prefix sum across the wave
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, MOE_WAVE);
        if (lane >= o) v += u;
    }
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive prefix sum of one int per thread over the whole block (blockDim.x a
// multiple of 64, at most 1024). `scratch` holds >= 17 ints of LDS. Returns the
// exclusive prefix; *total receives the block sum. Contains __syncthreads().
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = wave_inclusive_scan(v, lane);
    if (lane == 63) scratch[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int w = lane < nw ? scratch[lane] : 0;
        int wi = wave_inclusive_scan(w, lane);
        if (lane < nw) scratch[lane] = wi - w;
        if (lane == nw - 1) scratch[16] = wi;
    }
    __syncthreads();
    int res = scratch[wid] + inc - v;
    if (total) *total = scratch[16];
    __syncthreads();
    return res;
}

// ---- global -> LDS DMA (explicitly waited) ---------------------------------------

// One 16-byte global -> LDS DMA per lane: from base + voff (base wave-uniform
// in SGPRs, voff a per-lane 32-bit offset) to LDS address lds_base + 16 * lane
// (lds_base wave-uniform, in M0). Inline assembly so that the compiler inserts
// no waits of its own around it; every wait on these loads is explicit.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_base)
                 : "memory");
}

// dma16 with the nontemporal hint: for data read once (streamed weights), so
// that it does not displace lines that are read again.
__device__ __forceinline__ void dma16_nt(const uint8_t* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(base), "s"(lds_base)
                 : "memory");
}

// One 4-byte global -> LDS DMA per lane, to LDS address lds_base + 4 * lane.
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(lds_base)
                 : "memory");
}

// A 16-byte store with the nontemporal hint: for output that no later work of the
// same kernel reads (a GEMM's result rows), so that it does not displace operand
// lines from L2.
typedef int moe_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
    const moe_i32x4 w = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    __builtin_nontemporal_store(w, (moe_i32x4*)p);
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left alone
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

}  // namespace moe
