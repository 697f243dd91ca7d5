// Stage 1: the fused gate (scoring, grouped top-k, renormalisation, routed
// scaling factor): thirty-two or sixteen lanes per token where the expert count
// allows it, else one wavefront per token.
//
// Follows "[1/2] sgl-kernel: Fuse routed scaling factor into select_experts"
// (sglang PR #8364), Motivation and Modifications: the scaling factor is
// multiplied into the weights inside the gate, during the expert-weight
// normalisation, when the boolean argument asks for it.
#include "common.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;  // one wave per token, 256 threads

// a ranks before b: larger key first, equal keys by lower index
__device__ __forceinline__ bool ranks_before(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Cross-lane moves without LDS: DPP within rows of 16 lanes, and the gfx950
// permlane swaps across rows and halves of the wave.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

// wave-wide maximum, in every lane
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// merge two descending pairs (a1 >= a2, b1 >= b2) into the top two of the four
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
    const float n1 = fmaxf(a1, b1);
    const float n2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
    a1 = n1;
    a2 = n2;
}
template <int CTRL>
__device__ __forceinline__ void top2_step(float& a1, float& a2) {
    top2_merge(a1, a2, dpp<CTRL>(a1), dpp<CTRL>(a2));
}

// Each lane owns EPL consecutive experts: e = lane*EPL + i.
template <int EPL>
__global__ __launch_bounds__(256) void select_experts_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int E, int topk,
    int n_group, int topk_group, int score_fn, int renormalize, float rsf, int apply_rsf,
    int n_shared, float shared_weight, int stride, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
    __shared__ float s_key[kTokensPerBlock][EPL * 64];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + wid;
    const bool active = t < T;  // waves stay for the block barriers below
    const float* l = logits + (active ? t : 0) * E;

    float key[EPL], sc[EPL];
    bool ok[EPL];
    float lmax = -INFINITY;
    // all of the lane's logits and biases are loaded before any is used (indices
    // clamped into the row, values past E masked below): one memory round trip
    float lraw[EPL], braw[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        const int ec = e < E ? e : E - 1;
        lraw[i] = l[ec];
        braw[i] = bias ? bias[ec] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        ok[i] = active && e < E;
        const float lv = ok[i] ? lraw[i] : 0.0f;
        if (score_fn == MOE_SCORE_SIGMOID) {
            sc[i] = sigmoid_fixed(lv);
            key[i] = bias ? sc[i] + (ok[i] ? braw[i] : 0.0f) : sc[i];
        } else {
            sc[i] = lv;
            key[i] = lv;
            if (ok[i]) lmax = fmaxf(lmax, lv);
        }
    }

    // ---- group-limited selection ----
    // Fast path: a group spans LPG = (E / n_group) / EPL lanes, LPG in {1, 2, 4, 8}:
    // the top two biased keys of the group come from a DPP merge over its lanes,
    // and each lane ranks its group against all group scores (readlane).
    const int gsz = n_group > 1 ? E / n_group : E;
    const int lpg = gsz % EPL == 0 ? gsz / EPL : 0;
    if (n_group > 1 && (lpg == 1 || lpg == 2 || lpg == 4 || lpg == 8)) {
        float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) top2_merge(t1, t2, key[i], -INFINITY);
        if (lpg >= 2) top2_step<kDppXor1>(t1, t2);
        if (lpg >= 4) top2_step<kDppXor2>(t1, t2);
        if (lpg >= 8) top2_step<kDppHalfMirror>(t1, t2);
        const float gscore = gsz >= 2 ? t1 + t2 : t1;
        const int g = lane / lpg;
        int rank = 0;
        for (int g2 = 0; g2 < n_group; ++g2) {
            const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gscore), g2 * lpg));
            rank += (o > gscore || (o == gscore && g2 < g)) ? 1 : 0;
        }
        const bool keep = rank < topk_group;
#pragma unroll
        for (int i = 0; i < EPL; ++i) ok[i] = ok[i] && keep;
    } else if (n_group > 1) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) s_key[wid][lane * EPL + i] = key[i];
        __syncthreads();
        const int gs = E / n_group;
        float gscore = -INFINITY;
        if (lane < n_group) {
            float k1 = -INFINITY, k2 = -INFINITY;
            int i1 = 0x7fffffff, i2 = 0x7fffffff;
            for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
                const float v = s_key[wid][e];
                if (ranks_before(v, e, k1, i1)) { k2 = k1; i2 = i1; k1 = v; i1 = e; }
                else if (ranks_before(v, e, k2, i2)) { k2 = v; i2 = e; }
            }
            gscore = gs >= 2 ? k1 + k2 : k1;
        }
        uint64_t keep = 0;
        bool taken_g = false;
        for (int r = 0; r < topk_group; ++r) {
            float bk = (lane < n_group && !taken_g) ? gscore : -INFINITY;
            int bi = (lane < n_group && !taken_g) ? lane : 0x7fffffff;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float ok2 = __shfl_xor(bk, o, MOE_WAVE);
                const int oi = __shfl_xor(bi, o, MOE_WAVE);
                if (ranks_before(ok2, oi, bk, bi)) { bk = ok2; bi = oi; }
            }
            keep |= 1ull << bi;
            if (lane == bi) taken_g = true;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (ok[i] && !((keep >> (e / gs)) & 1ull)) ok[i] = false;
        }
    }

    // ---- top-k over the allowed experts ----
    // Round j: each lane's best allowed key (lowest index among equals), the
    // wave maximum by DPP, and the lowest lane holding it (ballot) owns the
    // winner: larger key first, equal keys by lower expert id.
    int my_id = 0;
    float my_sc = 0.0f;
    for (int j = 0; j < topk; ++j) {
        float lb = -INFINITY, lsc = 0.0f;
        int li = -1;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (ok[i] && (li < 0 || key[i] > lb)) { lb = key[i]; li = i; lsc = sc[i]; }
        const float m = wave_max_dpp(li >= 0 ? lb : -INFINITY);
        const uint64_t owners = __ballot(li >= 0 && lb == m);
        if (owners == 0) break;
        const int owner = __ffsll((unsigned long long)owners) - 1;
        const int wi = __builtin_amdgcn_readlane(li, owner);
        const float wsc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsc), owner));
        if (lane == j) { my_id = owner * EPL + wi; my_sc = wsc; }
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == wi) ok[i] = false;
        }
    }

    // ---- weights ----
    float v = 0.0f;
    float all = 1.0f;
    if (score_fn == MOE_SCORE_SOFTMAX) {
        const float m = wave_max(lmax);
        if (lane < topk) v = exp_fixed(my_sc - m);
        if (!renormalize) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (active && lane * EPL + i < E) part += exp_fixed(sc[i] - m);
            all = wave_sum(part);
        }
    } else if (lane < topk) {
        v = my_sc;
    }
    const float sel = wave_sum(lane < topk ? v : 0.0f);
    float w = v / (renormalize ? sel : all);
    if (apply_rsf) w = w * rsf;
    if (active && lane < topk) {
        ids_out[t * stride + lane] = my_id;
        w_out[t * stride + lane] = w;
    } else if (active && lane < topk + n_shared) {  // shared experts: ids E.., fixed weight
        ids_out[t * stride + lane] = E + (lane - topk);
        w_out[t * stride + lane] = shared_weight;
    }
}

// A row of LPT lanes: maximum / sum over it, in every lane (LPT 16 or 32):
// DPP inside each 16-lane row, then a permlane16 swap between row pairs.
template <int LPT>
__device__ __forceinline__ float row_max(float m) {
    m = fmaxf(m, dpp<kDppXor1>(m));
    m = fmaxf(m, dpp<kDppXor2>(m));
    m = fmaxf(m, dpp<kDppHalfMirror>(m));
    m = fmaxf(m, dpp<kDppMirror>(m));
    if (LPT == 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return m;
}
template <int LPT>
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    if (LPT == 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// LPT lanes per token, 64 / LPT tokens per wave (E = LPT * EPL, EPL in {4, 8,
// 16}): the serial part of the selection (one round per chosen expert) runs
// once for all the wave's tokens, and every cross-lane step stays inside the
// token's lanes (DPP rows, one permlane16 swap for LPT 32). Lane rl = lane %
// LPT of its token owns experts rl * EPL + i. Same per-expert arithmetic and
// ordering rules as select_experts_kernel; a group spans LPG = (E / n_group) /
// EPL lanes (1, 2, 4, 8 or 16) when n_group > 1.
template <int EPL, int SCORE, int LPT>
__global__ __launch_bounds__(256) void select_rows_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int topk,
    int n_group, int topk_group, int renormalize, float rsf, int apply_rsf,
    int n_shared, float shared_weight, int stride, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
    constexpr int E = LPT * EPL;
    constexpr int TPB = 256 / LPT;  // tokens per block
    static_assert(EPL <= 16, "the allowed set is a 16-bit mask per lane");
    const int lane = threadIdx.x & 63, rl = lane & (LPT - 1), rbase = lane & (64 - LPT);
    const int64_t t = (int64_t)blockIdx.x * TPB + (threadIdx.x / LPT);
    const bool active = t < T;
    const float* l = logits + (active ? t : 0) * E + rl * EPL;
    // the bias loads go to the logits row when there is no bias (masked below),
    // so every load of the lane is issued before the first use
    const bool has_bias = SCORE == MOE_SCORE_SIGMOID && bias != nullptr;
    const float* bl = has_bias ? bias + rl * EPL : l;

    float lraw[EPL], braw[EPL];
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
        const float4 v = *(const float4*)(l + i);
        lraw[i] = v.x; lraw[i + 1] = v.y; lraw[i + 2] = v.z; lraw[i + 3] = v.w;
        if (SCORE == MOE_SCORE_SIGMOID) {
            const float4 b = *(const float4*)(bl + i);
            braw[i] = b.x; braw[i + 1] = b.y; braw[i + 2] = b.z; braw[i + 3] = b.w;
        }
    }
    float key[EPL], sc[EPL];
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float lv = active ? lraw[i] : 0.0f;
        if (SCORE == MOE_SCORE_SIGMOID) {
            sc[i] = sigmoid_fixed(lv);
            key[i] = has_bias ? sc[i] + braw[i] : sc[i];
        } else {
            sc[i] = lv;
            key[i] = lv;
            lmax = fmaxf(lmax, lv);
        }
    }
    // bit i of okm: expert rl * EPL + i may still be chosen
    uint32_t okm = active ? (EPL == 32 ? 0xFFFFFFFFu : ((1u << EPL) - 1u)) : 0u;

    if (n_group > 1) {
        const int lpg = (E / n_group) / EPL;
        float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) top2_merge(t1, t2, key[i], -INFINITY);
        if (lpg >= 2) top2_step<kDppXor1>(t1, t2);
        if (lpg >= 4) top2_step<kDppXor2>(t1, t2);
        if (lpg >= 8) top2_step<kDppHalfMirror>(t1, t2);
        if (lpg >= 16) top2_step<kDppMirror>(t1, t2);
        const float gscore = t1 + t2;  // a group holds at least EPL >= 4 experts
        const int g = rl / lpg;
        int rank = 0;
        for (int g2 = 0; g2 < n_group; ++g2) {
            const float o = __shfl(gscore, rbase + g2 * lpg, MOE_WAVE);
            rank += (o > gscore || (o == gscore && g2 < g)) ? 1 : 0;
        }
        if (rank >= topk_group) okm = 0u;
    }

    // round j: the row's best allowed key (larger key, then lower expert id)
    int my_id = 0;
    float my_sc = 0.0f;
    for (int j = 0; j < topk; ++j) {
        float lb = -INFINITY, lsc = 0.0f;
        int li = -1;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const bool take = ((okm >> i) & 1u) && (li < 0 || key[i] > lb);
            lb = take ? key[i] : lb;
            lsc = take ? sc[i] : lsc;
            li = take ? i : li;
        }
        const float m = row_max<LPT>(li >= 0 ? lb : -INFINITY);
        const uint64_t owners = __ballot(li >= 0 && lb == m);
        const uint32_t sub = (uint32_t)(owners >> rbase) & (LPT == 32 ? 0xFFFFFFFFu : 0xFFFFu);
        const int owner = sub ? __builtin_ctz(sub) : 0;
        const int wi = __shfl(li, rbase + owner, MOE_WAVE);
        const float wsc = __shfl(lsc, rbase + owner, MOE_WAVE);
        const bool hit = sub != 0;
        my_id = (hit && rl == j) ? owner * EPL + wi : my_id;
        my_sc = (hit && rl == j) ? wsc : my_sc;
        okm &= (hit && rl == owner) ? ~(1u << wi) : 0xFFFFFFFFu;
    }

    float v = 0.0f, all = 1.0f;
    if (SCORE == MOE_SCORE_SOFTMAX) {
        const float m = row_max<LPT>(lmax);
        if (rl < topk) v = exp_fixed(my_sc - m);
        if (!renormalize) {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (active) part += exp_fixed(sc[i] - m);
            all = row_sum<LPT>(part);
        }
    } else if (rl < topk) {
        v = my_sc;
    }
    const float sel = row_sum<LPT>(rl < topk ? v : 0.0f);
    float w = v / (renormalize ? sel : all);
    if (apply_rsf) w = w * rsf;
    if (active && rl < topk) {
        ids_out[t * stride + rl] = my_id;
        w_out[t * stride + rl] = w;
    } else if (active && rl < topk + n_shared) {
        ids_out[t * stride + rl] = E + (rl - topk);
        w_out[t * stride + rl] = shared_weight;
    }
}

}  // namespace
}  // namespace moe

namespace moe {

// Argument checks and launch of the select kernel (shared by moe_select_experts
// and moe_router_select).
int launch_select_experts(const float* logits, const float* correction_bias, int64_t T, int32_t E,
                          int32_t topk, int32_t n_group, int32_t topk_group, int32_t score_fn,
                          int32_t renormalize, float routed_scaling_factor, int32_t apply_rsf,
                          int32_t* topk_ids, float* topk_weights, hipStream_t s, int32_t n_shared,
                          float shared_weight) {
    if (T < 0 || E <= 0 || topk <= 0 || n_group <= 0 || topk_group <= 0) return MOE_ERR_INVALID_ARG;
    if (n_shared < 0 || topk + n_shared > 64) return n_shared < 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
    if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (E > 512 || topk > 32 || topk > E || n_group > 64) return MOE_ERR_UNSUPPORTED;
    if (E % n_group != 0 || topk_group > n_group) return MOE_ERR_INVALID_ARG;
    if ((int64_t)topk_group * (E / n_group) < topk) return MOE_ERR_INVALID_ARG;
    if (score_fn == MOE_SCORE_SOFTMAX && (correction_bias || n_group > 1)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_weights))
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    // sixteen lanes per token when E = 16 * EPL (EPL 4, 8 or 16), every output
    // slot fits a lane of the row, and a group covers whole lanes
    const int epl16 = E % 16 == 0 ? E / 16 : 0;
    const int gsz = E / n_group;
    const bool rows_ok = (epl16 == 4 || epl16 == 8 || epl16 == 16) && topk + n_shared <= 16 &&
                         (!correction_bias || aligned16(correction_bias)) &&
                         (n_group == 1 || (gsz % epl16 == 0 && 16 % (gsz / epl16) == 0));
    // thirty-two lanes per token for E = 256 (eight experts per lane)
    const bool rows32 = E == 256 && topk + n_shared <= 32 &&
                        (!correction_bias || aligned16(correction_bias)) &&
                        (n_group == 1 || (gsz % 8 == 0 && gsz / 8 <= 16 && 32 % (gsz / 8) == 0));
    if (rows32) {
        const dim3 g32((unsigned)ceil_div(T, 8)), b32(256);
        if (score_fn == MOE_SCORE_SIGMOID)
            hipLaunchKernelGGL((select_rows_kernel<8, MOE_SCORE_SIGMOID, 32>), g32, b32, 0, s, logits, correction_bias,
                               T, topk, n_group, topk_group, renormalize, routed_scaling_factor, apply_rsf,
                               n_shared, shared_weight, topk + n_shared, topk_ids, topk_weights);
        else
            hipLaunchKernelGGL((select_rows_kernel<8, MOE_SCORE_SOFTMAX, 32>), g32, b32, 0, s, logits, correction_bias,
                               T, topk, n_group, topk_group, renormalize, routed_scaling_factor, apply_rsf,
                               n_shared, shared_weight, topk + n_shared, topk_ids, topk_weights);
        return launch_status();
    }
    if (rows_ok) {
        const dim3 g16((unsigned)ceil_div(T, 16)), b16(256);
#define MOE_LAUNCH_ROWS(EPL, SC)                                                                  \
    hipLaunchKernelGGL((select_rows_kernel<EPL, SC, 16>), g16, b16, 0, s, logits, correction_bias, T, topk, \
                       n_group, topk_group, renormalize, routed_scaling_factor, apply_rsf,       \
                       n_shared, shared_weight, topk + n_shared, topk_ids, topk_weights)
        if (score_fn == MOE_SCORE_SIGMOID) {
            if (epl16 == 4) MOE_LAUNCH_ROWS(4, MOE_SCORE_SIGMOID);
            else if (epl16 == 8) MOE_LAUNCH_ROWS(8, MOE_SCORE_SIGMOID);
            else MOE_LAUNCH_ROWS(16, MOE_SCORE_SIGMOID);
        } else {
            if (epl16 == 4) MOE_LAUNCH_ROWS(4, MOE_SCORE_SOFTMAX);
            else if (epl16 == 8) MOE_LAUNCH_ROWS(8, MOE_SCORE_SOFTMAX);
            else MOE_LAUNCH_ROWS(16, MOE_SCORE_SOFTMAX);
        }
#undef MOE_LAUNCH_ROWS
        return launch_status();
    }
    const dim3 grid((unsigned)ceil_div(T, kTokensPerBlock)), block(256);
#define MOE_LAUNCH_SELECT(EPL)                                                                     \
    hipLaunchKernelGGL(select_experts_kernel<EPL>, grid, block, 0, s, logits, correction_bias, T, \
                       E, topk, n_group, topk_group, score_fn, renormalize,                      \
                       routed_scaling_factor, apply_rsf, n_shared, shared_weight, topk + n_shared, \
                       topk_ids, topk_weights)
    if (E <= 64) MOE_LAUNCH_SELECT(1);
    else if (E <= 128) MOE_LAUNCH_SELECT(2);
    else if (E <= 256) MOE_LAUNCH_SELECT(4);
    else MOE_LAUNCH_SELECT(8);
#undef MOE_LAUNCH_SELECT
    return launch_status();
}

}  // namespace moe

extern "C" int moe_select_experts(const float* logits, const float* correction_bias, int64_t T,
                                  int32_t E, int32_t topk, int32_t n_group, int32_t topk_group,
                                  int32_t score_fn, int32_t renormalize,
                                  float routed_scaling_factor, int32_t apply_rsf,
                                  int32_t* topk_ids, float* topk_weights, void* stream) {
    return moe::launch_select_experts(logits, correction_bias, T, E, topk, n_group, topk_group,
                                      score_fn, renormalize, routed_scaling_factor, apply_rsf,
                                      topk_ids, topk_weights, (hipStream_t)stream, 0, 0.0f);
}

extern "C" int moe_select_experts_shared(const float* logits, const float* correction_bias, int64_t T,
                                         int32_t E, int32_t topk, int32_t n_group, int32_t topk_group,
                                         int32_t score_fn, int32_t renormalize,
                                         float routed_scaling_factor, int32_t apply_rsf,
                                         int32_t n_shared, float shared_weight, int32_t* topk_ids,
                                         float* topk_weights, void* stream) {
    return moe::launch_select_experts(logits, correction_bias, T, E, topk, n_group, topk_group,
                                      score_fn, renormalize, routed_scaling_factor, apply_rsf,
                                      topk_ids, topk_weights, (hipStream_t)stream, n_shared,
                                      shared_weight);
}
