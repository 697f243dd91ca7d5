/*
 * libmoe: the expert-parallel FP8 MoE layer's hot path on one MI355X (gfx950).
 *
 * Five stages, each one call, each enqueued on a caller stream:
 *   moe_select_experts     fused gate: scoring, grouped top-k, renormalisation,
 *                          routed scaling factor folded in
 *   moe_pre_reorder_quant  expert-contiguous permutation + dynamic FP8 quant
 *   moe_grouped_gemm_fp8   FP8 GEMM over the local experts' row segments,
 *                          activation scale indexed by row
 *   moe_act_requant        SiLU(gate) * up, then dynamic FP8 requantisation
 *   moe_post_reorder       top-k weighted combine back to token order
 * and extensions:
 *   moe_router_select      router projection (bf16 MFMA) + stage 1
 *   moe_select_experts_shared, moe_pre_reorder_quant_shared
 *                          shared experts fused as extra local experts
 *   moe_grouped_gemm_mxfp4 stage 3 with MXFP4 expert weights
 *
 * Conventions shared by every call
 *   - C linkage; all tensors are device pointers to caller-owned memory,
 *     row-major and densely packed. The library allocates nothing, keeps no
 *     pointer after a call returns, and holds no state between calls.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work and returns; nothing synchronises the host. The number of
 *     local rows M is data dependent and stays on the device in
 *     seg_indptr[num_local].
 *   - Every argument check runs on the host before anything is enqueued; a
 *     rejected call returns a negative moe_status and enqueues nothing. A launch
 *     failure returns MOE_ERR_HIP.
 *   - Device pointers must be 16-byte aligned, and the innermost extents of
 *     bf16/FP8 tensors (H, I, N, K) multiples of 16 (MOE_ERR_UNSUPPORTED otherwise).
 *   - bf16 tensors are passed as `void*` (raw 16-bit patterns). FP8 is OCP
 *     E4M3FN (bias 7, max 448, no infinities) stored as `uint8_t` codes.
 *   - Dynamic activation scales are s = max(amax, 1e-10) / 448 and the codes
 *     are e4m3_rne(clamp(x * (448 / max(amax, 1e-10)), -448, 448)).
 *   - Overlapping calls on one stream are ordered by the stream; calls on
 *     different streams that share buffers race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,         /* a required pointer is NULL */
    MOE_ERR_INVALID_ARG = -2,  /* a count is negative / out of range, or a pointer is misaligned */
    MOE_ERR_SHAPE = -3,        /* a buffer size does not match what the mode needs */
    MOE_ERR_UNSUPPORTED = -4,  /* a combination this library does not implement */
    MOE_ERR_WORKSPACE = -5,    /* workspace missing or smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = -6           /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Activation scale granularity: one scale for the tensor, one per row, or one
 * per row and 128-column group along K. */
typedef enum { MOE_ACT_PER_TENSOR = 0, MOE_ACT_PER_TOKEN = 1, MOE_ACT_PER_GROUP = 2 } moe_act_quant;

/* Weight scale granularity: one per expert, one per output channel (row n of
 * an expert's [N, K] matrix), or one per 128x128 block of [N, K]. */
typedef enum { MOE_W_PER_EXPERT = 0, MOE_W_PER_CHANNEL = 1, MOE_W_BLOCK = 2 } moe_w_quant;

/*
 * Stage 1, the fused gate.
 * Source: "[1/2] sgl-kernel: Fuse routed scaling factor into select_experts"
 * (sglang PR #8364), Motivation and Modifications: the gate takes a boolean
 * that multiplies the routed scaling factor into the expert weights while they
 * are normalised.
 *
 *   logits          fp32 [T, E], router logits.
 *   correction_bias fp32 [E] or NULL; sigmoid scoring only. Steers selection,
 *                   does not enter the weights.
 *   score_fn        MOE_SCORE_SOFTMAX: keys are the logits; weights are the
 *                   softmax probabilities of the selected experts (divided by
 *                   their sum if renormalize). Needs n_group == topk_group == 1
 *                   and correction_bias == NULL.
 *                   MOE_SCORE_SIGMOID: s = 1/(1+exp(-l)), key = s + bias; with
 *                   n_group > 1 the experts form n_group equal groups, a group
 *                   scores the sum of its two largest keys, the topk_group best
 *                   groups are kept and the top-k keys are taken inside them;
 *                   weights are s of the selected experts (divided by their sum
 *                   if renormalize).
 *   apply_rsf       nonzero: weights *= routed_scaling_factor.
 *   topk_ids        int32 [T, topk] out, global expert ids, best first; equal
 *                   keys (and group scores) are ordered by the lower index.
 *   topk_weights    fp32 [T, topk] out.
 * Limits: 1 <= E <= 512, 1 <= topk <= min(E, 32), E % n_group == 0,
 * n_group <= 64, 1 <= topk_group <= n_group, topk_group * E / n_group >= topk.
 */
int moe_select_experts(const float* logits, const float* correction_bias, int64_t T, int32_t E,
                       int32_t topk, int32_t n_group, int32_t topk_group, int32_t score_fn,
                       int32_t renormalize, float routed_scaling_factor, int32_t apply_rsf,
                       int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * Router projection + stage 1 (extension: the gate from hidden states).
 * Source: the fused gate of "[1/2] sgl-kernel: Fuse routed scaling factor into
 * select_experts" (sglang PR #8364), Motivation: the gate scores the router's
 * logits; this call computes those logits first.
 *
 *   logits[t, e] = sum_h x[t, h] * wg[e, h], fp32 accumulation of the bf16
 *   products (summation order of the matrix cores), written to `logits`, then
 *   moe_select_experts on them with the same stage-1 arguments.
 *   x_bf16   bf16 [T, H];  wg_bf16  bf16 [E, H] (one row per expert, the
 *            transpose of the [H, E] projection);  logits  fp32 [T, E] out.
 *   workspace  device scratch of at least moe_router_workspace_bytes(T, H, E)
 *            bytes, 16-byte aligned (split-K partial logits, summed in a fixed
 *            order, so the logits are the same on every call); may be NULL
 *            when that size is 0. Too small: MOE_ERR_WORKSPACE.
 * Limits: H % 8 == 0, E % 4 == 0, and those of moe_select_experts. A stage-1
 * argument error is reported before anything is enqueued.
 */
int moe_router_select(const void* x_bf16, const void* wg_bf16, const float* correction_bias,
                      int64_t T, int32_t H, int32_t E, int32_t topk, int32_t n_group,
                      int32_t topk_group, int32_t score_fn, int32_t renormalize,
                      float routed_scaling_factor, int32_t apply_rsf, float* logits,
                      int32_t* topk_ids, float* topk_weights, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes moe_router_select needs for this shape (0 when it needs none). */
size_t moe_router_workspace_bytes(int64_t T, int32_t H, int32_t E);

/*
 * Shared-expert fusion (extension). The pages note that shared-expert fusion is
 * now allowed together with the fused MoE path ("[1/2] sgl-kernel: Fuse routed
 * scaling factor into select_experts", sglang PR #8364, review summary); the
 * arithmetic is this library's reading: the n_shared shared experts are extra
 * slots every token takes, with ids E.. and weight shared_weight, and they run
 * as local experts num_routed.. inside the same grouped GEMMs (w13 / w2 hold
 * num_routed + n_shared experts, the shared ones last; every expert has the
 * same N and K).
 *
 * moe_select_experts_shared: moe_select_experts, then slots topk..topk+n_shared-1
 *   of each token get id E + s and weight shared_weight. topk_ids and
 *   topk_weights are [T, topk + n_shared]. Limit: topk + n_shared <= 64.
 */
int moe_select_experts_shared(const float* logits, const float* correction_bias, int64_t T,
                              int32_t E, int32_t topk, int32_t n_group, int32_t topk_group,
                              int32_t score_fn, int32_t renormalize, float routed_scaling_factor,
                              int32_t apply_rsf, int32_t n_shared, float shared_weight,
                              int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_pre_reorder_quant_shared: moe_pre_reorder_quant where ids in
 *   [expert_start, expert_start + num_routed) are local experts 0..num_routed-1
 *   and ids in [shared_base, shared_base + n_shared) local experts num_routed..;
 *   seg_indptr has num_routed + n_shared + 1 entries, m_cap >= T * min(topk,
 *   num_routed + n_shared) (topk = slots per token, shared ones included), and
 *   the workspace is moe_workspace_bytes(T, topk, num_routed + n_shared).
 *   The two id ranges must not overlap (MOE_ERR_INVALID_ARG); 0 <= n_shared <= 64.
 */
int moe_pre_reorder_quant_shared(const void* x_bf16, const int32_t* topk_ids, int64_t T, int32_t H,
                                 int32_t topk, int32_t expert_start, int32_t num_routed,
                                 int32_t shared_base, int32_t n_shared, int32_t act_quant,
                                 int64_t m_cap, uint8_t* a_q, float* a_scale, int64_t a_scale_numel,
                                 int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace that moe_pre_reorder_quant and moe_act_requant
 * need for these sizes (the same buffer may serve both calls in turn). */
size_t moe_workspace_bytes(int64_t T, int32_t topk, int32_t num_local);

/*
 * Stage 2, permutation into expert-contiguous rows + dynamic FP8 quantisation.
 * Source: "Support token-level quantization for EP MoE" (sglang PR #6782),
 * change summary of pre_reorder_triton_kernel and EPMoELayer: per-token maxima
 * give per-token scales, which are reordered with the rows through src2dst.
 *
 *   x_bf16      bf16 [T, H] tokens.
 *   topk_ids    int32 [T, topk] from stage 1 (global ids). Pair f = t*topk + j
 *               is local when expert_start <= id < expert_start + num_local.
 *   act_quant   MOE_ACT_PER_TENSOR (one scale over all of x; a_scale[0]),
 *               MOE_ACT_PER_TOKEN (a_scale[row]) or MOE_ACT_PER_GROUP
 *               (a_scale[row * ceil(H/128) + g]).
 *   m_cap       rows allocated in a_q / dst2src / scales; must be at least
 *               T * min(topk, num_local).
 *   a_q         e4m3 [m_cap, H] out. Local pairs of expert e occupy rows
 *               seg_indptr[e] .. seg_indptr[e+1]-1 in increasing f; every
 *               local row of a token holds that token's codes. Rows >= M are
 *               not written.
 *   a_scale     fp32 out, a_scale_numel = 1 | m_cap | m_cap*ceil(H/128).
 *   src2dst     int32 [T*topk] out: row of pair f, or -1 if not local.
 *   dst2src     int32 [m_cap] out: pair of row r for r < M, -1 for r >= M.
 *   seg_indptr  int32 [num_local+1] out: segment starts, seg_indptr[num_local] = M.
 *   workspace   device scratch of at least moe_workspace_bytes(T, topk, num_local).
 * num_local may be 0 (every pair non-local) and T may be 0.
 */
int moe_pre_reorder_quant(const void* x_bf16, const int32_t* topk_ids, int64_t T, int32_t H,
                          int32_t topk, int32_t expert_start, int32_t num_local,
                          int32_t act_quant, int64_t m_cap, uint8_t* a_q, float* a_scale,
                          int64_t a_scale_numel, int32_t* src2dst, int32_t* dst2src,
                          int32_t* seg_indptr, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * moe_pre_reorder_quant without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and checks as
 * moe_pre_reorder_quant; the scratch lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends. The
 * call allocates and frees nothing. Its scratch need is that of
 * moe_workspace_bytes(T, topk, num_local) for this stage; a shape that needs
 * more (about T * topk / 64 * num_local * 8 bytes) returns MOE_ERR_WORKSPACE
 * before anything is enqueued. Calls on one GPU share the array: calls that
 * overlap in time on the same GPU (two streams, two threads) race and give
 * undefined results; calls in stream order are safe.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_pre_reorder_quant_noalloc(const void* x_bf16, const int32_t* topk_ids, int64_t T, int32_t H,
                                  int32_t topk, int32_t expert_start, int32_t num_local,
                                  int32_t act_quant, int64_t m_cap, uint8_t* a_q, float* a_scale,
                                  int64_t a_scale_numel, int32_t* src2dst, int32_t* dst2src,
                                  int32_t* seg_indptr, void* stream);

/*
 * Stage 3 (and 5), the grouped FP8 GEMM over the local experts.
 * Source: "Fix one bug in the grouped-gemm triton kernel" (sglang PR #6772),
 * Highlights: without block quantisation the activation scale is loaded at the
 * tile's rows (m_range_start + offs_am), not at the expert id; "Support
 * token-level quantization for EP MoE" (PR #6782): the launcher checks the
 * scale's shape for the per-token mode and accepts 1-D or 2-D scales.
 *
 * For every local expert e and row r in [seg_indptr[e], seg_indptr[e+1]):
 *   C[r, n] = bf16( sum_kb sa(r, kb) * sb(e, n, kb) * sum_{k in kb} A[r,k] * B[e,n,k] )
 * accumulated in fp32, kb running over 128-wide K blocks when either scale
 * varies along K (a single block otherwise).
 *   a_q         e4m3 [m_cap, K]; rows >= M are ignored.
 *   a_scale     fp32, indexed by ROW: numel 1 (per tensor), m_cap (per token)
 *               or m_cap*ceil(K/128) (per group).
 *   b_q         e4m3 [num_local, N, K] (output x input, K contiguous).
 *   b_scale     fp32, numel num_local (per expert), num_local*N (per channel)
 *               or num_local*ceil(N/128)*ceil(K/128) (block, [e][n/128][k/128]).
 *   seg_indptr  int32 [num_local+1] on the device (from stage 2). Values are
 *               clamped to [0, m_cap] before use.
 *   c_bf16      bf16 [m_cap, N] out; only rows < M are written.
 * A scale count that does not match its mode returns MOE_ERR_SHAPE.
 */
int moe_grouped_gemm_fp8(const uint8_t* a_q, const float* a_scale, int64_t a_scale_numel,
                         int32_t act_quant, const uint8_t* b_q, const float* b_scale,
                         int64_t b_scale_numel, int32_t w_quant, const int32_t* seg_indptr,
                         int32_t num_local, int64_t m_cap, int32_t N, int32_t K, void* c_bf16,
                         void* stream);

/*
 * Stage 3 (and 5) with FP4 expert weights.
 * Source: "[1/2] sgl-kernel: Fuse routed scaling factor into select_experts"
 * (sglang PR #8364), Summary of Changes and Highlights: the layer is run with
 * FP4-quantised expert weights (an FP4 checkpoint in its benchmark commands).
 * The pages do not define the encoding; this call takes OCP MXFP4, the format
 * the gfx950 matrix cores consume natively.
 *
 * For every local expert e and row r in [seg_indptr[e], seg_indptr[e+1]):
 *   C[r, n] = bf16( sa(r) * sb(e, n) * sum_k A[r,k] * e2m1(B[e,n,k]) * 2^(S[e,n,k/32] - 127) )
 * accumulated in fp32.
 *   a_q         e4m3 [m_cap, K]; rows >= M are ignored.
 *   a_scale     fp32, indexed by ROW: numel 1 (per tensor) or m_cap (per token).
 *               Per-group activation scales return MOE_ERR_UNSUPPORTED.
 *   b_fp4       packed E2M1 codes [num_local, N, K/2]: element k of a row is
 *               byte k/2, the low nibble for even k (bit 3 sign, bits 2..1
 *               exponent with bias 1, bit 0 mantissa).
 *   b_e8m0      uint8 E8M0 block scales [num_local, N, K/32], 2^(s - 127);
 *               4-byte aligned.
 *   b_scale     fp32 factor, numel num_local (per expert) or num_local*N (per
 *               channel); MOE_W_BLOCK returns MOE_ERR_UNSUPPORTED.
 *   seg_indptr  int32 [num_local+1] on the device, clamped to [0, m_cap].
 *   c_bf16      bf16 [m_cap, N] out; only rows < M are written.
 * K must be a multiple of 128 and N of 16 (MOE_ERR_UNSUPPORTED otherwise).
 */
int moe_grouped_gemm_mxfp4(const uint8_t* a_q, const float* a_scale, int64_t a_scale_numel,
                           int32_t act_quant, const uint8_t* b_fp4, const uint8_t* b_e8m0,
                           const float* b_scale, int64_t b_scale_numel, int32_t w_quant,
                           const int32_t* seg_indptr, int32_t num_local, int64_t m_cap, int32_t N,
                           int32_t K, void* c_bf16, void* stream);

/*
 * Stage 4, SiLU-and-mul + dynamic FP8 requantisation of the w2 input.
 * Source: "Support token-level quantization for EP MoE" (sglang PR #6782),
 * change summary of layer.py: down_input is produced by the activation in the
 * activation dtype and then quantised per token, which yields w2_input_scale.
 *
 *   gateup_bf16  bf16 [m_cap, 2I]: gate in columns [0, I), up in [I, 2I).
 *   Rows r < M = seg_indptr[num_local]:
 *     h = bf16( SiLU(gate) * up ),  SiLU(g) = g / (1 + exp(-g))
 *   then h is quantised like stage 2 (per tensor over all M*I values, per row,
 *   or per 128-column group) into a_q e4m3 [m_cap, I] and a_scale.
 *   workspace    device scratch of at least moe_workspace_bytes(...).
 */
int moe_act_requant(const void* gateup_bf16, const int32_t* seg_indptr, int32_t num_local,
                    int64_t m_cap, int32_t I, int32_t act_quant, uint8_t* a_q, float* a_scale,
                    int64_t a_scale_numel, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 5, top-k weighted combine back to token order.
 * Source: "[1/2] sgl-kernel: Fuse routed scaling factor into select_experts"
 * (sglang PR #8364), Motivation: moe_sum_reduce is the weighted sum over each
 * token's selected experts (where the scaling factor lives when it is not
 * folded into the gate).
 *
 *   out[t, :] = bf16( sum_j topk_weights[t, j] * down[src2dst[t*topk+j], :] )
 * over slots j with 0 <= src2dst < m_cap, in slot order, fp32; tokens with no
 * local pair get zeros.
 *   down_bf16   bf16 [m_cap, H];  out_bf16  bf16 [T, H] out.
 */
int moe_post_reorder(const void* down_bf16, const int32_t* src2dst, const float* topk_weights,
                     int64_t T, int32_t H, int32_t topk, int64_t m_cap, void* out_bf16,
                     void* stream);

/* Human-readable name of a moe_status value. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
