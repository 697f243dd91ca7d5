/*
 * CPU oracle for the expert-parallel FP8 MoE layer's hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * Plain, slow loops that follow the definitions:
 *   - select_experts: "[1/2] sgl-kernel: Fuse routed scaling factor into
 *     select_experts" (sglang PR #8364), Motivation and Modifications (the
 *     routed scaling factor is multiplied in during the expert-weight
 *     normalisation of the fused gate, behind a boolean flag).
 *   - pre_reorder with per-token dynamic FP8 quantisation: "Support token-level
 *     quantization for EP MoE" (sglang PR #6782), change summary for
 *     pre_reorder_triton_kernel and EPMoELayer (per-token maxima, scales
 *     reordered through src2dst).
 *   - grouped GEMM with scale_a indexed by row: "Fix one bug in the grouped-gemm
 *     triton kernel" (sglang PR #6772), Highlights (m_range_start + offs_am
 *     instead of expert_id, FP8 without block quant).
 *   - activation and per-token requantisation of down_input: PR #6782 change
 *     summary for layer.py (sglang_per_token_quant_fp8 after the activation).
 *   - top-k weighted combine: PR #8364 Motivation (moe_sum_reduce is the
 *     final weighted sum over the selected experts).
 *   - router projection (logits the gate scores): PR #8364 Motivation.
 *   - FP4 expert weights: PR #8364 Summary of Changes, Highlights (the fusion
 *     targets FP4-quantised MoE experts) and its benchmark commands (an FP4
 *     checkpoint). The pages do not define the FP4 encoding; it is read as OCP
 *     MXFP4 (E2M1 elements, one E8M0 scale per 32 elements along K), the
 *     format the gfx950 matrix cores take natively.
 *
 * Precision: the GEMM accumulates in fp32 over dequantised FP8 operands. Every
 * step whose floating-point result decides an integer (expert ids, FP8 codes)
 * is evaluated in fp32 with a fixed operation order, so that the GPU can be
 * compared bit for bit: sigmoid/SiLU use exp_ref (Cody-Waite reduction by ln 2
 * plus a degree-7 Taylor polynomial in Horner form with fused multiply-adds),
 * and quantisation multiplies by the correctly rounded reciprocal 448/amax.
 * Routing weights and the final combine are evaluated in fp64.
 *
 * Compile with -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define E4M3_MAX 448.0f
#define QB 128 /* block / group size for block quantisation */

enum { SCORE_SOFTMAX = 0, SCORE_SIGMOID = 1 };
enum { ACT_PER_TENSOR = 0, ACT_PER_TOKEN = 1, ACT_PER_GROUP = 2 };
enum { W_PER_EXPERT = 0, W_PER_CHANNEL = 1, W_BLOCK = 2 };
enum { ORACLE_FLAG_SCALE_A_BY_EXPERT = 1 }; /* planted defect for mutation tests */

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field
 * 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; no infinities; max 448. */
double oracle_e4m3_value(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

static float g_e4m3[256];   /* decoded codes (NaN for the two NaN codes) */
static int g_tables_ready = 0;

static void init_tables(void) {
    if (g_tables_ready) return;
    for (int c = 0; c < 256; ++c) g_e4m3[c] = (float)oracle_e4m3_value((uint8_t)c);
    g_tables_ready = 1;
}

/* Round an fp32 value to the nearest e4m3 value, ties to the even code, after
 * saturating to +-448. Non-negative codes 0x00..0x7E are increasing in value,
 * so the two neighbours of |v| are found by binary search over them. The sign
 * of v (also of -0 and of values that round to zero) is kept. */
uint8_t oracle_e4m3_encode(float v) {
    init_tables();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a > E4M3_MAX) a = E4M3_MAX;
    int lo = 0, hi = 0x7E;                      /* largest code with value <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_e4m3[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (c < 0x7E && g_e4m3[c] != a) {
        double dlo = (double)a - (double)g_e4m3[c];
        double dhi = (double)g_e4m3[c + 1] - (double)a;
        if (dhi < dlo || (dhi == dlo && ((c + 1) & 1) == 0)) c = c + 1;
    }
    return (uint8_t)(sign | c);
}

float oracle_e4m3_decode(uint8_t code) { init_tables(); return g_e4m3[code]; }

/* fp32 -> bf16, round to nearest even (finite inputs). */
uint16_t oracle_bf16_rne(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp64 -> bf16, round to nearest even, in one rounding: the value is scaled so
 * that bf16's 8 significant bits are the integer part, rounded with rint
 * (round-half-even), scaled back, then stored exactly. */
uint16_t oracle_bf16_rne_f64(double d) {
    if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
    int ex;
    frexp(d, &ex);                          /* |d| = m * 2^ex, 0.5 <= m < 1 */
    if (ex < -125) ex = -125;               /* bf16 subnormals: fixed quantum 2^-133 */
    double q = ldexp(1.0, ex - 8);
    double r = rint(d / q) * q;
    float f = (float)r;                     /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* exp(x) in fp32 with a fixed operation sequence:
 *   x is clamped to [-80, 80] (results stay normal);
 *   n = rint(x * log2(e));
 *   r = x - n*ln2 by a two-constant Cody-Waite reduction, each step one fma;
 *   p = degree-7 Taylor polynomial of e^r in Horner form (one fma per step);
 *   result = p * 2^n (exact scaling). */
float oracle_exp_ref(float x) {
    const float LOG2E = 1.44269504088896341f;
    const float LN2_HI = 0.693145751953125f;          /* 16 significant bits */
    const float LN2_LO = 1.42860682030941723212e-6f;  /* ln2 - LN2_HI */
    if (x < -80.0f) x = -80.0f;
    if (x > 80.0f) x = 80.0f;
    float n = rintf(x * LOG2E);
    float r = fmaf(-n, LN2_HI, x);
    r = fmaf(-n, LN2_LO, r);
    float p = (float)(1.0 / 5040.0);
    p = fmaf(p, r, (float)(1.0 / 720.0));
    p = fmaf(p, r, (float)(1.0 / 120.0));
    p = fmaf(p, r, (float)(1.0 / 24.0));
    p = fmaf(p, r, (float)(1.0 / 6.0));
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* logistic sigmoid 1 / (1 + e^-x) in fp32 (IEEE division). */
float oracle_sigmoid(float x) { return 1.0f / (1.0f + oracle_exp_ref(-x)); }

/* SiLU(g) * u rounded to bf16: g / (1 + e^-g), then times u, then bf16. */
uint16_t oracle_silu_mul_bf16(float g, float u) {
    float s = g / (1.0f + oracle_exp_ref(-g));
    return oracle_bf16_rne(s * u);
}

/* The scalar definitions above over an array (for dense device comparisons):
 * exp_out[i] = exp_ref(x[i]), sig_out[i] = sigmoid(x[i]) and silu_out[i] =
 * x[i] / (1 + exp_ref(-x[i])), the fp32 SiLU before the multiply by up. */
int oracle_math_vec(const float* x, int64_t n, float* exp_out, float* sig_out, float* silu_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        exp_out[i] = oracle_exp_ref(x[i]);
        sig_out[i] = oracle_sigmoid(x[i]);
        silu_out[i] = x[i] / (1.0f + oracle_exp_ref(-x[i]));
    }
    return 0;
}

/* Dynamic FP8 scale of a group of values with maximum magnitude amax:
 * scale = amax'/448 (stored, used to dequantise) and inv = 448/amax' (used to
 * quantise), with amax' = max(amax, 1e-10) so that all-zero rows stay finite. */
static void dyn_scale(float amax, float* scale, float* inv) {
    float a = amax > 1e-10f ? amax : 1e-10f;
    *scale = a / E4M3_MAX;
    *inv = E4M3_MAX / a;
}

static uint8_t quant_one(float x, float inv) {
    float q = x * inv;
    if (q > E4M3_MAX) q = E4M3_MAX;
    if (q < -E4M3_MAX) q = -E4M3_MAX;
    return oracle_e4m3_encode(q);
}

/* ------------------------------------------------------------------------- */
/* (1) select_experts                                                          */
/* ------------------------------------------------------------------------- */

/* a ranks before b: larger key first, equal keys by lower index. */
static int ranks_before(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

/* Fused gate for one batch of tokens.
 *  softmax: selection keys are the logits (softmax is monotone); weights are
 *           the selected softmax probabilities, divided by their sum when
 *           renormalize is set.
 *  sigmoid: s = sigmoid(l); key c = s + bias (the bias only steers selection).
 *           With n_group > 1 experts split into n_group equal groups, each
 *           group is scored by the sum of its two largest keys, the topk_group
 *           best groups are kept, and the top-k keys are taken among their
 *           experts. Weights are the unbiased s, divided by their sum when
 *           renormalize is set.
 *  Ids are written best first (ties to the lower id / lower group). When
 *  apply_rsf is set the weights are multiplied by routed_scaling_factor. */
int oracle_select_experts(const float* logits, const float* bias, int64_t T, int E, int topk,
                          int n_group, int topk_group, int score_fn, int renormalize, float rsf,
                          int apply_rsf, int32_t* ids, float* weights) {
    if (E <= 0 || topk <= 0 || topk > E || n_group <= 0 || E % n_group != 0) return -2;
    if (topk_group <= 0 || topk_group > n_group) return -2;
    if (topk_group * (E / n_group) < topk) return -2;
    if (score_fn == SCORE_SOFTMAX && (bias || n_group > 1)) return -4; /* not defined for softmax */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        float* key = (float*)malloc(sizeof(float) * E);
        float* s = (float*)malloc(sizeof(float) * E);
        char* allowed = (char*)malloc(E);
        char* taken = (char*)malloc(E);
        for (int e = 0; e < E; ++e) {
            if (score_fn == SCORE_SIGMOID) {
                s[e] = oracle_sigmoid(l[e]);
                key[e] = bias ? s[e] + bias[e] : s[e];
            } else {
                s[e] = l[e];
                key[e] = l[e];
            }
            allowed[e] = 1;
            taken[e] = 0;
        }
        if (n_group > 1) {
            int gs = E / n_group;
            float* gscore = (float*)malloc(sizeof(float) * n_group);
            char* gkeep = (char*)calloc(n_group, 1);
            for (int g = 0; g < n_group; ++g) {
                int b1 = -1, b2 = -1;
                for (int e = g * gs; e < (g + 1) * gs; ++e) {
                    if (b1 < 0 || ranks_before(key[e], e, key[b1], b1)) { b2 = b1; b1 = e; }
                    else if (b2 < 0 || ranks_before(key[e], e, key[b2], b2)) { b2 = e; }
                }
                gscore[g] = b2 >= 0 ? key[b1] + key[b2] : key[b1];
            }
            for (int j = 0; j < topk_group; ++j) {
                int best = -1;
                for (int g = 0; g < n_group; ++g)
                    if (!gkeep[g] && (best < 0 || ranks_before(gscore[g], g, gscore[best], best)))
                        best = g;
                gkeep[best] = 1;
            }
            for (int e = 0; e < E; ++e) allowed[e] = gkeep[e / gs];
            free(gscore);
            free(gkeep);
        }
        int32_t* out_id = ids + t * topk;
        for (int j = 0; j < topk; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (allowed[e] && !taken[e] && (best < 0 || ranks_before(key[e], e, key[best], best)))
                    best = e;
            taken[best] = 1;
            out_id[j] = best;
        }
        /* weights in fp64 */
        double v[1024];
        double sel = 0.0, all = 0.0;
        if (score_fn == SCORE_SOFTMAX) {
            double m = l[0];
            for (int e = 1; e < E; ++e) if (l[e] > m) m = l[e];
            for (int e = 0; e < E; ++e) all += exp((double)l[e] - m);
            for (int j = 0; j < topk; ++j) { v[j] = exp((double)l[out_id[j]] - m); sel += v[j]; }
        } else {
            for (int j = 0; j < topk; ++j) { v[j] = (double)s[out_id[j]]; sel += v[j]; }
            all = 1.0;
        }
        double denom = renormalize ? sel : all;
        for (int j = 0; j < topk; ++j) {
            double w = v[j] / denom;
            if (apply_rsf) w *= (double)rsf;
            weights[t * topk + j] = (float)w;
        }
        free(key); free(s); free(allowed); free(taken);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* (2) pre_reorder: permutation and dynamic FP8 quantisation                  */
/* ------------------------------------------------------------------------- */

/* Local expert index of a global expert id for one GPU's share: routed experts
 * [expert_start, expert_start + num_routed) are local 0.., shared experts (ids
 * [shared_base, shared_base + n_shared), appended to every token's slots) are
 * local num_routed.., any other id is not local (-1). Shared experts treated as
 * always-selected extra local experts is this build's reading of the pages'
 * "shared expert fusion" (sglang PR #8364 review summary). */
static int local_index(int id, int expert_start, int num_routed, int shared_base, int n_shared) {
    int r = id - expert_start;
    if (r >= 0 && r < num_routed) return r;
    int q = id - shared_base;
    if (q >= 0 && q < n_shared) return num_routed + q;
    return -1;
}

/* Pairs f = t*topk + slot whose expert is local (expert_start <= id <
 * expert_start + num_local) are laid out expert by expert; inside an expert in
 * increasing f. seg_indptr[e] is the first row of local expert e,
 * seg_indptr[num_local] = M. Non-local pairs get src2dst = -1; rows M..m_cap-1
 * of dst2src are -1. */
int oracle_permute_map(const int32_t* ids, int64_t T, int topk, int expert_start, int num_routed,
                       int shared_base, int n_shared, int64_t m_cap, int32_t* src2dst,
                       int32_t* dst2src, int32_t* seg_indptr) {
    int num_local = num_routed + n_shared;
    int64_t P = T * topk;
    int64_t* cnt = (int64_t*)calloc(num_local + 1, sizeof(int64_t));
    int64_t* fill = (int64_t*)calloc(num_local + 1, sizeof(int64_t));
    for (int64_t f = 0; f < P; ++f) {
        int e = local_index(ids[f], expert_start, num_routed, shared_base, n_shared);
        if (e >= 0) cnt[e]++;
    }
    int64_t run = 0;
    for (int e = 0; e < num_local; ++e) { seg_indptr[e] = (int32_t)run; run += cnt[e]; }
    seg_indptr[num_local] = (int32_t)run;
    if (run > m_cap) { free(cnt); free(fill); return -3; }
    for (int64_t r = 0; r < m_cap; ++r) dst2src[r] = -1;
    for (int64_t f = 0; f < P; ++f) {
        int e = local_index(ids[f], expert_start, num_routed, shared_base, n_shared);
        if (e >= 0) {
            int64_t r = seg_indptr[e] + fill[e]++;
            src2dst[f] = (int32_t)r;
            dst2src[r] = (int32_t)f;
        } else {
            src2dst[f] = -1;
        }
    }
    free(cnt);
    free(fill);
    return 0;
}

int oracle_permute(const int32_t* ids, int64_t T, int topk, int expert_start, int num_local,
                   int64_t m_cap, int32_t* src2dst, int32_t* dst2src, int32_t* seg_indptr) {
    return oracle_permute_map(ids, T, topk, expert_start, num_local, 0, 0, m_cap, src2dst, dst2src,
                              seg_indptr);
}

/* Quantise token rows of x (bf16 [T,H]) into the expert-sorted rows named by
 * src2dst. Modes: one scale for the whole of x (per tensor, a_scale[0]); one
 * per token (a_scale[row]); one per 128-column group (a_scale[row*G + g]).
 * Every local destination row of a token receives the same codes and scales. */
int oracle_pre_reorder_quant(const uint16_t* x, const int32_t* src2dst, int64_t T, int H, int topk,
                             int act_quant, uint8_t* a_q, float* a_scale) {
    int G = (H + QB - 1) / QB;
    float t_scale = 0.0f, t_inv = 0.0f;
    if (act_quant == ACT_PER_TENSOR) {
        float amax = 0.0f;
        for (int64_t i = 0; i < T * (int64_t)H; ++i) {
            float a = fabsf(oracle_bf16_to_f32(x[i]));
            if (a > amax) amax = a;
        }
        dyn_scale(amax, &t_scale, &t_inv);
        a_scale[0] = t_scale;
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int j = 0; j < topk; ++j) any |= src2dst[t * topk + j] >= 0;
        if (!any) continue;
        const uint16_t* xr = x + t * H;
        uint8_t* codes = (uint8_t*)malloc(H);
        float scales[1024];
        if (act_quant == ACT_PER_GROUP) {
            for (int g = 0; g < G; ++g) {
                float amax = 0.0f, sc, inv;
                int k1 = (g + 1) * QB < H ? (g + 1) * QB : H;
                for (int k = g * QB; k < k1; ++k) {
                    float a = fabsf(oracle_bf16_to_f32(xr[k]));
                    if (a > amax) amax = a;
                }
                dyn_scale(amax, &sc, &inv);
                scales[g] = sc;
                for (int k = g * QB; k < k1; ++k) codes[k] = quant_one(oracle_bf16_to_f32(xr[k]), inv);
            }
        } else {
            float sc = t_scale, inv = t_inv;
            if (act_quant == ACT_PER_TOKEN) {
                float amax = 0.0f;
                for (int k = 0; k < H; ++k) {
                    float a = fabsf(oracle_bf16_to_f32(xr[k]));
                    if (a > amax) amax = a;
                }
                dyn_scale(amax, &sc, &inv);
            }
            scales[0] = sc;
            for (int k = 0; k < H; ++k) codes[k] = quant_one(oracle_bf16_to_f32(xr[k]), inv);
        }
        for (int j = 0; j < topk; ++j) {
            int32_t r = src2dst[t * topk + j];
            if (r < 0) continue;
            memcpy(a_q + (int64_t)r * H, codes, H);
            if (act_quant == ACT_PER_TOKEN) a_scale[r] = scales[0];
            if (act_quant == ACT_PER_GROUP)
                for (int g = 0; g < G; ++g) a_scale[(int64_t)r * G + g] = scales[g];
        }
        free(codes);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* (3) grouped GEMM                                                            */
/* ------------------------------------------------------------------------- */

static float a_scale_at(const float* sa, int mode, int64_t row, int kb, int KB) {
    if (mode == ACT_PER_TENSOR) return sa[0];
    if (mode == ACT_PER_TOKEN) return sa[row];
    return sa[row * KB + kb];
}

static float b_scale_at(const float* sb, int mode, int e, int n, int kb, int N, int KB) {
    if (mode == W_PER_EXPERT) return sb[e];
    if (mode == W_PER_CHANNEL) return sb[(int64_t)e * N + n];
    int NB = (N + QB - 1) / QB;
    return sb[((int64_t)e * NB + n / QB) * KB + kb];
}

/* One output row: C[n] = bf16( sum_k Ahat[k] * Bhat[e][n][k] ), fp32, k ascending,
 * with Ahat = fp32(dec(A)*sa) and Bhat = fp32(dec(B)*sb). */
static void gemm_row(const float* ahat, const float* bhat, int N, int K, uint16_t* c) {
    for (int n = 0; n < N; ++n) {
        const float* b = bhat + (int64_t)n * K;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            float p = ahat[k] * b[k];
            acc = acc + p;
        }
        c[n] = oracle_bf16_rne(acc);
    }
}

static void dequant_b(const uint8_t* b_q, const float* b_scale, int w_quant, int e, int N, int K,
                      float* bhat) {
    int KB = (K + QB - 1) / QB;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            bhat[(int64_t)n * K + k] = oracle_e4m3_decode(b_q[((int64_t)e * N + n) * K + k])
                                       * b_scale_at(b_scale, w_quant, e, n, k / QB, N, KB);
}

static void dequant_a_row(const uint8_t* a_q, const float* a_scale, int act_quant, int64_t row,
                          int64_t scale_row, int K, float* ahat) {
    int KB = (K + QB - 1) / QB;
    for (int k = 0; k < K; ++k)
        ahat[k] = oracle_e4m3_decode(a_q[row * K + k]) * a_scale_at(a_scale, act_quant, scale_row, k / QB, KB);
}

/* For each local expert e and each row r in [seg_indptr[e], seg_indptr[e+1]):
 * C[r, :] = A[r, :] x B[e]^T with the activation scale taken at row r (never at
 * e). flags & ORACLE_FLAG_SCALE_A_BY_EXPERT plants the opposite indexing (the
 * defect the row indexing fixes) for mutation tests. */
int oracle_grouped_gemm(const uint8_t* a_q, const float* a_scale, int act_quant, const uint8_t* b_q,
                        const float* b_scale, int w_quant, const int32_t* seg_indptr, int num_local,
                        int N, int K, uint16_t* c, int flags) {
    float* bhat = (float*)malloc(sizeof(float) * (size_t)N * K);
    for (int e = 0; e < num_local; ++e) {
        int64_t r0 = seg_indptr[e], r1 = seg_indptr[e + 1];
        if (r1 <= r0) continue;
        dequant_b(b_q, b_scale, w_quant, e, N, K, bhat);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = r0; r < r1; ++r) {
            float* ahat = (float*)malloc(sizeof(float) * K);
            int64_t srow = (flags & ORACLE_FLAG_SCALE_A_BY_EXPERT) ? e : r;
            dequant_a_row(a_q, a_scale, act_quant, r, srow, K, ahat);
            gemm_row(ahat, bhat, N, K, c + r * N);
            free(ahat);
        }
    }
    free(bhat);
    return 0;
}

/* Selected output rows only (for sampled checks at full size): c_rows[i, :] =
 * C[rows[i], :] of oracle_grouped_gemm. Rows outside every segment give zeros. */
int oracle_grouped_gemm_rows(const uint8_t* a_q, const float* a_scale, int act_quant,
                             const uint8_t* b_q, const float* b_scale, int w_quant,
                             const int32_t* seg_indptr, int num_local, int N, int K,
                             const int64_t* rows, int64_t nrows, uint16_t* c_rows) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        int e = -1;
        for (int q = 0; q < num_local; ++q)
            if (r >= seg_indptr[q] && r < seg_indptr[q + 1]) e = q;
        uint16_t* out = c_rows + i * N;
        if (e < 0) { memset(out, 0, sizeof(uint16_t) * (size_t)N); continue; }
        float* ahat = (float*)malloc(sizeof(float) * K);
        float* bhat = (float*)malloc(sizeof(float) * (size_t)K);
        dequant_a_row(a_q, a_scale, act_quant, r, r, K, ahat);
        int KB = (K + QB - 1) / QB;
        for (int n = 0; n < N; ++n) {
            for (int k = 0; k < K; ++k)
                bhat[k] = oracle_e4m3_decode(b_q[((int64_t)e * N + n) * K + k])
                          * b_scale_at(b_scale, w_quant, e, n, k / QB, N, KB);
            gemm_row(ahat, bhat, 1, K, out + n);
        }
        free(ahat);
        free(bhat);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* (3b) grouped GEMM with MXFP4 weights                                        */
/* ------------------------------------------------------------------------- */

/* OCP Microscaling (MX) FP4 element, E2M1: bit 3 sign, bits 2..1 exponent
 * (bias 1), bit 0 mantissa. Exponent field 0 is subnormal: 0.5 * m. Otherwise
 * 2^(e-1) * (1 + m/2). No NaN or infinity; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(uint8_t nibble) {
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* OCP MX shared scale, E8M0: 2^(s - 127); s = 255 is NaN. */
double oracle_e8m0_value(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* Element k of row n of expert e of packed MXFP4 weights [E, N, K/2]: byte
 * k/2, the low nibble for even k, the high nibble for odd k. */
static uint8_t fp4_code(const uint8_t* b_fp4, int e, int N, int K, int n, int k) {
    uint8_t byte = b_fp4[((int64_t)e * N + n) * (K / 2) + k / 2];
    return (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
}

/* Bhat[n][k] = fp32( fp32(e2m1(code) * 2^(s[n][k/32]-127)) * sb(e, n) ): the
 * block product is exact, the per-expert / per-channel factor rounds once. */
static float fp4_bhat(const uint8_t* b_fp4, const uint8_t* b_e8m0, const float* b_scale, int w_quant,
                      int e, int N, int K, int n, int k) {
    float v = (float)(oracle_e2m1_value(fp4_code(b_fp4, e, N, K, n, k))
                      * oracle_e8m0_value(b_e8m0[((int64_t)e * N + n) * (K / 32) + k / 32]));
    float sb = w_quant == W_PER_EXPERT ? b_scale[e] : b_scale[(int64_t)e * N + n];
    return v * sb;
}

/* Stage 3 with FP4 weights: for each local expert e and row r of its segment,
 * C[r, n] = bf16( sum_k Ahat[r][k] * Bhat[e][n][k] ), fp32, k ascending, with
 * Ahat as in the FP8 GEMM (activation scale at row r) and Bhat decoded from
 * MXFP4 codes with one E8M0 scale per 32 consecutive K elements of a row.
 * Weight factor modes: per expert or per output channel. K % 32 == 0. */
int oracle_grouped_gemm_mxfp4(const uint8_t* a_q, const float* a_scale, int act_quant,
                              const uint8_t* b_fp4, const uint8_t* b_e8m0, const float* b_scale,
                              int w_quant, const int32_t* seg_indptr, int num_local, int N, int K,
                              uint16_t* c) {
    if (K % 32 != 0 || (w_quant != W_PER_EXPERT && w_quant != W_PER_CHANNEL)) return 1;
    float* bhat = (float*)malloc(sizeof(float) * (size_t)N * K);
    for (int e = 0; e < num_local; ++e) {
        int64_t r0 = seg_indptr[e], r1 = seg_indptr[e + 1];
        if (r1 <= r0) continue;
#pragma omp parallel for schedule(static)
        for (int n = 0; n < N; ++n)
            for (int k = 0; k < K; ++k)
                bhat[(int64_t)n * K + k] = fp4_bhat(b_fp4, b_e8m0, b_scale, w_quant, e, N, K, n, k);
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = r0; r < r1; ++r) {
            float* ahat = (float*)malloc(sizeof(float) * K);
            dequant_a_row(a_q, a_scale, act_quant, r, r, K, ahat);
            gemm_row(ahat, bhat, N, K, c + r * N);
            free(ahat);
        }
    }
    free(bhat);
    return 0;
}

/* Selected output rows of oracle_grouped_gemm_mxfp4 (zeros outside every segment). */
int oracle_grouped_gemm_mxfp4_rows(const uint8_t* a_q, const float* a_scale, int act_quant,
                                   const uint8_t* b_fp4, const uint8_t* b_e8m0, const float* b_scale,
                                   int w_quant, const int32_t* seg_indptr, int num_local, int N,
                                   int K, const int64_t* rows, int64_t nrows, uint16_t* c_rows) {
    if (K % 32 != 0 || (w_quant != W_PER_EXPERT && w_quant != W_PER_CHANNEL)) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        int e = -1;
        for (int q = 0; q < num_local; ++q)
            if (r >= seg_indptr[q] && r < seg_indptr[q + 1]) e = q;
        uint16_t* out = c_rows + i * N;
        if (e < 0) { memset(out, 0, sizeof(uint16_t) * (size_t)N); continue; }
        float* ahat = (float*)malloc(sizeof(float) * K);
        float* bhat = (float*)malloc(sizeof(float) * (size_t)K);
        dequant_a_row(a_q, a_scale, act_quant, r, r, K, ahat);
        for (int n = 0; n < N; ++n) {
            for (int k = 0; k < K; ++k) bhat[k] = fp4_bhat(b_fp4, b_e8m0, b_scale, w_quant, e, N, K, n, k);
            gemm_row(ahat, bhat, 1, K, out + n);
        }
        free(ahat);
        free(bhat);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* (4) SiLU-and-mul + dynamic requantisation                                  */
/* ------------------------------------------------------------------------- */

static void act_row(const uint16_t* gu, int I, uint16_t* h) {
    for (int i = 0; i < I; ++i)
        h[i] = oracle_silu_mul_bf16(oracle_bf16_to_f32(gu[i]), oracle_bf16_to_f32(gu[I + i]));
}

static void quant_row_bf16(const uint16_t* h, int K, int act_quant, float t_scale, float t_inv,
                           uint8_t* q, float* scales) {
    if (act_quant == ACT_PER_GROUP) {
        int G = (K + QB - 1) / QB;
        for (int g = 0; g < G; ++g) {
            int k1 = (g + 1) * QB < K ? (g + 1) * QB : K;
            float amax = 0.0f, sc, inv;
            for (int k = g * QB; k < k1; ++k) {
                float a = fabsf(oracle_bf16_to_f32(h[k]));
                if (a > amax) amax = a;
            }
            dyn_scale(amax, &sc, &inv);
            scales[g] = sc;
            for (int k = g * QB; k < k1; ++k) q[k] = quant_one(oracle_bf16_to_f32(h[k]), inv);
        }
        return;
    }
    float sc = t_scale, inv = t_inv;
    if (act_quant == ACT_PER_TOKEN) {
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float a = fabsf(oracle_bf16_to_f32(h[k]));
            if (a > amax) amax = a;
        }
        dyn_scale(amax, &sc, &inv);
        scales[0] = sc;
    }
    for (int k = 0; k < K; ++k) q[k] = quant_one(oracle_bf16_to_f32(h[k]), inv);
}

/* Rows r < M = seg_indptr[num_local] of gateup (bf16 [m_cap, 2I], gate in
 * columns [0, I), up in [I, 2I)): h = bf16(SiLU(gate) * up), then h is
 * quantised like the pre_reorder input (per tensor over all M*I values, per
 * row, or per 128-column group). */
int oracle_act_requant(const uint16_t* gateup, const int32_t* seg_indptr, int num_local, int I,
                       int act_quant, uint8_t* a_q, float* a_scale) {
    int64_t M = seg_indptr[num_local];
    int G = (I + QB - 1) / QB;
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M > 0 ? M : 1) * I);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r) act_row(gateup + r * 2 * (int64_t)I, I, h + r * I);
    float t_scale = 0.0f, t_inv = 0.0f;
    if (act_quant == ACT_PER_TENSOR) {
        float amax = 0.0f;
        for (int64_t i = 0; i < M * (int64_t)I; ++i) {
            float a = fabsf(oracle_bf16_to_f32(h[i]));
            if (a > amax) amax = a;
        }
        dyn_scale(amax, &t_scale, &t_inv);
        a_scale[0] = t_scale;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r) {
        float scales[1024];
        quant_row_bf16(h + r * I, I, act_quant, t_scale, t_inv, a_q + r * I, scales);
        if (act_quant == ACT_PER_TOKEN) a_scale[r] = scales[0];
        if (act_quant == ACT_PER_GROUP)
            for (int g = 0; g < G; ++g) a_scale[r * G + g] = scales[g];
    }
    free(h);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* (5) post_reorder: top-k weighted combine                                   */
/* ------------------------------------------------------------------------- */

/* out[t, :] = bf16( sum over slots j with a local expert of w[t,j] * down[src2dst[t*k+j], :] ),
 * summed in fp64 in slot order; tokens without a local pair get +0. */
int oracle_post_reorder(const uint16_t* down, const int32_t* src2dst, const float* w, int64_t T,
                        int H, int topk, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < topk; ++j) {
                int32_t r = src2dst[t * topk + j];
                if (r < 0) continue;
                acc += (double)w[t * topk + j] * (double)oracle_bf16_to_f32(down[(int64_t)r * H + h]);
            }
            out[t * H + h] = oracle_bf16_rne_f64(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Router projection (the gate's input)                                       */
/* ------------------------------------------------------------------------- */

/* logits[t, e] = fp32( sum_h x[t, h] * wg[e, h] ) with x, wg bf16. Every product
 * of two bf16 values is exact in fp64 and the fp64 sum over h (ascending) is
 * exact to far below fp32 resolution for the sizes here, so this is the
 * correctly rounded fp32 value of the exact dot product, up to fp64 rounding.
 * The pages' fused gate scores these logits ("[1/2] sgl-kernel: Fuse routed
 * scaling factor into select_experts", sglang PR #8364, Motivation). */
int oracle_router_logits(const uint16_t* x, const uint16_t* wg, int64_t T, int H, int E,
                         float* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)oracle_bf16_to_f32(x[t * H + h]) * (double)oracle_bf16_to_f32(wg[(int64_t)e * H + h]);
            logits[t * E + e] = (float)acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Dense per-token layer: no permutation, same per-row arithmetic             */
/* ------------------------------------------------------------------------- */

/* For every token and every slot whose expert is local, run quantise -> w13 ->
 * SiLU-and-mul -> requantise -> w2 on the token's own row, then combine. Used
 * to check the permuted path (segments, src2dst, row-indexed scales). */
int oracle_dense_layer_map(const uint16_t* x, const int32_t* ids, const float* w, int64_t T, int H,
                           int I, int topk, int expert_start, int num_routed, int shared_base,
                           int n_shared, int act_quant, const uint8_t* w13, const float* s13,
                           const uint8_t* w2, const float* s2, int w_quant, uint16_t* out) {
    int N1 = 2 * I;
    int G1 = (H + QB - 1) / QB, G2 = (I + QB - 1) / QB;
    int64_t P = T * topk;
    /* activation quantisation of the input rows */
    uint8_t* xq = (uint8_t*)malloc((size_t)T * H);
    float* xs = (float*)malloc(sizeof(float) * (size_t)T * G1);
    float t_scale = 0.0f, t_inv = 0.0f;
    if (act_quant == ACT_PER_TENSOR) {
        float amax = 0.0f;
        for (int64_t i = 0; i < T * (int64_t)H; ++i) {
            float a = fabsf(oracle_bf16_to_f32(x[i]));
            if (a > amax) amax = a;
        }
        dyn_scale(amax, &t_scale, &t_inv);
    }
    for (int64_t t = 0; t < T; ++t) {
        float scales[1024];
        quant_row_bf16(x + t * H, H, act_quant, t_scale, t_inv, xq + t * H, scales);
        for (int g = 0; g < G1; ++g)
            xs[t * G1 + g] = act_quant == ACT_PER_TENSOR ? t_scale : scales[act_quant == ACT_PER_TOKEN ? 0 : g];
    }
    /* w13 + activation for every local pair */
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)P * I);
    uint16_t* c13 = (uint16_t*)malloc(sizeof(uint16_t) * N1);
    float* ahat = (float*)malloc(sizeof(float) * (H > I ? H : I));
    float* bhat1 = (float*)malloc(sizeof(float) * (size_t)N1 * H);
    float* bhat2 = (float*)malloc(sizeof(float) * (size_t)H * I);
    for (int64_t f = 0; f < P; ++f) {
        int e = local_index(ids[f], expert_start, num_routed, shared_base, n_shared);
        if (e < 0) continue;
        int64_t t = f / topk;
        float sa_row[1024];
        for (int g = 0; g < G1; ++g) sa_row[g] = xs[t * G1 + g];
        for (int k = 0; k < H; ++k)
            ahat[k] = oracle_e4m3_decode(xq[t * H + k]) * sa_row[act_quant == ACT_PER_GROUP ? k / QB : 0];
        dequant_b(w13, s13, w_quant, e, N1, H, bhat1);
        gemm_row(ahat, bhat1, N1, H, c13);
        act_row(c13, I, h + f * I);
    }
    /* requantisation of h */
    float h_scale = 0.0f, h_inv = 0.0f;
    if (act_quant == ACT_PER_TENSOR) {
        float amax = 0.0f;
        for (int64_t f = 0; f < P; ++f) {
            int e = local_index(ids[f], expert_start, num_routed, shared_base, n_shared);
            if (e < 0) continue;
            for (int i = 0; i < I; ++i) {
                float a = fabsf(oracle_bf16_to_f32(h[f * I + i]));
                if (a > amax) amax = a;
            }
        }
        dyn_scale(amax, &h_scale, &h_inv);
    }
    uint8_t* hq = (uint8_t*)malloc(I);
    uint16_t* c2 = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)P * H);
    for (int64_t f = 0; f < P; ++f) {
        int e = local_index(ids[f], expert_start, num_routed, shared_base, n_shared);
        if (e < 0) continue;
        float scales[1024];
        quant_row_bf16(h + f * I, I, act_quant, h_scale, h_inv, hq, scales);
        for (int k = 0; k < I; ++k) {
            float sa = act_quant == ACT_PER_TENSOR ? h_scale : scales[act_quant == ACT_PER_TOKEN ? 0 : k / QB];
            ahat[k] = oracle_e4m3_decode(hq[k]) * sa;
        }
        dequant_b(w2, s2, w_quant, e, H, I, bhat2);
        gemm_row(ahat, bhat2, H, I, c2 + f * H);
    }
    /* combine in slot order, fp64 */
    for (int64_t t = 0; t < T; ++t)
        for (int hh = 0; hh < H; ++hh) {
            double acc = 0.0;
            for (int j = 0; j < topk; ++j) {
                int64_t f = t * topk + j;
                if (local_index(ids[f], expert_start, num_routed, shared_base, n_shared) < 0) continue;
                acc += (double)w[f] * (double)oracle_bf16_to_f32(c2[f * H + hh]);
            }
            out[t * H + hh] = oracle_bf16_rne_f64(acc);
        }
    (void)G2;
    free(xq); free(xs); free(h); free(c13); free(ahat); free(bhat1); free(bhat2); free(hq); free(c2);
    return 0;
}

int oracle_dense_layer(const uint16_t* x, const int32_t* ids, const float* w, int64_t T, int H,
                       int I, int topk, int expert_start, int num_local, int act_quant,
                       const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                       int w_quant, uint16_t* out) {
    return oracle_dense_layer_map(x, ids, w, T, H, I, topk, expert_start, num_local, 0, 0, act_quant,
                                  w13, s13, w2, s2, w_quant, out);
}

/* ------------------------------------------------------------------------- */

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
