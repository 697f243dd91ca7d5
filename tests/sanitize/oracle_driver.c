/*
 * Runs every entry point of the CPU oracle on small seeded inputs, in every
 * scoring, activation-quantisation and weight-scale mode, with and without a
 * shared expert, for an AddressSanitizer / UndefinedBehaviorSanitizer build
 * (tests/test_oracle_sanitize.py). Test infrastructure only: it includes
 * oracle.c as one translation unit and checks nothing but memory and UB.
 */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint32_t g_rs = 12345u;
static uint32_t rnd(void) { g_rs = g_rs * 1664525u + 1013904223u; return g_rs >> 8; }
static float frand(void) { return (float)(rnd() & 0xFFFF) / 32768.0f - 1.0f; }
static uint8_t e4m3_finite(void) { uint8_t c = (uint8_t)(rnd() & 0xFF); return (c & 0x7F) == 0x7F ? 0x3C : c; }

static void* xalloc(size_t n) { void* p = calloc(n ? n : 1, 1); if (!p) exit(3); return p; }

static int64_t a_scales(int mode, int64_t m_cap, int K) {
    return mode == ACT_PER_TENSOR ? 1 : mode == ACT_PER_TOKEN ? m_cap : m_cap * ((K + QB - 1) / QB);
}
static int64_t b_scales(int mode, int El, int N, int K) {
    return mode == W_PER_EXPERT ? El : mode == W_PER_CHANNEL ? (int64_t)El * N
                                                             : (int64_t)El * ((N + QB - 1) / QB) * ((K + QB - 1) / QB);
}

static int run(int score_fn, int act_quant, int w_quant, int n_shared) {
    const int64_t T = 37;
    const int H = 256, I = 128, E = 16, topk = 4, expert_start = 5, num_routed = 6;
    const int n_group = score_fn == SCORE_SIGMOID ? 4 : 1, topk_group = score_fn == SCORE_SIGMOID ? 2 : 1;
    const int slots = topk + n_shared, El = num_routed + n_shared;
    const int64_t m_cap = T * (slots < El ? slots : El);

    float* logits = xalloc(sizeof(float) * T * E);
    float* bias = xalloc(sizeof(float) * E);
    for (int64_t i = 0; i < T * E; ++i) logits[i] = 3.0f * frand();
    for (int e = 0; e < E; ++e) bias[e] = 0.01f * frand();
    int32_t* ids0 = xalloc(sizeof(int32_t) * T * topk);
    float* w0 = xalloc(sizeof(float) * T * topk);
    if (oracle_select_experts(logits, score_fn == SCORE_SIGMOID ? bias : NULL, T, E, topk, n_group,
                              topk_group, score_fn, 1, 2.5f, 1, ids0, w0)) return 1;
    int32_t* ids = xalloc(sizeof(int32_t) * T * slots);
    float* w = xalloc(sizeof(float) * T * slots);
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < topk; ++j) { ids[t * slots + j] = ids0[t * topk + j]; w[t * slots + j] = w0[t * topk + j]; }
        for (int j = 0; j < n_shared; ++j) { ids[t * slots + topk + j] = E + j; w[t * slots + topk + j] = 1.0f; }
    }
    int32_t* s2d = xalloc(sizeof(int32_t) * T * slots);
    int32_t* d2s = xalloc(sizeof(int32_t) * m_cap);
    int32_t* seg = xalloc(sizeof(int32_t) * (El + 1));
    if (oracle_permute_map(ids, T, slots, expert_start, num_routed, E, n_shared, m_cap, s2d, d2s, seg)) return 2;
    const int64_t M = seg[El];

    uint16_t* x = xalloc(sizeof(uint16_t) * T * H);
    for (int64_t i = 0; i < T * H; ++i) x[i] = oracle_bf16_rne(frand());
    uint8_t* a13 = xalloc(m_cap * H);
    float* sa13 = xalloc(sizeof(float) * a_scales(act_quant, m_cap, H));
    if (oracle_pre_reorder_quant(x, s2d, T, H, slots, act_quant, a13, sa13)) return 3;

    const int N1 = 2 * I;
    uint8_t* w13 = xalloc((size_t)El * N1 * H);
    uint8_t* w2 = xalloc((size_t)El * H * I);
    for (size_t i = 0; i < (size_t)El * N1 * H; ++i) w13[i] = e4m3_finite();
    for (size_t i = 0; i < (size_t)El * H * I; ++i) w2[i] = e4m3_finite();
    const int64_t nb13 = b_scales(w_quant, El, N1, H), nb2 = b_scales(w_quant, El, H, I);
    float* sb13 = xalloc(sizeof(float) * nb13);
    float* sb2 = xalloc(sizeof(float) * nb2);
    for (int64_t i = 0; i < nb13; ++i) sb13[i] = 1e-3f * (1.5f + frand());
    for (int64_t i = 0; i < nb2; ++i) sb2[i] = 1e-3f * (1.5f + frand());

    uint16_t* c13 = xalloc(sizeof(uint16_t) * m_cap * N1);
    if (oracle_grouped_gemm(a13, sa13, act_quant, w13, sb13, w_quant, seg, El, N1, H, c13, 0)) return 4;
    int64_t rows[3] = {0, M > 0 ? M - 1 : 0, M / 2};
    uint16_t* crows = xalloc(sizeof(uint16_t) * 3 * N1);
    if (M > 0 && oracle_grouped_gemm_rows(a13, sa13, act_quant, w13, sb13, w_quant, seg, El, N1, H, rows, 3, crows))
        return 5;

    uint8_t* a2 = xalloc(m_cap * I);
    float* sa2 = xalloc(sizeof(float) * a_scales(act_quant, m_cap, I));
    if (oracle_act_requant(c13, seg, El, I, act_quant, a2, sa2)) return 6;
    uint16_t* c2 = xalloc(sizeof(uint16_t) * m_cap * H);
    if (oracle_grouped_gemm(a2, sa2, act_quant, w2, sb2, w_quant, seg, El, H, I, c2, 0)) return 7;
    uint16_t* out = xalloc(sizeof(uint16_t) * T * H);
    if (oracle_post_reorder(c2, s2d, w, T, H, slots, out)) return 8;
    uint16_t* dense = xalloc(sizeof(uint16_t) * T * H);
    if (oracle_dense_layer_map(x, ids, w, T, H, I, slots, expert_start, num_routed, E, n_shared, act_quant,
                               w13, sb13, w2, sb2, w_quant, dense)) return 9;

    uint16_t* wg = xalloc(sizeof(uint16_t) * E * H);
    for (int64_t i = 0; i < (int64_t)E * H; ++i) wg[i] = oracle_bf16_rne(0.02f * frand());
    float* lg = xalloc(sizeof(float) * T * E);
    if (oracle_router_logits(x, wg, T, H, E, lg)) return 10;

    if (act_quant != ACT_PER_GROUP && w_quant != W_BLOCK) {  /* MXFP4 weights */
        uint8_t* f4 = xalloc((size_t)El * N1 * H / 2);
        uint8_t* e8 = xalloc((size_t)El * N1 * (H / 32));
        for (size_t i = 0; i < (size_t)El * N1 * H / 2; ++i) f4[i] = (uint8_t)rnd();
        for (size_t i = 0; i < (size_t)El * N1 * (H / 32); ++i) e8[i] = (uint8_t)(118 + rnd() % 5);
        uint16_t* c4 = xalloc(sizeof(uint16_t) * m_cap * N1);
        if (oracle_grouped_gemm_mxfp4(a13, sa13, act_quant, f4, e8, sb13, w_quant, seg, El, N1, H, c4)) return 11;
        if (M > 0 && oracle_grouped_gemm_mxfp4_rows(a13, sa13, act_quant, f4, e8, sb13, w_quant, seg, El, N1, H,
                                                    rows, 3, crows)) return 12;
        free(f4); free(e8); free(c4);
    }

    free(logits); free(bias); free(ids0); free(w0); free(ids); free(w); free(s2d); free(d2s); free(seg);
    free(x); free(a13); free(sa13); free(w13); free(w2); free(sb13); free(sb2); free(c13); free(crows);
    free(a2); free(sa2); free(c2); free(out); free(dense); free(wg); free(lg);
    return 0;
}

int main(void) {
    int cases = 0;
    for (int sf = 0; sf < 2; ++sf)
        for (int aq = 0; aq < 3; ++aq)
            for (int wq = 0; wq < 3; ++wq)
                for (int ns = 0; ns < 2; ++ns) {
                    int rc = run(sf, aq, wq, ns);
                    if (rc) { printf("case score=%d act=%d w=%d shared=%d failed: %d\n", sf, aq, wq, ns, rc); return rc; }
                    ++cases;
                }
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3_encode(oracle_e4m3_decode((uint8_t)c));
    for (int n = 0; n < 16; ++n) (void)oracle_e2m1_value((uint8_t)n);
    printf("oracle driver: %d cases ok\n", cases);
    return 0;
}
