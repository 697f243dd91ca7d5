// Stage 3 (and 5): grouped FP8 GEMM over the local experts' row segments on
// CDNA4 MFMA (v_mfma_f32_16x16x128_f8f6f4, OCP e4m3 x e4m3 -> fp32).
//
// Follows "Fix one bug in the grouped-gemm triton kernel" (sglang PR #6772),
// Highlights: without block quantisation the activation scale is read at the
// tile's own rows (m_range_start + offs_am), never at the expert id; and
// "Support token-level quantization for EP MoE" (PR #6782): the launcher
// checks the activation scale's size for its mode.
//
// Design
//   - Persistent grid (a multiple of 8 blocks, about two per CU). Every block
//     derives the tile list on the device from seg_indptr, so the host never
//     learns M and nothing synchronises: a tile is (expert, n-tile, m-tile) in
//     expert-major order with the m-tile fastest, so blocks running together
//     share one expert's B columns and A rows through L2.
//   - XCD-aware: workgroups are dealt to the 8 XCDs round robin, so block b
//     (XCD b % 8) takes tiles from the XCD's own contiguous eighth of the list.
//   - Tile 128 x 128 x 128 (BM x BN x BK), 256 threads = 4 waves in 2 x 2, each
//     wave 64 x 64 = 4 x 4 MFMA 16x16x128 tiles. A and B tiles are staged
//     through LDS with a 16-byte XOR swizzle (chunk c of row r at c ^ (r & 7))
//     so both the row-wise stores and the MFMA operand reads avoid bank
//     conflicts; the next K step's global loads are in flight while the MFMAs
//     of the current one run.
//   - Scales: when neither scale varies along K the fp32 accumulator is
//     multiplied once by sa(row) * sb(e, n) in the epilogue. Otherwise every
//     128-wide K step (exactly one MFMA deep) is accumulated separately and
//     added with its factor sa(row, kb) * sb(e, n, kb).
#include "common.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kMaxLocal = 1024;
constexpr int kBlocksPerCU = 2;

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ v8i lds_operand(const uint8_t* lds, int row, int lane) {
    const int c = (lane >> 4) * 2;
    const uint4 lo = *(const uint4*)(lds + swz(row, c));
    const uint4 hi = *(const uint4*)(lds + swz(row, c + 1));
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

template <bool KDEP>
__global__ __launch_bounds__(kThreads, kBlocksPerCU) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const float* __restrict__ sb, int w_quant,
    const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds_a[BM * BK];
    __shared__ __align__(16) uint8_t lds_b[BN * BK];
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];
    __shared__ float s_sa[BM];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int n_tiles = (N + BN - 1) / BN;
    const int KB = (K + MOE_QB - 1) / MOE_QB;
    const int NB = (N + MOE_QB - 1) / MOE_QB;

    // ---- tile table from seg_indptr (clamped to [0, m_cap], made monotone) ----
    for (int e = tid; e <= num_local; e += kThreads) {
        int64_t v = seg_in[e];
        v = v < 0 ? 0 : (v > m_cap ? m_cap : v);
        s_seg[e] = (int)v;
    }
    __syncthreads();
    const int per = (num_local + kThreads - 1) / kThreads;
    int my_tiles = 0;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < num_local) {
            const int rows = s_seg[e + 1] - s_seg[e];
            my_tiles += rows > 0 ? ((rows + BM - 1) / BM) * n_tiles : 0;
        }
    }
    int total = 0;
    int run = block_exclusive_scan(my_tiles, scan_scratch, &total);
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < num_local) {
            s_tstart[e] = run;
            const int rows = s_seg[e + 1] - s_seg[e];
            run += rows > 0 ? ((rows + BM - 1) / BM) * n_tiles : 0;
        }
    }
    if (tid == 0) s_tstart[num_local] = total;
    __syncthreads();

    // ---- this block's share of the tile list ----
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd_blocks = gridDim.x >> 3;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd;
    const int lt_end = lt_begin + per_xcd < total ? lt_begin + per_xcd : total;

    for (int lt = lt_begin + slot; lt < lt_end; lt += per_xcd_blocks) {
        // expert: largest e with s_tstart[e] <= lt
        int lo = 0, hi = num_local - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tstart[mid] <= lt) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int seg0 = s_seg[e], seg1 = s_seg[e + 1];
        const int mt_e = (seg1 - seg0 + BM - 1) / BM;
        const int idx = lt - s_tstart[e];
        const int nt = idx / mt_e, mt = idx - nt * mt_e;
        const int row0 = seg0 + mt * BM;
        const int row_end = row0 + BM < seg1 ? row0 + BM : seg1;
        const int n0 = nt * BN;

        // global -> register mapping: 1024 16-byte chunks per operand, 4 per
        // thread; thread tid owns row (tid >> 3) + 32 i, 16-byte column (tid & 7).
        const int lr = tid >> 3, lc = (tid & 7) * 16;
        const uint8_t* a_base = A + (int64_t)(row0 + lr) * K + lc;
        const uint8_t* b_base = B + ((int64_t)e * N + n0 + lr) * K + lc;
        const int64_t step32 = (int64_t)32 * K;
        uint4 ra[4], rb[4];
        auto gload = [&](int kk) {
            const bool kin = kk + lc < K;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool aok = kin && row0 + lr + 32 * i < row_end;
                const bool bok = kin && n0 + lr + 32 * i < N;
                ra[i] = aok ? *(const uint4*)(a_base + i * step32 + kk) : make_uint4(0, 0, 0, 0);
                rb[i] = bok ? *(const uint4*)(b_base + i * step32 + kk) : make_uint4(0, 0, 0, 0);
            }
        };

        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        gload(0);
        for (int kk = 0, kb = 0; kk < K; kk += BK, ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *(uint4*)(lds_a + swz(lr + 32 * i, tid & 7)) = ra[i];
                *(uint4*)(lds_b + swz(lr + 32 * i, tid & 7)) = rb[i];
            }
            if (KDEP && act_quant == MOE_ACT_PER_GROUP && tid < BM) {
                // activation scales of this K block for the tile's rows (row-indexed)
                const int r = row0 + tid < row_end ? row0 + tid : row0;
                s_sa[tid] = sa[(int64_t)r * KB + kb];
            }
            __syncthreads();
            if (kk + BK < K) gload(kk + BK);

            v8i af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_operand(lds_a, wm * 64 + i * 16 + (lane & 15), lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = lds_operand(lds_b, wn * 64 + j * 16 + (lane & 15), lane);

            if (!KDEP) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[i], bfr[j], acc[i][j], 0, 0, 0, 0, 0, 0);
            } else {
                const float sbv = w_quant == MOE_W_BLOCK ? sb[((int64_t)e * NB + n0 / MOE_QB) * KB + kb] : 1.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float f[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        f[v] = (act_quant == MOE_ACT_PER_GROUP ? s_sa[wm * 64 + i * 16 + (lane >> 4) * 4 + v] : 1.0f) * sbv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[i], bfr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][v] = acc[i][j][v] + t[v] * f[v];
                    }
                }
            }
            __syncthreads();
        }

        // ---- epilogue: remaining scales, bf16, store rows of this expert only ----
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = row0 + wm * 64 + i * 16 + (lane >> 4) * 4 + v;
                if (r >= row_end) continue;
                float srow = 1.0f;
                if (!(KDEP && act_quant == MOE_ACT_PER_GROUP))
                    srow = act_quant == MOE_ACT_PER_TENSOR ? sa[0] : sa[r];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 64 + j * 16 + (lane & 15);
                    if (n >= N) continue;
                    float scol = 1.0f;
                    if (!(KDEP && w_quant == MOE_W_BLOCK))
                        scol = w_quant == MOE_W_PER_EXPERT ? sb[e] : sb[(int64_t)e * N + n];
                    const float outv = acc[i][j][v] * (srow * scol);
                    C[(int64_t)r * N + n] = (uint16_t)f32_to_bf16_bits(outv);
                }
            }
        }
    }
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_gemm_fp8(const uint8_t* a_q, const float* a_scale, int64_t a_scale_numel,
                                    int32_t act_quant, const uint8_t* b_q, const float* b_scale,
                                    int64_t b_scale_numel, int32_t w_quant,
                                    const int32_t* seg_indptr, int32_t num_local, int64_t m_cap,
                                    int32_t N, int32_t K, void* c_bf16, void* stream) {
    using namespace moe;
    if (num_local < 0 || m_cap < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
    if (act_quant < MOE_ACT_PER_TENSOR || act_quant > MOE_ACT_PER_GROUP) return MOE_ERR_INVALID_ARG;
    if (w_quant < MOE_W_PER_EXPERT || w_quant > MOE_W_BLOCK) return MOE_ERR_INVALID_ARG;
    if (K % 16 != 0 || N % 16 != 0 || num_local > kMaxLocal) return MOE_ERR_UNSUPPORTED;
    if (m_cap > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
    const int64_t KB = ceil_div(K, MOE_QB), NB = ceil_div(N, MOE_QB);
    const int64_t want_a = act_quant == MOE_ACT_PER_TENSOR ? 1 : act_quant == MOE_ACT_PER_TOKEN ? m_cap : m_cap * KB;
    const int64_t want_b = w_quant == MOE_W_PER_EXPERT ? num_local
                         : w_quant == MOE_W_PER_CHANNEL ? (int64_t)num_local * N
                                                        : (int64_t)num_local * NB * KB;
    if (a_scale_numel != want_a || b_scale_numel != want_b) return MOE_ERR_SHAPE;
    if (!seg_indptr) return MOE_ERR_NULL;
    if (num_local == 0 || m_cap == 0) return MOE_OK;  // no rows can exist
    if (!a_q || !a_scale || !b_q || !b_scale || !c_bf16) return MOE_ERR_NULL;
    if (!aligned16(a_q) || !aligned16(b_q) || !aligned16(c_bf16)) return MOE_ERR_INVALID_ARG;

    (void)hipGetLastError();
    const int64_t upper_tiles = (ceil_div(m_cap, BM) + num_local) * ceil_div(N, BN);
    int64_t grid = (int64_t)device_cu_count() * kBlocksPerCU;
    if (grid > ceil_div(upper_tiles, 8) * 8) grid = ceil_div(upper_tiles, 8) * 8;
    if (grid < 8) grid = 8;
    grid = ceil_div(grid, 8) * 8;
    const bool kdep = act_quant == MOE_ACT_PER_GROUP || w_quant == MOE_W_BLOCK;
    hipStream_t s = (hipStream_t)stream;
    if (kdep)
        hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr, num_local,
                           m_cap, N, K, (uint16_t*)c_bf16);
    else
        hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr, num_local,
                           m_cap, N, K, (uint16_t*)c_bf16);
    return launch_status();
}
