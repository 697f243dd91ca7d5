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
//   - Persistent grid (a multiple of 8 blocks, two per CU). Every block derives
//     the tile list on the device from seg_indptr, so the host never learns M
//     and nothing synchronises: a tile is (expert, n-tile, m-tile) in
//     expert-major order with the m-tile fastest, so blocks running together
//     share one expert's B columns and A rows through L2.
//   - XCD-aware: workgroups are dealt to the 8 XCDs round robin, so block b
//     (XCD b % 8) takes tiles from the XCD's own contiguous eighth of the list.
//   - Tile 128 x 128 x 128 (BM x BN x BK), 256 threads = 4 waves in 2 x 2, each
//     wave 64 x 64 = 4 x 4 MFMA 16x16x128 blocks. The MFMA is issued as B x A
//     so that a lane's four accumulator values are four adjacent output columns
//     of one row.
//   - Operands are staged through two LDS buffers: the global loads of K step
//     k+1 are in flight (in registers) while step k's MFMAs run, then written
//     to the other buffer; one barrier per K step. LDS rows are 128 bytes =
//     eight 16-byte chunks, chunk c of row r stored at c ^ perm8(r), which keeps
//     both the row-wise stores and the MFMA operand reads (16 rows x one chunk
//     per 16 lanes) free of bank conflicts on the 64-bank LDS.
//   - Scales: when neither scale varies along K the fp32 accumulator is
//     multiplied once by sa(row) * sb(e, n) in the epilogue. Otherwise every
//     128-wide K step (exactly one MFMA deep) is accumulated separately and
//     added with its factor sa(row, kb) * sb(e, n, kb).
//   - Epilogue: each wave converts its 64 x 64 outputs to bf16 into LDS and
//     writes them back as 16-byte row segments (eight rows of 128 bytes per
//     store instruction).
#include "common.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kMaxLocal = 1024;
constexpr int kBlocksPerCU = 2;
constexpr int kStage = (BM + BN) * BK;  // one LDS buffer: A tile then B tile

// Chunk permutation of row r (a bijection of 0..7 for every r): bits 2..1 are
// r's bits 2..1, bit 0 is r bit 0 ^ r bit 3. Any 8 consecutive rows at one
// chunk hit 8 distinct 16-byte bank groups of a 128-byte window, and any 16
// consecutive rows 16 distinct ones of a 256-byte window.
__device__ __forceinline__ int perm8(int r) { return (r & 6) | ((r ^ (r >> 3)) & 1); }

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ perm8(r)) << 4); }

// MFMA 16x16x128 operand: lane l supplies row (or column) row0 + l % 16 and K
// bytes [32 * (l / 16), +32), i.e. chunks 2*(l/16) and 2*(l/16)+1.
__device__ __forceinline__ v8i lds_operand(const uint8_t* lds, int row, int lane) {
    const int c = (lane >> 4) * 2;
    const uint4 lo = *(const uint4*)(lds + swz(row, c));
    const uint4 hi = *(const uint4*)(lds + swz(row, c + 1));
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

// Epilogue staging: a wave's 64 x 64 bf16 block, rows of 128 bytes, 16-byte
// chunk q of row r at q ^ (r & 7).
__device__ __forceinline__ int ep_off(int r, int q) { return r * 128 + ((q ^ (r & 7)) << 4); }

template <bool KDEP>
__global__ __launch_bounds__(kThreads, kBlocksPerCU) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const float* __restrict__ sb, int w_quant,
    const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds[2 * kStage];
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];
    __shared__ float s_sa[2][BM];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int n_tiles = (N + BN - 1) / BN;
    const int KB = (K + MOE_QB - 1) / MOE_QB;
    const int NB = (N + MOE_QB - 1) / MOE_QB;
    const int nk = (K + BK - 1) / BK;

    // ---- tile table from seg_indptr (clamped to [0, m_cap]) ----
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

    // global -> register mapping: 1024 16-byte chunks per operand, 4 per thread;
    // thread tid owns row (tid >> 3) + 32 i, 16-byte column (tid & 7).
    const int lr = tid >> 3, lc = (tid & 7) * 16;

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
        const bool group_act = KDEP && act_quant == MOE_ACT_PER_GROUP;
        const bool block_w = KDEP && w_quant == MOE_W_BLOCK;

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

        // acc[i][j][v]: row wm*64 + 16 i + lane % 16, column wn*64 + 16 j + 4 (lane / 16) + v
        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        gload(0);
        for (int kb = 0; kb < nk; ++kb) {
            uint8_t* la = lds + (kb & 1) * kStage;
            uint8_t* lb = la + BM * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *(uint4*)(la + swz(lr + 32 * i, tid & 7)) = ra[i];
                *(uint4*)(lb + swz(lr + 32 * i, tid & 7)) = rb[i];
            }
            if (group_act && tid < BM) {
                // activation scales of this K block for the tile's rows (row-indexed)
                const int r = row0 + tid < row_end ? row0 + tid : row0;
                s_sa[kb & 1][tid] = sa[(int64_t)r * KB + kb];
            }
            // One barrier per step: buffer kb & 1 is complete, and every wave has
            // finished reading it two steps ago, before anyone refills it.
            __syncthreads();
            if (kb + 1 < nk) gload((kb + 1) * BK);

            v8i af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_operand(la, wm * 64 + i * 16 + (lane & 15), lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = lds_operand(lb, wn * 64 + j * 16 + (lane & 15), lane);

            if (!KDEP) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bfr[j], af[i], acc[i][j], 0, 0, 0, 0, 0, 0);
            } else {
                const float sbv = block_w ? sb[((int64_t)e * NB + n0 / MOE_QB) * KB + kb] : 1.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float f = (group_act ? s_sa[kb & 1][wm * 64 + i * 16 + (lane & 15)] : 1.0f) * sbv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bfr[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][v] = acc[i][j][v] + t[v] * f;
                    }
                }
            }
        }
        __syncthreads();  // every wave is done with the operand buffers

        // ---- epilogue: remaining scales, bf16 into LDS, 16-byte row stores ----
        uint8_t* ep = lds + wid * (64 * 128);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = i * 16 + (lane & 15);
            const int r = row0 + wm * 64 + rl;
            float srow = 1.0f;
            if (!group_act) srow = act_quant == MOE_ACT_PER_TENSOR ? sa[0] : sa[r < row_end ? r : row0];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cl = j * 16 + (lane >> 4) * 4;
                uint32_t h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float scol = 1.0f;
                    if (!block_w) {
                        const int n = n0 + wn * 64 + cl + v;
                        scol = w_quant == MOE_W_PER_EXPERT ? sb[e] : sb[(int64_t)e * N + (n < N ? n : N - 1)];
                    }
                    h[v] = f32_to_bf16_bits(acc[i][j][v] * (srow * scol));
                }
                *(uint2*)(ep + ep_off(rl, cl >> 3) + (cl & 7) * 2) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
        }
        __syncthreads();  // the staged block is complete (lanes read other lanes' values)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int rl = t * 8 + (lane >> 3), q = lane & 7;
            const int r = row0 + wm * 64 + rl;
            const int n = n0 + wn * 64 + q * 8;
            const uint4 v = *(const uint4*)(ep + ep_off(rl, q));
            if (r < row_end && n < N) *(uint4*)(C + (int64_t)r * N + n) = v;
        }
        __syncthreads();  // the LDS is free for the next tile's operands
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
