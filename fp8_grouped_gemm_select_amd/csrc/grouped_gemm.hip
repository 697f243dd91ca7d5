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
//   Two kernels share the tile schedule: a persistent grid in which every block
//   derives the tile list on the device from seg_indptr (the host never learns
//   M and nothing synchronises). A tile is (expert, n-tile, m-tile) in
//   expert-major order with the m-tile fastest, so blocks running together
//   share one expert's B columns and A rows through L2. Workgroups are dealt to
//   the 8 XCDs round robin, so block b (XCD b % 8) takes tiles from its XCD's
//   own contiguous eighth of the list.
//
//   grouped_gemm_dma_kernel (K % 128 == 0, every workload here): 128 x 256
//   tiles, one 512-thread block per CU, operands straight from memory into a
//   three-stage LDS ring by global_load_lds_dwordx4; see its own comment.
//
//   grouped_gemm_kernel (any K % 16 == 0): 128 x 128 x 128 tiles, two
//   256-thread blocks per CU; loads staged through registers into two LDS
//   buffers (step k+1 in flight while step k's MFMAs run), one barrier per K
//   step, zero fill past K.
//
//   Both: waves own 64 x 64 outputs = 4 x 4 MFMA 16x16x128 blocks, issued as
//   B x A so that a lane's four accumulator values are four adjacent output
//   columns of one row. LDS rows are 128 bytes = eight 16-byte chunks, chunk c
//   of row r stored at c ^ perm8(r), which keeps the row-wise fills and the
//   MFMA operand reads (16 rows x one chunk per 16 lanes) free of bank
//   conflicts on the 64-bank LDS. Scales: when neither scale varies along K the
//   fp32 accumulator is multiplied once by sa(row) * sb(e, n) in the epilogue;
//   otherwise every 128-wide K step (exactly one MFMA deep) is accumulated
//   separately and added with its factor sa(row, kb) * sb(e, n, kb). Epilogue:
//   each wave converts its 64 x 64 outputs to bf16 into LDS and writes them
//   back as 16-byte row segments (eight rows of 128 bytes per store), with the
//   nontemporal hint: the result rows are not read again by the kernel, and
//   kept out of L2 they leave it to the operand lines (the block-scaled
//   workload's GEMMs 2-5 % faster, and the combine after them, which then
//   finds no dirty result lines to write back, 14 %).
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

// The e4m3 operand of the scaled MFMA with an E2M1 first operand: the hardware
// pairs the e4m3 lane's low 16 bytes with K [16 (l/16), +16) and its high 16
// bytes with K [64 + 16 (l/16), +16) of the E2M1 operand, whose lane l holds
// the 32 elements of K block l/16 (measured on gfx950). So lane l reads chunks
// l/16 and l/16 + 4 of the row.
__device__ __forceinline__ v8i lds_operand_x4(const uint8_t* lds, int row, int lane) {
    const int c = lane >> 4;
    const uint4 lo = *(const uint4*)(lds + swz(row, c));
    const uint4 hi = *(const uint4*)(lds + swz(row, c + 4));
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

// Epilogue staging: a wave's 64 x 64 bf16 block, rows of 128 bytes, 16-byte
// chunk q of row r at q ^ (r & 7).
__device__ __forceinline__ int ep_off(int r, int q) { return r * 128 + ((q ^ (r & 7)) << 4); }

// Tile table in LDS from seg_indptr (entries clamped to [0, m_cap]): s_seg[e]
// = first row of expert e, s_tstart[e] = index of its first tile in the list
// (experts in order, each with ceil(rows / TM) * ceil(N / TN) tiles). Returns the
// number of tiles. All threads of the block take part.
template <int TM, int TN>
__device__ int build_tile_table(const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N,
                                int* s_seg, int* s_tstart, int* scan_scratch) {
    const int tid = threadIdx.x, nthreads = blockDim.x;
    const int n_tiles = (N + TN - 1) / TN;
    for (int e = tid; e <= num_local; e += nthreads) {
        int64_t v = seg_in[e];
        v = v < 0 ? 0 : (v > m_cap ? m_cap : v);
        s_seg[e] = (int)v;
    }
    __syncthreads();
    const int per = (num_local + nthreads - 1) / nthreads;
    int my_tiles = 0;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < num_local) {
            const int rows = s_seg[e + 1] - s_seg[e];
            my_tiles += rows > 0 ? ((rows + TM - 1) / TM) * n_tiles : 0;
        }
    }
    int total = 0;
    int run = block_exclusive_scan(my_tiles, scan_scratch, &total);
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < num_local) {
            s_tstart[e] = run;
            const int rows = s_seg[e + 1] - s_seg[e];
            run += rows > 0 ? ((rows + TM - 1) / TM) * n_tiles : 0;
        }
    }
    if (tid == 0) s_tstart[num_local] = total;
    __syncthreads();
    return total;
}

// Tile lt of the list: expert e (largest e with s_tstart[e] <= lt), its first
// row row0 and row end, and the first output column n0.
struct TileCoord {
    int e, row0, row_end, n0;
};
template <int TM, int TN>
__device__ __forceinline__ TileCoord tile_coord(int lt, const int* s_seg, const int* s_tstart, int num_local) {
    int lo = 0, hi = num_local - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tstart[mid] <= lt) lo = mid; else hi = mid - 1;
    }
    TileCoord t;
    t.e = lo;
    const int seg0 = s_seg[lo], seg1 = s_seg[lo + 1];
    const int mt_e = (seg1 - seg0 + TM - 1) / TM;
    const int idx = lt - s_tstart[lo];
    const int nt = idx / mt_e, mt = idx - nt * mt_e;
    t.row0 = seg0 + mt * TM;
    t.row_end = t.row0 + TM < seg1 ? t.row0 + TM : seg1;
    t.n0 = nt * TN;
    return t;
}

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
    const int KB = (K + MOE_QB - 1) / MOE_QB;
    const int NB = (N + MOE_QB - 1) / MOE_QB;
    const int nk = (K + BK - 1) / BK;

    const int total = build_tile_table<BM, BN>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);

    // ---- this block's share of the tile list ----
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd_blocks = gridDim.x >> 3;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd;
    const int lt_end = lt_begin + per_xcd < total ? lt_begin + per_xcd : total;

    // global -> register mapping: 1024 16-byte chunks per operand, 4 per thread;
    // thread tid owns row (tid >> 3) + 32 i, 16-byte column (tid & 7).
    const int lr = tid >> 3, lc = (tid & 7) * 16;

    for (int lt = lt_begin + slot; lt < lt_end; lt += per_xcd_blocks) {
        const TileCoord tc = tile_coord<BM, BN>(lt, s_seg, s_tstart, num_local);
        const int e = tc.e, row0 = tc.row0, row_end = tc.row_end, n0 = tc.n0;
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
                        for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(t[v], f, acc[i][j][v]);
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
            if (r < row_end && n < N) store16_nt(C + (int64_t)r * N + n, v);
        }
        __syncthreads();  // the LDS is free for the next tile's operands
    }
}


// ---- large-tile kernel: 128 x 256 tiles, 8 waves, LDS-DMA into a 3-stage ring ----
//
// One 512-thread block per CU (two waves per SIMD). Waves in 2 (M) x 4 (N),
// each owns 64 x 64 outputs (4 x 4 MFMA 16x16x128). Operands go from memory to
// LDS with global_load_lds_dwordx4 (no register staging): a stage holds the A
// tile (128 rows) and the B tile (256 rows) of one 128-byte K step, in the same
// perm8-swizzled row layout as above. Each wave waits only for its own loads
// of the step it is about to read, then one barrier per step publishes the
// stage. Requires K % 128 == 0 (every stage is whole; no zero fill). Rows past
// the valid range re-read the last valid row, so every wave issues the same
// loads every step.
//
// Plain FP8 path (scales constant along K): the operands of step k+1 are read
// from LDS into a second register set while step k's MFMAs run (one operand
// read per two MFMAs), and the six DMA instructions of step k+3 go out one per
// MFMA pair into the slot step k has just left. After the barrier of a step
// the matrix core has its operands at once; the loads no longer queue behind
// one another at the end of the step. The tile's epilogue scales (128 row and
// 256 column values) arrive in LDS by 4-byte DMA with its first step, so no
// registers hold them during the K loop. Other paths (K-dependent scales,
// FP4 weights): operands read after the barrier, DMA of step k+2 issued
// before the reads.
constexpr int DBM = 128, DBN = 256, DBK = 128;
constexpr int kDThreads = 512;
constexpr int kDStages = 3;
constexpr int kDStageA = DBM * DBK;             // 16 KB
constexpr int kDStage = (DBM + DBN) * DBK;      // 48 KB
constexpr int kDmaA = DBM * DBK / 1024 / 8;     // 1 KB DMA instructions per wave per stage: 2
constexpr int kDmaB = DBN * DBK / 1024 / 8;     // 4
constexpr int kDma = kDmaA + kDmaB;             // 6
// MXFP4 weights: a stage's B tile is 256 rows of 64 bytes (128 E2M1 codes)
// followed by the rows' E8M0 scales of the step (one dword per row).
constexpr int kDmaB4 = DBN * DBK / 2 / 1024 / 8;  // 2
constexpr int kDStageS4 = kDStageA + DBN * DBK / 2;  // scale dwords at +32 KB
constexpr int kDma4 = kDmaA + kDmaB4 + 1;         // 5 (A, B, scales)

// Chunk position of 16-byte chunk c of a 64-byte B row r (FP4): c ^ ((r >> 2) & 3).
// Sixteen consecutive rows read at one chunk hit sixteen distinct 16-byte bank
// groups of the 64-bank LDS.
__device__ __forceinline__ int fp4_pos(int r, int c) { return c ^ ((r >> 2) & 3); }

// Per-tile state of the large-tile kernel: coordinates and per-lane DMA offsets.
struct DTile {
    int e, row0, row_end, n0, a_rows, b_rows, sa_row, nb_w;
    const uint8_t* a_g;
    const uint8_t* b_g;
    const uint8_t* s_g;  // FP4: E8M0 scales of the tile's first weight row
    uint32_t a_off[kDmaA], b_off[kDmaB], s_off;
};

// FP4: B holds MXFP4 weights (packed E2M1 [E, N, K/2], element k in byte k/2,
// low nibble for even k) with E8M0 scales Be8 [E, N, K/32]; the MFMA takes the
// codes as its first operand (format E2M1) with the row's scale byte of the
// lane's 32-element block, the activations as e4m3 with scale 2^0.
template <bool KDEP, bool FP4>
__global__ __launch_bounds__(kDThreads, 1) void grouped_gemm_dma_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Be8, const float* __restrict__ sb,
    int w_quant, const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    static_assert(!(KDEP && FP4), "FP4 weights take no K-dependent scales");
    constexpr int kDmaN = FP4 ? kDma4 : kDma;
    __shared__ __align__(16) uint8_t lds[kDStages * kDStage];
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];
    __shared__ float s_sa[kDStages][DBM];
    // epilogue scales of a tile on the register-prefetch path: sa of its 128
    // rows, then sb of its 256 columns; two buffers, tiles alternate
    __shared__ __align__(16) float s_scale[2][DBM + DBN];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 2, wn = wid & 3;
    const int KB = K / MOE_QB;
    const int NB = (N + MOE_QB - 1) / MOE_QB;
    const int nk = K / DBK;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)lds;
    const bool group_act = KDEP && act_quant == MOE_ACT_PER_GROUP;
    const bool block_w = KDEP && w_quant == MOE_W_BLOCK;

    const int total = build_tile_table<DBM, DBN>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);

    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd_blocks = gridDim.x >> 3;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd;
    const int lt_end = lt_begin + per_xcd < total ? lt_begin + per_xcd : total;

    auto setup = [&](int lt) {
        const TileCoord tc = tile_coord<DBM, DBN>(lt, s_seg, s_tstart, num_local);
        DTile t;
        t.e = tc.e;
        t.row0 = tc.row0;
        t.row_end = tc.row_end;
        t.n0 = tc.n0;
        t.a_rows = tc.row_end - tc.row0;
        t.b_rows = N - tc.n0 < DBN ? N - tc.n0 : DBN;
        // the weight-scale block of this wave's 64 columns (clamped: in a partial
        // tile a wave's columns can start past N; its outputs are not stored)
        t.nb_w = (t.n0 + wn * 64) / MOE_QB < NB ? (t.n0 + wn * 64) / MOE_QB : NB - 1;
        // per-lane DMA offsets: instruction i of this wave fills LDS rows
        // 8 * (wave's first block + i) + lane / 8, chunk position lane % 8, which
        // holds global chunk (lane % 8) ^ perm8(row)
#pragma unroll
        for (int i = 0; i < kDmaA; ++i) {
            const int r = (wid * kDmaA + i) * 8 + (lane >> 3);
            const int g = r < t.a_rows ? r : t.a_rows - 1;
            t.a_off[i] = (uint32_t)g * (uint32_t)K + (uint32_t)((((lane & 7) ^ perm8(r)) << 4));
        }
        if (FP4) {
            // instruction i of wave w fills 64-byte rows 16 (2 w + i) + lane / 4 at
            // position lane % 4; the scale DMA of wave w loads the dwords of rows
            // 64 (w % 4) + lane (waves w and w + 4 write the same values)
#pragma unroll
            for (int i = 0; i < kDmaB4; ++i) {
                const int r = (wid * kDmaB4 + i) * 16 + (lane >> 2);
                const int g = r < t.b_rows ? r : t.b_rows - 1;
                t.b_off[i] = (uint32_t)g * (uint32_t)(K / 2) + (uint32_t)(fp4_pos(r, lane & 3) << 4);
            }
            const int rs = (wid & 3) * 64 + lane;
            t.s_off = (uint32_t)(rs < t.b_rows ? rs : t.b_rows - 1) * (uint32_t)(K / 32);
            t.b_g = B + ((int64_t)t.e * N + t.n0) * (K / 2);
            t.s_g = Be8 + ((int64_t)t.e * N + t.n0) * (K / 32);
        } else {
#pragma unroll
            for (int i = 0; i < kDmaB; ++i) {
                const int r = (wid * kDmaB + i) * 8 + (lane >> 3);
                const int g = r < t.b_rows ? r : t.b_rows - 1;
                t.b_off[i] = (uint32_t)g * (uint32_t)K + (uint32_t)((((lane & 7) ^ perm8(r)) << 4));
            }
            t.b_g = B + ((int64_t)t.e * N + t.n0) * K;
            t.s_g = nullptr;
            t.s_off = 0;
        }
        t.a_g = A + (int64_t)t.row0 * K;
        t.sa_row = t.row0 + ((tid & (DBM - 1)) < t.a_rows ? (tid & (DBM - 1)) : t.a_rows - 1);
        return t;
    };
    auto issue = [&](const DTile& t, int k) {  // DMA of K step k into stage k % 3
        const uint32_t st = lds0 + (uint32_t)((k % kDStages) * kDStage);
        const uint8_t* ab = uniform_ptr(t.a_g + k * DBK);
        const uint32_t la = __builtin_amdgcn_readfirstlane(st + wid * kDmaA * 1024);
#pragma unroll
        for (int i = 0; i < kDmaA; ++i) dma16(ab, t.a_off[i], la + i * 1024);
        if (FP4) {
            const uint8_t* bb = uniform_ptr(t.b_g + k * (DBK / 2));
            const uint32_t lb = __builtin_amdgcn_readfirstlane(st + kDStageA + wid * kDmaB4 * 1024);
#pragma unroll
            for (int i = 0; i < kDmaB4; ++i) dma16(bb, t.b_off[i], lb + i * 1024);
            const uint8_t* sbp = uniform_ptr(t.s_g + k * (DBK / 32));
            dma4(sbp, t.s_off, __builtin_amdgcn_readfirstlane(st + kDStageS4 + (wid & 3) * 256));
        } else {
            const uint8_t* bb = uniform_ptr(t.b_g + k * DBK);
            const uint32_t lb = __builtin_amdgcn_readfirstlane(st + kDStageA + wid * kDmaB * 1024);
#pragma unroll
            for (int i = 0; i < kDmaB; ++i) dma16(bb, t.b_off[i], lb + i * 1024);
        }
    };

    // Epilogue scales of tile t into s_scale[p] by 4-byte DMA (plain FP8 path):
    // waves 0-1 the rows' sa, waves 2-5 the columns' sb (indices clamped).
    const uint32_t lds_scale = (uint32_t)(uintptr_t)(const void*)&s_scale[0][0];
    auto issue_scales = [&](const DTile& t, int p) {
        if (wid < 2) {
            const int r = wid * 64 + lane;
            const int g = t.row0 + (r < t.a_rows ? r : t.a_rows - 1);
            const uint32_t off = act_quant == MOE_ACT_PER_TENSOR ? 0u : (uint32_t)g * 4u;
            dma4((const uint8_t*)sa, off, __builtin_amdgcn_readfirstlane(lds_scale + (uint32_t)(p * (DBM + DBN) + wid * 64) * 4u));
        } else if (wid < 6) {
            const int c = (wid - 2) * 64 + lane;
            const int n = t.n0 + c < N ? t.n0 + c : N - 1;
            const uint32_t off = w_quant == MOE_W_PER_EXPERT ? (uint32_t)t.e * 4u : (uint32_t)((int64_t)t.e * N + n) * 4u;
            dma4((const uint8_t*)sb, off, __builtin_amdgcn_readfirstlane(lds_scale + (uint32_t)(p * (DBM + DBN) + DBM + c - lane) * 4u));
        }
    };
    int par = 0;  // s_scale buffer of the current tile

    int lt = lt_begin + slot;
    if (lt >= lt_end) return;  // the whole block has no tile

    // Issue order: [activation group scales of step j+1] [DMA of step j+2] per
    // step j, after the first tile's [scales 0] [DMA 0] [DMA 1]; a following
    // tile's [scales 0] [DMA 0] [DMA 1] go out before the previous tile's
    // epilogue (whose stores come after them). At step k the wave needs DMA(k)
    // and the scales of step k; at most DMA(k+1) and epilogue stores were
    // issued after them, so vmcnt(kDma) suffices while k + 1 < nk (it may also
    // wait for some of those stores, never for less than it needs).
    DTile cur = setup(lt);
    float q = 0.f;
    if (group_act) q = sa[(int64_t)cur.sa_row * KB];
    if constexpr (!FP4 && !KDEP) issue_scales(cur, par);
    issue(cur, 0);
    if (nk > 1) issue(cur, 1);

    while (true) {
        // epilogue scales of this tile (in flight during the K loop, except on the
        // register-prefetch path, which needs the registers)
        float srow[4], scol[4][4];
        auto load_scales = [&]() {
            if constexpr (!FP4 && !KDEP) {
#pragma unroll
                for (int i = 0; i < 4; ++i) srow[i] = s_scale[par][wm * 64 + i * 16 + (lane & 15)];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 v4 = *(const float4*)&s_scale[par][DBM + wn * 64 + j * 16 + (lane >> 4) * 4];
                    scol[j][0] = v4.x; scol[j][1] = v4.y; scol[j][2] = v4.z; scol[j][3] = v4.w;
                }
                return;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = cur.row0 + wm * 64 + i * 16 + (lane & 15);
            srow[i] = group_act ? 1.0f : (act_quant == MOE_ACT_PER_TENSOR ? sa[0] : sa[r < cur.row_end ? r : cur.row0]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = cur.n0 + wn * 64 + j * 16 + (lane >> 4) * 4 + v;
                scol[j][v] = block_w ? 1.0f : (w_quant == MOE_W_PER_EXPERT ? sb[cur.e] : sb[(int64_t)cur.e * N + (n < N ? n : N - 1)]);
            }

        };
        if constexpr (FP4 || KDEP) load_scales();

        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        if constexpr (!FP4 && !KDEP) {
            // operands of step k+1 are read into registers while step k's MFMAs run
            v8i fa0[4], fb0[4], fa1[4], fb1[4];
            auto read_step = [&](int k, v8i (&fa)[4], v8i (&fb)[4]) {
                const uint8_t* la = lds + (k % kDStages) * kDStage;
                const uint8_t* lb = la + kDStageA;
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = lds_operand(la, wm * 64 + i * 16 + (lane & 15), lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[j] = lds_operand(lb, wn * 64 + j * 16 + (lane & 15), lane);
            };
            auto mfmas = [&](v8i (&ca)[4], v8i (&cb)[4]) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            cb[j], ca[i], acc[i][j], 0, 0, 0, 0, 0, 0);
            };
            // one of the wave's six DMA instructions of K step k (0-1: A, 2-5: B)
            auto dma_one = [&](const DTile& t, int k, int i) {
                const uint32_t st = lds0 + (uint32_t)((k % kDStages) * kDStage);
                if (i < kDmaA) {
                    dma16(uniform_ptr(t.a_g + k * DBK), t.a_off[i],
                          __builtin_amdgcn_readfirstlane(st + (wid * kDmaA + i) * 1024));
                } else {
                    dma16(uniform_ptr(t.b_g + k * DBK), t.b_off[i - kDmaA],
                          __builtin_amdgcn_readfirstlane(st + kDStageA + (wid * kDmaB + i - kDmaA) * 1024));
                }
            };
            // step k (k + 1 < nk): publish step k+1; then eight groups of one operand
            // read of step k+1, two MFMAs of step k and (groups 0-5) one DMA of step k+3
            auto body = [&](int k, v8i (&ca)[4], v8i (&cb)[4], v8i (&na)[4], v8i (&nb)[4]) {
                if (k + 2 < nk) wait_vmcnt<kDma>();
                else wait_vmcnt<0>();
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of step k are done
                __syncthreads();  // step k+1 complete in LDS; the slot of step k is free
                const uint8_t* la1 = lds + ((k + 1) % kDStages) * kDStage;
                const uint8_t* lb1 = la1 + kDStageA;
                const bool more = k + 3 < nk;
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    if (g < 4) na[g] = lds_operand(la1, wm * 64 + g * 16 + (lane & 15), lane);
                    else nb[g - 4] = lds_operand(lb1, wn * 64 + (g - 4) * 16 + (lane & 15), lane);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i = (2 * g + h) >> 2, j = (2 * g + h) & 3;
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            cb[j], ca[i], acc[i][j], 0, 0, 0, 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (g < kDma && more) dma_one(cur, k + 3, g);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (nk > 1) wait_vmcnt<kDma>();
            else wait_vmcnt<0>();
            __syncthreads();  // step 0 complete
            read_step(0, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            if (nk > 2) issue(cur, 2);
            int k = 0;
            for (; k + 2 < nk; k += 2) {
                body(k, fa0, fb0, fa1, fb1);
                body(k + 1, fa1, fb1, fa0, fb0);
            }
            if (k + 1 < nk) {
                body(k, fa0, fb0, fa1, fb1);
                mfmas(fa1, fb1);
            } else {
                mfmas(fa0, fb0);
            }
        } else {
            for (int k = 0; k < nk; ++k) {
                if (k + 1 < nk) wait_vmcnt<kDmaN>();
                else wait_vmcnt<0>();
                if (group_act && tid < DBM) s_sa[k % kDStages][tid] = q;
                __syncthreads();  // stage k complete; every wave is done with stage k-1
                if (group_act && k + 1 < nk) q = sa[(int64_t)cur.sa_row * KB + k + 1];
                if (k + 2 < nk) issue(cur, k + 2);

                const uint8_t* la = lds + (k % kDStages) * kDStage;
                const uint8_t* lb = la + kDStageA;
                v8i af[4], bfr[4];
                if (FP4) {
                    // lane l: 16 bytes = the 32 codes of K block l / 16 of row l % 16,
                    // and that block's E8M0 scale; the activations in the matching order
#pragma unroll
                    for (int i = 0; i < 4; ++i) af[i] = lds_operand_x4(la, wm * 64 + i * 16 + (lane & 15), lane);
                    const uint8_t* lsc = la + kDStageS4;
                    int scl[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rb = wn * 64 + j * 16 + (lane & 15);
                        const uint4 q = *(const uint4*)(lb + rb * 64 + (fp4_pos(rb, lane >> 4) << 4));
                        bfr[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                        scl[j] = (int)lsc[rb * 4 + (lane >> 4)];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                bfr[j], af[i], acc[i][j], 4, 0, 0, scl[j], 0, 127);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) af[i] = lds_operand(la, wm * 64 + i * 16 + (lane & 15), lane);
#pragma unroll
                    for (int j = 0; j < 4; ++j) bfr[j] = lds_operand(lb, wn * 64 + j * 16 + (lane & 15), lane);
                    {  // K-dependent scales
                        const float sbv = block_w ? sb[((int64_t)cur.e * NB + cur.nb_w) * KB + k] : 1.0f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float f = (group_act ? s_sa[k % kDStages][wm * 64 + i * 16 + (lane & 15)] : 1.0f) * sbv;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    bfr[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                                for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(t[v], f, acc[i][j][v]);
                            }
                        }
                    }
                }
            }
        }
        if constexpr (!FP4 && !KDEP) load_scales();
        __syncthreads();  // every wave is done with the operand stages

        // next tile: its first two stages (slots 0 and 1) load during this epilogue
        const int lt_next = lt + per_xcd_blocks;
        const bool has_next = lt_next < lt_end;
        DTile nxt;
        if (has_next) {
            nxt = setup(lt_next);
            if (group_act) q = sa[(int64_t)nxt.sa_row * KB];
            if constexpr (!FP4 && !KDEP) issue_scales(nxt, par ^ 1);
            issue(nxt, 0);
            if (nk > 1) issue(nxt, 1);
        }

        // ---- epilogue: scales, bf16 into LDS slot 2, 16-byte row stores, in two
        // halves of 32 rows per wave (4 KB per wave) ----
        uint8_t* ep = lds + 2 * kDStage + wid * (32 * 128);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * h + ii;
                const int rl = ii * 16 + (lane & 15);  // row within the half
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cl = j * 16 + (lane >> 4) * 4;
                    float hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) hv[v] = acc[i][j][v] * (srow[i] * scol[j][v]);
                    *(uint2*)(ep + ep_off(rl, cl >> 3) + (cl & 7) * 2) =
                        make_uint2(bf16x2_rne(hv[0], hv[1]), bf16x2_rne(hv[2], hv[3]));
                }
            }
            // the staging area is the wave's own: its LDS writes are complete
            // (in order, one wave) before its lanes read each other's values
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int rl = t * 8 + (lane >> 3), qc = lane & 7;
                const int r = cur.row0 + wm * 64 + h * 32 + rl;
                const int n = cur.n0 + wn * 64 + qc * 8;
                const uint4 v = *(const uint4*)(ep + ep_off(rl, qc));
                if (r < cur.row_end && n < N) store16_nt(C + (int64_t)r * N + n, v);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // the half is read back before it is overwritten
            __builtin_amdgcn_wave_barrier();
        }
        if (!has_next) break;
        cur = nxt;
        lt = lt_next;
        par ^= 1;
    }
}

// ---- 256 x 256 tiles: eight waves (two per SIMD), two-stage LDS-DMA ring ----
//
// The block-scaled modes (1 x 128 activation groups or 128 x 128 weight blocks)
// when the segments can fill 256-row tiles. There every 128-deep MFMA result is
// added into the fp32 accumulators on the VALU with its own factor, so the
// register-prefetch schedule of the 128 x 256 kernel does not fit (it spills);
// a 256 x 256 tile halves the barriers and loads per flop instead. A step moves
// 64 KB (256 A rows and 256 B rows of 128 bytes) for 16.8 MFLOP, about 31 bytes
// per clock at one CU's MFMA rate through its L2 -> LDS path (which sustains
// about 50).
//
// Waves 2 (M) x 4 (N). Wave (wm, wn) owns the 64 columns wn*64.. (four 16-column
// MFMA blocks) and the eight 16-row blocks 2i + wm (i = 0..7): the row blocks
// alternate between the two wave rows, so a tile with fewer valid rows keeps
// both busy. Row blocks past the tile's valid rows skip their operand reads and
// MFMAs, and A DMA instructions whose eight rows are all past them are not
// issued. Accumulators: 8 x 4 blocks x 4 values = 128 fp32 per lane.
//
// Step k of a tile (stage s): wait for this wave's DMA of the step, one barrier
// (the stage is complete; every wave is done with the other stage, so it is
// free), then the DMA of the next step into the other stage -- the next step of
// this tile, or the first step of the block's next tile -- interleaved with the
// first four row blocks, then the MFMAs: the four B operands read once, A block
// i+1 read while block i's four MFMAs run. After the last step a barrier frees
// its stage, which then stages the bf16 tile for 16-byte row stores while the
// next tile's first step loads into the other one.
constexpr int GT = 256;                   // tile rows = tile columns
constexpr int kGStageA = GT * 128;        // 32 KB
constexpr int kGStage = 2 * kGStageA;     // 64 KB: A rows then B rows
constexpr int kGDma = GT * 128 / 1024 / 8;  // 1 KB DMA instructions per wave per operand per step: 4

struct GTile {
    int e, row0, row_end, n0, a_rows, b_rows, sa_row;
    const uint8_t* a_g;
    const uint8_t* b_g;
    uint32_t a_off[kGDma], b_off[kGDma];
};

template <bool KDEP>
__global__ __launch_bounds__(kDThreads, 1) void grouped_gemm_256_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const float* __restrict__ sb, int w_quant,
    const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds[2 * kGStage];
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];
    __shared__ float s_sa[2][GT];  // activation group scales of a step's rows (per-group mode)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 2, wn = wid & 3;
    const int KB = K / MOE_QB;
    const int NB = (N + MOE_QB - 1) / MOE_QB;
    const int nk = K / 128;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)lds;
    const bool group_act = KDEP && act_quant == MOE_ACT_PER_GROUP;
    const bool block_w = KDEP && w_quant == MOE_W_BLOCK;

    const int total = build_tile_table<GT, GT>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd_blocks = gridDim.x >> 3;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd;
    const int lt_end = lt_begin + per_xcd < total ? lt_begin + per_xcd : total;

    // DMA instruction q = wid + 8 i of an operand fills its rows 8 q .. 8 q + 7
    // (lane l: row 8 q + l / 8, LDS chunk position l % 8, which holds global
    // chunk (l % 8) ^ perm8(row)); rows past the valid ones re-read the last one
    auto setup = [&](int lt) {
        const TileCoord tc = tile_coord<GT, GT>(lt, s_seg, s_tstart, num_local);
        GTile t;
        t.e = __builtin_amdgcn_readfirstlane(tc.e);
        t.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
        t.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
        t.n0 = __builtin_amdgcn_readfirstlane(tc.n0);
        t.a_rows = tc.row_end - tc.row0;
        t.b_rows = N - tc.n0 < GT ? N - tc.n0 : GT;
#pragma unroll
        for (int i = 0; i < kGDma; ++i) {
            const int r = (wid + 8 * i) * 8 + (lane >> 3);
            const int ga = r < t.a_rows ? r : t.a_rows - 1;
            const int gb = r < t.b_rows ? r : t.b_rows - 1;
            const uint32_t chunk = (uint32_t)((((lane & 7) ^ perm8(r)) << 4));
            t.a_off[i] = (uint32_t)ga * (uint32_t)K + chunk;
            t.b_off[i] = (uint32_t)gb * (uint32_t)K + chunk;
        }
        t.a_g = A + (int64_t)t.row0 * K;
        t.b_g = B + ((int64_t)t.e * N + t.n0) * K;
        t.sa_row = t.row0 + ((tid & (GT - 1)) < t.a_rows ? (tid & (GT - 1)) : t.a_rows - 1);
        return t;
    };
    // part i (0..3) of the DMA of K step k of tile t into stage st: this wave's
    // A and B instruction wid + 8 i
    auto issue_part = [&](const GTile& t, int k, int st, int i) {
        const uint32_t base = lds0 + (uint32_t)(st * kGStage) + (uint32_t)((wid + 8 * i) * 1024);
        if ((wid + 8 * i) * 8 < t.a_rows)
            dma16(uniform_ptr(t.a_g + k * 128), t.a_off[i], __builtin_amdgcn_readfirstlane(base));
        if ((wid + 8 * i) * 8 < t.b_rows)
            dma16(uniform_ptr(t.b_g + k * 128), t.b_off[i], __builtin_amdgcn_readfirstlane(base + kGStageA));
    };

    int lt = lt_begin + slot;
    if (lt >= lt_end) return;  // the whole block has no tile

    GTile cur = setup(lt);
    float q = 0.f;  // this thread's activation group scale of the next step (per-group mode)
    if (group_act) q = sa[(int64_t)cur.sa_row * KB];
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_part(cur, 0, 0, i);
    int s = 0;  // stage of the current step

    while (true) {
        const int lt_next = lt + per_xcd_blocks;
        const bool has_next = lt_next < lt_end;
        GTile nxt = cur;
        if (has_next) nxt = setup(lt_next);
        const bool col_ok0 = wn * 64 < cur.b_rows;  // the wave has columns in this tile

        v4f acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        for (int k = 0; k < nk; ++k) {
            wait_vmcnt<0>();
            if (group_act && tid < GT) s_sa[s][tid] = q;
            __syncthreads();  // stage s complete; stage s ^ 1 free
            // what the next step in this block's sequence loads into stage s ^ 1
            const bool more = k + 1 < nk;
            const GTile& tn = more ? cur : nxt;
            const int kn = more ? k + 1 : 0;
            const bool issue = more || has_next;
            if (group_act && issue) q = sa[(int64_t)tn.sa_row * KB + kn];
            const int nb_w = (cur.n0 + wn * 64) / MOE_QB < NB ? (cur.n0 + wn * 64) / MOE_QB : NB - 1;
            const float sbv = block_w ? sb[((int64_t)cur.e * NB + nb_w) * KB + k] : 1.0f;

            const uint8_t* la = lds + s * kGStage;
            const uint8_t* lb = la + kGStageA;
            v8i bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = lds_operand(lb, wn * 64 + j * 16 + (lane & 15), lane);
            v8i af = lds_operand(la, wm * 16 + (lane & 15), lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < 4 && issue) issue_part(tn, kn, s ^ 1, i);
                const int rb = 2 * i + wm;
                if (rb * 16 < cur.a_rows && col_ok0) {
                    v8i an = af;
                    if (i + 1 < 8 && (rb + 2) * 16 < cur.a_rows)
                        an = lds_operand(la, (rb + 2) * 16 + (lane & 15), lane);
                    if constexpr (!KDEP) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                bfr[j], af, acc[i][j], 0, 0, 0, 0, 0, 0);
                    } else {
                        // each MFMA starts from zero and is added with the step's factor; two
                        // results in flight, so MFMA j + 1 runs while result j is added
                        const float f = (group_act ? s_sa[s][rb * 16 + (lane & 15)] : 1.0f) * sbv;
                        const v4f z = v4f{0.f, 0.f, 0.f, 0.f};
                        v4f t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[0], af, z, 0, 0, 0, 0, 0, 0);
                        v4f t1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[1], af, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][0][v] = __builtin_fmaf(t0[v], f, acc[i][0][v]);
                        t0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[2], af, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][1][v] = __builtin_fmaf(t1[v], f, acc[i][1][v]);
                        t1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[3], af, z, 0, 0, 0, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][2][v] = __builtin_fmaf(t0[v], f, acc[i][2][v]);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][3][v] = __builtin_fmaf(t1[v], f, acc[i][3][v]);
                    }
                    af = an;
                }
            }
            s ^= 1;
        }
        // s is the stage of the next tile's first step; s ^ 1 held this tile's last
        __syncthreads();  // every wave is done reading stage s ^ 1

        // ---- epilogue: scales, bf16 into stage s ^ 1 (8 KB per wave), 16-byte
        // row stores, in two halves of four row blocks ----
        float srow[8], scol[4][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = cur.row0 + (2 * i + wm) * 16 + (lane & 15);
            srow[i] = group_act ? 1.0f : (act_quant == MOE_ACT_PER_TENSOR ? sa[0] : sa[r < cur.row_end ? r : cur.row0]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = cur.n0 + wn * 64 + j * 16 + (lane >> 4) * 4 + v;
                scol[j][v] = block_w ? 1.0f : (w_quant == MOE_W_PER_EXPERT ? sb[cur.e] : sb[(int64_t)cur.e * N + (n < N ? n : N - 1)]);
            }
        uint8_t* ep = lds + (s ^ 1) * kGStage + wid * (64 * 128);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 4 * h + ii;
                const int rl = ii * 16 + (lane & 15);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cl = j * 16 + (lane >> 4) * 4;
                    float hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) hv[v] = acc[i][j][v] * (srow[i] * scol[j][v]);
                    *(uint2*)(ep + ep_off(rl, cl >> 3) + (cl & 7) * 2) =
                        make_uint2(bf16x2_rne(hv[0], hv[1]), bf16x2_rne(hv[2], hv[3]));
                }
            }
            // the staging area is the wave's own: its LDS writes are complete (in
            // order, one wave) before its lanes read each other's values
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int rl = t * 8 + (lane >> 3), qc = lane & 7;
                const int r = cur.row0 + (2 * (4 * h + (rl >> 4)) + wm) * 16 + (rl & 15);
                const int n = cur.n0 + wn * 64 + qc * 8;
                const uint4 v = *(const uint4*)(ep + ep_off(rl, qc));
                if (r < cur.row_end && n < N) store16_nt(C + (int64_t)r * N + n, v);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // the half is read back before it is overwritten
            __builtin_amdgcn_wave_barrier();
        }
        if (!has_next) break;
        cur = nxt;
        lt = lt_next;
    }
    wait_vmcnt<0>();
}

// ---- FP4 weights, 256-deep K steps: 128 x 256 tiles, two-stage DMA ring ----
//
// With MXFP4 weights a 128-deep K step moves 64 bytes per weight row, half a
// cache line; the CU's load path costs per line touched, so this kernel steps
// K by 256: a stage holds A (128 rows x 256 bytes, chunk c of row r at
// c ^ (r & 15)), B (256 rows x 128 bytes = 256 codes, the perm8 layout) and the
// rows' eight E8M0 scales, 66 KB; two stages fit. The DMA of step k+1 is issued
// at step k (the same lead in time as two 128-deep steps), each step waits for
// all of its loads, and the epilogue stages through the slot that is idle
// while the next tile's first step loads. Waves, MFMA operand order and
// epilogue as in the 128 x 256 FP8 kernel; each step is two 128-deep MFMA
// steps. Requires K % 256 == 0.
constexpr int F4K = 256;
constexpr int kF4StageA = DBM * F4K;                 // 32 KB
constexpr int kF4StageB = DBN * F4K / 2;             // 32 KB
constexpr int kF4StageS = DBN * F4K / 32;            // 2 KB
constexpr int kF4Stage = kF4StageA + kF4StageB + kF4StageS;
constexpr int kF4DmaA = kF4StageA / 1024 / 8;        // 4
constexpr int kF4DmaB = kF4StageB / 1024 / 8;        // 4

__device__ __forceinline__ int swz256(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

struct F4Tile {
    int e, row0, row_end, n0, a_rows, b_rows;
    const uint8_t* a_g;
    const uint8_t* b_g;
    const uint8_t* s_g;
    uint32_t a_off[kF4DmaA], b_off[kF4DmaB], s_off;
};

__global__ __launch_bounds__(kDThreads, 1) void grouped_gemm_fp4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Be8, const float* __restrict__ sb,
    int w_quant, const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds[2 * kF4Stage];
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 2, wn = wid & 3;
    const int nk = K / F4K;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)lds;

    const int total = build_tile_table<DBM, DBN>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd_blocks = gridDim.x >> 3;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd;
    const int lt_end = lt_begin + per_xcd < total ? lt_begin + per_xcd : total;

    auto setup = [&](int lt) {
        const TileCoord tc = tile_coord<DBM, DBN>(lt, s_seg, s_tstart, num_local);
        F4Tile t;
        t.e = tc.e;
        t.row0 = tc.row0;
        t.row_end = tc.row_end;
        t.n0 = tc.n0;
        t.a_rows = tc.row_end - tc.row0;
        t.b_rows = N - tc.n0 < DBN ? N - tc.n0 : DBN;
        // A: instruction i of wave w fills rows 4 (4 w + i) + lane / 16 at
        // position lane % 16 (global chunk (lane % 16) ^ (row & 15))
#pragma unroll
        for (int i = 0; i < kF4DmaA; ++i) {
            const int r = (wid * kF4DmaA + i) * 4 + (lane >> 4);
            const int g = r < t.a_rows ? r : t.a_rows - 1;
            t.a_off[i] = (uint32_t)g * (uint32_t)K + (uint32_t)((((lane & 15) ^ (r & 15)) << 4));
        }
        // B: instruction i of wave w fills rows 8 (4 w + i) + lane / 8 at
        // position lane % 8 (global chunk (lane % 8) ^ perm8(row))
#pragma unroll
        for (int i = 0; i < kF4DmaB; ++i) {
            const int r = (wid * kF4DmaB + i) * 8 + (lane >> 3);
            const int g = r < t.b_rows ? r : t.b_rows - 1;
            t.b_off[i] = (uint32_t)g * (uint32_t)(K / 2) + (uint32_t)((((lane & 7) ^ perm8(r)) << 4));
        }
        // scales: wave w loads dword lane % 2 of rows 32 w + lane / 2
        const int rs = wid * 32 + (lane >> 1);
        t.s_off = (uint32_t)(rs < t.b_rows ? rs : t.b_rows - 1) * (uint32_t)(K / 32) + (uint32_t)((lane & 1) * 4);
        t.a_g = A + (int64_t)t.row0 * K;
        t.b_g = B + ((int64_t)t.e * N + t.n0) * (K / 2);
        t.s_g = Be8 + ((int64_t)t.e * N + t.n0) * (K / 32);
        return t;
    };
    auto issue = [&](const F4Tile& t, int k, int s) {  // DMA of K step k into stage s
        const uint32_t st = lds0 + (uint32_t)(s * kF4Stage);
        const uint8_t* ab = uniform_ptr(t.a_g + k * F4K);
        const uint32_t la = __builtin_amdgcn_readfirstlane(st + wid * kF4DmaA * 1024);
#pragma unroll
        for (int i = 0; i < kF4DmaA; ++i) dma16(ab, t.a_off[i], la + i * 1024);
        const uint8_t* bb = uniform_ptr(t.b_g + k * (F4K / 2));
        const uint32_t lb = __builtin_amdgcn_readfirstlane(st + kF4StageA + wid * kF4DmaB * 1024);
#pragma unroll
        for (int i = 0; i < kF4DmaB; ++i) dma16(bb, t.b_off[i], lb + i * 1024);
        dma4(uniform_ptr(t.s_g + k * (F4K / 32)), t.s_off,
             __builtin_amdgcn_readfirstlane(st + kF4StageA + kF4StageB + wid * 256));
    };

    int lt = lt_begin + slot;
    if (lt >= lt_end) return;  // the whole block has no tile

    F4Tile cur = setup(lt);
    issue(cur, 0, 0);

    while (true) {
        float srow[4], scol[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = cur.row0 + wm * 64 + i * 16 + (lane & 15);
            srow[i] = act_quant == MOE_ACT_PER_TENSOR ? sa[0] : sa[r < cur.row_end ? r : cur.row0];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = cur.n0 + wn * 64 + j * 16 + (lane >> 4) * 4 + v;
                scol[j][v] = w_quant == MOE_W_PER_EXPERT ? sb[cur.e] : sb[(int64_t)cur.e * N + (n < N ? n : N - 1)];
            }

        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        for (int k = 0; k < nk; ++k) {
            wait_vmcnt<0>();
            __syncthreads();  // stage k complete; every wave is done with the other stage
            if (k + 1 < nk) issue(cur, k + 1, (k + 1) & 1);

            const uint8_t* la = lds + (k & 1) * kF4Stage;
            const uint8_t* lb = la + kF4StageA;
            const uint8_t* lsc = lb + kF4StageB;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // two 128-deep MFMA steps
                v8i af[4], bfr[4];
                int scl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // activations in the order the scaled MFMA pairs with E2M1
                    // lanes: chunks l/16 and l/16 + 4 of this 128-deep half
                    const int r = wm * 64 + i * 16 + (lane & 15);
                    const int c = h * 8 + (lane >> 4);
                    const uint4 lo = *(const uint4*)(la + swz256(r, c));
                    const uint4 hi = *(const uint4*)(la + swz256(r, c + 4));
                    af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rb = wn * 64 + j * 16 + (lane & 15);
                    const uint4 q = *(const uint4*)(lb + swz(rb, h * 4 + (lane >> 4)));
                    bfr[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                    scl[j] = (int)lsc[rb * 8 + h * 4 + (lane >> 4)];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bfr[j], af[i], acc[i][j], 4, 0, 0, scl[j], 0, 127);
            }
        }
        __syncthreads();  // every wave is done with both stages

        // the next tile's first step loads into stage 0 during this epilogue
        const int lt_next = lt + per_xcd_blocks;
        const bool has_next = lt_next < lt_end;
        F4Tile nxt;
        if (has_next) {
            nxt = setup(lt_next);
            issue(nxt, 0, 0);
        }

        // ---- epilogue through stage 1: scales, bf16, 16-byte row stores, two
        // halves of 32 rows per wave ----
        uint8_t* ep = lds + kF4Stage + wid * (32 * 128);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * h + ii;
                const int rl = ii * 16 + (lane & 15);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cl = j * 16 + (lane >> 4) * 4;
                    float hv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) hv[v] = acc[i][j][v] * (srow[i] * scol[j][v]);
                    *(uint2*)(ep + ep_off(rl, cl >> 3) + (cl & 7) * 2) =
                        make_uint2(bf16x2_rne(hv[0], hv[1]), bf16x2_rne(hv[2], hv[3]));
                }
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int rl = t * 8 + (lane >> 3), qc = lane & 7;
                const int r = cur.row0 + wm * 64 + h * 32 + rl;
                const int n = cur.n0 + wn * 64 + qc * 8;
                const uint4 v = *(const uint4*)(ep + ep_off(rl, qc));
                if (r < cur.row_end && n < N) store16_nt(C + (int64_t)r * N + n, v);
            }
            __syncthreads();
        }
        if (!has_next) break;
        cur = nxt;
        lt = lt_next;
    }
    wait_vmcnt<0>();
}

// ---- few rows per expert: weight streaming ----
//
// When every local expert holds a handful of rows (decode), a 128-row tile is
// mostly padding and the GEMM's cost is reading each expert's weights once from
// HBM. Here a unit is (expert, 16 of its rows, 16 output columns) over the whole
// of K, listed like the tiles above (m fastest, so an expert's 16-row blocks of
// one column block run side by side and share its weights in L2), and every
// wave of a persistent grid takes its XCD's units in turn on its own: once the
// unit list is built no LDS and no barrier is shared between waves, so no wave
// waits for another's loads.
//
// Weights cannot go straight into MFMA registers at full HBM rate: a 16x16x128
// operand spreads one load instruction over 16 rows of 64 bytes, and 128-byte
// row segments stream about a fifth faster. So both operands go through the
// wave's own LDS ring by global_load_lds_dwordx4, eight rows of 128 bytes per
// instruction (the weights with the nontemporal hint unless the expert has
// more than 16 rows, whose row blocks share them through L2), SSTAGES stages of one K
// step each. A wave's units form one stream of K steps: step j + SSTAGES - 1 is
// issued while step j is consumed, across unit boundaries, so the ring never
// drains between units. Per step the wave issues exactly kSDma DMA
// instructions: its 16 weight rows (two), the unit's 16 activation rows (two;
// rows past the unit's last one re-read it, from L2) and two 4-byte DMAs of the
// unit's epilogue scales (16 row scales, 16 column scales; re-sent each step
// into one of two buffers by unit parity). A step: wait for the step's loads,
// issue the next, one MFMA B x A. After a unit's last step the wave scales,
// rounds to bf16 and stores its 16 x 16 outputs.
constexpr int SC = 16;                       // output columns per unit
constexpr int SM = 16;                       // rows per unit
constexpr int SSTAGES = 4;
constexpr int kSStageB = SC * 128;           // 2 KB
constexpr int kSStage = kSStageB + SM * 128;  // + 2 KB of activations
constexpr int kSDma = 6;                     // DMA instructions per wave per step

// vmcnt wait: at most n steps of this wave's DMA (kSDma each) still in flight
__device__ __forceinline__ void wait_steps(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<kSDma>(); break;
        default: wait_vmcnt<2 * kSDma>(); break;
    }
}
static_assert(SSTAGES - 2 == 2, "wait_steps covers 0 .. SSTAGES - 2 steps");

struct SUnit {
    int row0, row_end, n0;
    int shared_b;        // the expert has more than SM rows: other units read these weights too
    const uint8_t* a_g;  // first activation row of the unit
    const uint8_t* b_g;  // first weight row of the unit
    uint32_t offb0, offb1, offa0, offa1, offsa, offsb;  // per-lane DMA offsets (see setup)
};

__global__ __launch_bounds__(256, 2) void grouped_gemm_stream_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const float* __restrict__ sb, int w_quant,
    const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds[4][SSTAGES * kSStage];
    __shared__ __align__(16) float s_scale[4][2][128];  // per wave, per unit parity: row scales, column scales
    __shared__ int s_seg[kMaxLocal + 1];
    __shared__ int s_tstart[kMaxLocal + 1];
    __shared__ int scan_scratch[17];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nk = K / 128;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)&lds[wid][0];
    const uint32_t lds_sc = (uint32_t)(uintptr_t)(const void*)&s_scale[wid][0][0];

    const int total = build_tile_table<SM, SC>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);
    // this XCD's waves take its contiguous eighth of the units in turn
    const int xcd = blockIdx.x & 7;
    const int per_xcd_waves = (gridDim.x >> 3) * 4;
    const int wx = (blockIdx.x >> 3) * 4 + wid;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd + wx;
    const int lt_end = xcd * per_xcd + per_xcd < total ? xcd * per_xcd + per_xcd : total;
    if (lt_begin >= lt_end) return;
    const int n_units = (lt_end - lt_begin + per_xcd_waves - 1) / per_xcd_waves;
    const int n_steps = n_units * nk;

    // DMA offsets of unit u: weight rows 8 i + lane / 8 (i = 0, 1) and activation
    // rows likewise (past the unit's valid rows: its last one); chunk lane % 8 of
    // an LDS row holds global chunk (lane % 8) ^ perm8(row). Scales: lane l the
    // row scale of row l % 16 (clamped) and the column scale of column l % 16.
    auto setup = [&](int u) {
        const TileCoord tc = tile_coord<SM, SC>(lt_begin + u * per_xcd_waves, s_seg, s_tstart, num_local);
        SUnit t;
        t.row0 = tc.row0;
        t.row_end = tc.row_end;
        t.n0 = tc.n0;
        t.shared_b = s_seg[tc.e + 1] - s_seg[tc.e] > SM;
        const int a_rows = tc.row_end - tc.row0;
        t.a_g = A + (int64_t)tc.row0 * K;
        t.b_g = B + ((int64_t)tc.e * N + tc.n0) * K;
        const int c = lane & 7, r0 = lane >> 3, r1 = 8 + (lane >> 3);
        t.offb0 = (uint32_t)r0 * (uint32_t)K + (uint32_t)((c ^ perm8(r0)) << 4);
        t.offb1 = (uint32_t)r1 * (uint32_t)K + (uint32_t)((c ^ perm8(r1)) << 4);
        t.offa0 = (uint32_t)(r0 < a_rows ? r0 : a_rows - 1) * (uint32_t)K + (uint32_t)((c ^ perm8(r0)) << 4);
        t.offa1 = (uint32_t)(r1 < a_rows ? r1 : a_rows - 1) * (uint32_t)K + (uint32_t)((c ^ perm8(r1)) << 4);
        const int l = lane & 15;
        t.offsa = act_quant == MOE_ACT_PER_TENSOR ? 0u : (uint32_t)(tc.row0 + (l < a_rows ? l : a_rows - 1)) * 4u;
        t.offsb = w_quant == MOE_W_PER_EXPERT ? (uint32_t)tc.e * 4u
                                              : (uint32_t)((int64_t)tc.e * N + tc.n0 + l) * 4u;
        return t;
    };
    // issue step k of unit u (descriptor t) into stage s
    const uint8_t* sa_b = uniform_ptr((const uint8_t*)sa);
    const uint8_t* sb_b = uniform_ptr((const uint8_t*)sb);
    auto issue = [&](const SUnit& t, int u, int k, int s) {
        const uint32_t st = lds0 + (uint32_t)(s * kSStage);
        const uint8_t* bb = uniform_ptr(t.b_g + k * 128);
        const uint8_t* ab = uniform_ptr(t.a_g + k * 128);
        if (t.shared_b) {  // read again by the expert's other row blocks: keep in L2
            dma16(bb, t.offb0, __builtin_amdgcn_readfirstlane(st));
            dma16(bb, t.offb1, __builtin_amdgcn_readfirstlane(st + 1024));
        } else {
            dma16_nt(bb, t.offb0, __builtin_amdgcn_readfirstlane(st));
            dma16_nt(bb, t.offb1, __builtin_amdgcn_readfirstlane(st + 1024));
        }
        dma16(ab, t.offa0, __builtin_amdgcn_readfirstlane(st + kSStageB));
        dma16(ab, t.offa1, __builtin_amdgcn_readfirstlane(st + kSStageB + 1024));
        const uint32_t sc = lds_sc + (uint32_t)((u & 1) * 128 * 4);
        dma4(sa_b, t.offsa, __builtin_amdgcn_readfirstlane(sc));
        dma4(sb_b, t.offsb, __builtin_amdgcn_readfirstlane(sc + 64 * 4));
    };

    // issue cursor (unit ui, step ki; ji steps issued so far) runs SSTAGES - 1 ahead
    int ui = 0, ki = 0, ji = 0;
    SUnit ti = setup(0);
    SUnit tc = ti;  // unit being consumed
    for (; ji < SSTAGES - 1 && ji < n_steps; ++ji) {
        issue(ti, ui, ki, ji % SSTAGES);
        if (++ki == nk) { ki = 0; if (++ui < n_units) ti = setup(ui); }
    }
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    int uc = 0, kc = 0;
    for (int j = 0; j < n_steps; ++j) {
        // step j's loads are done once at most the later issued steps remain
        wait_steps(ji - 1 - j);
        // lgkmcnt(0): the reads of step j - 1, whose stage the next issue fills, are done
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (ji < n_steps) {
            issue(ti, ui, ki, ji % SSTAGES);
            ++ji;
            if (++ki == nk) { ki = 0; if (++ui < n_units) ti = setup(ui); }
        }
        const uint8_t* st = &lds[wid][(j % SSTAGES) * kSStage];
        const v8i bo = lds_operand(st, lane & 15, lane);
        const v8i ao = lds_operand(st + kSStageB, lane & 15, lane);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bo, ao, acc, 0, 0, 0, 0, 0, 0);
        if (++kc == nk) {
            // lane l, value v: row row0 + l % 16, column n0 + 4 (l / 16) + v
            const float* sc = &s_scale[wid][uc & 1][0];
            const int m = tc.row0 + (lane & 15);
            const int nl = 4 * (lane >> 4);
            const float srow = sc[lane & 15];
            float hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) hv[v] = acc[v] * (srow * sc[64 + nl + v]);
            if (m < tc.row_end)
                *(uint2*)(C + (int64_t)m * N + tc.n0 + nl) =
                    make_uint2(bf16x2_rne(hv[0], hv[1]), bf16x2_rne(hv[2], hv[3]));
            acc = v4f{0.f, 0.f, 0.f, 0.f};
            kc = 0;
            if (++uc < n_units) tc = setup(uc);
        }
    }
    wait_vmcnt<0>();
}

// ---- few rows per expert, MXFP4 weights: weight streaming ----
//
// The scheme of the FP8 streaming kernel with 256-deep K steps, so that a weight
// row's step is one 128-byte line (256 E2M1 codes) as in the FP8 kernel: per
// step a wave's stage holds its 16 weight rows (2 KB, perm8 layout) and the
// unit's activation rows of 256 bytes (chunk c of row r at c ^ r), and two
// 128-deep scaled MFMAs consume it with the operand orders of the tiled FP4
// kernel. A unit has 8 rows here (an 8 x 256-byte activation stage), so that four
// stages per wave fit two blocks per CU; the MFMA's lanes for rows 8-15 read
// rows 0-7 again and those outputs are not stored.
//
// The weights' E8M0 block scales (8 bytes per row per step) come eight steps at
// a time: one 16-byte DMA per lane brings 64 bytes of each of the 16 rows into
// one of two per-wave buffers (alternating by group of eight steps), issued
// with the group's first step; per step they would cost as many cache lines
// as the codes. So the DMA count of a step varies: weights (two) and
// activations (two), plus one at a group's first step, plus two (the unit's
// fp32 row and column scales, into the buffer of the unit's parity) at a unit's
// first step. A step waits until only the DMAs of the steps issued after it
// are in flight, from the recorded counts of the last two issued steps.
constexpr int S4K = 256;
constexpr int S4M = 8;                          // rows per unit
constexpr int S4STAGES = 4;
constexpr int S4G = 8;                          // K steps per E8M0 scale group
constexpr int kS4StageB = SC * 128;             // 2 KB of E2M1 codes
constexpr int kS4StageA = S4M * S4K;            // 2 KB of activations
constexpr int kS4Stage = kS4StageB + kS4StageA;
constexpr int kS4Group = SC * S4G * 8;          // 1 KB of E8M0 scales per group
constexpr int kS4MaxLocal = 256;

// vmcnt wait for at most n of this wave's DMA instructions still in flight
// (n <= 14: the two later issued steps, at most seven each)
__device__ __forceinline__ void wait_dma4(int n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        default: wait_vmcnt<14>(); break;
    }
}
static_assert(S4STAGES - 2 == 2, "wait_dma4 covers the two later issued steps");

struct S4Unit {
    int row0, row_end, n0, shared_b;
    const uint8_t* a_g;  // first activation row
    const uint8_t* b_g;  // first weight row (E2M1 codes)
    const uint8_t* e_g;  // its E8M0 scales
    uint32_t offb0, offb1, offa0, offa1, offsa, offsb;
};

__global__ __launch_bounds__(256, 2) void grouped_gemm_stream_fp4_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, int act_quant,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Be8, const float* __restrict__ sb, int w_quant,
    const int32_t* __restrict__ seg_in, int num_local, int64_t m_cap, int N, int K,
    uint16_t* __restrict__ C) {
    __shared__ __align__(16) uint8_t lds[4][S4STAGES * kS4Stage];
    __shared__ __align__(16) uint8_t s_e8[4][2][kS4Group];
    __shared__ __align__(16) float s_scale[4][2][128];
    __shared__ int s_seg[kS4MaxLocal + 1];
    __shared__ int s_tstart[kS4MaxLocal + 1];
    __shared__ int scan_scratch[17];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nk = K / S4K;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const void*)&lds[wid][0];
    const uint32_t lds_e8 = (uint32_t)(uintptr_t)(const void*)&s_e8[wid][0][0];
    const uint32_t lds_sc = (uint32_t)(uintptr_t)(const void*)&s_scale[wid][0][0];

    const int total = build_tile_table<S4M, SC>(seg_in, num_local, m_cap, N, s_seg, s_tstart, scan_scratch);
    const int xcd = blockIdx.x & 7;
    const int per_xcd_waves = (gridDim.x >> 3) * 4;
    const int wx = (blockIdx.x >> 3) * 4 + wid;
    const int per_xcd = (total + 7) / 8;
    const int lt_begin = xcd * per_xcd + wx;
    const int lt_end = xcd * per_xcd + per_xcd < total ? xcd * per_xcd + per_xcd : total;
    if (lt_begin >= lt_end) return;
    const int n_units = (lt_end - lt_begin + per_xcd_waves - 1) / per_xcd_waves;
    const int n_steps = n_units * nk;
    const int gpu = (nk + S4G - 1) / S4G;  // scale groups per unit

    auto setup = [&](int u) {
        const TileCoord tc = tile_coord<S4M, SC>(lt_begin + u * per_xcd_waves, s_seg, s_tstart, num_local);
        S4Unit t;
        t.row0 = tc.row0;
        t.row_end = tc.row_end;
        t.n0 = tc.n0;
        t.shared_b = s_seg[tc.e + 1] - s_seg[tc.e] > S4M;
        const int a_rows = tc.row_end - tc.row0;
        t.a_g = A + (int64_t)tc.row0 * K;
        t.b_g = B + ((int64_t)tc.e * N + tc.n0) * (K / 2);
        t.e_g = Be8 + ((int64_t)tc.e * N + tc.n0) * (K / 32);
        // weights: rows 8 i + lane / 8 at chunk position lane % 8 (global chunk
        // (lane % 8) ^ perm8(row))
        const int c8 = lane & 7, r0 = lane >> 3, r1 = 8 + (lane >> 3);
        t.offb0 = (uint32_t)r0 * (uint32_t)(K / 2) + (uint32_t)((c8 ^ perm8(r0)) << 4);
        t.offb1 = (uint32_t)r1 * (uint32_t)(K / 2) + (uint32_t)((c8 ^ perm8(r1)) << 4);
        // activations: rows 4 i + lane / 16 (clamped to the unit's rows) at chunk
        // position lane % 16 (global chunk (lane % 16) ^ row)
        const int c16 = lane & 15, q0 = lane >> 4, q1 = 4 + (lane >> 4);
        t.offa0 = (uint32_t)(q0 < a_rows ? q0 : a_rows - 1) * (uint32_t)K + (uint32_t)((c16 ^ q0) << 4);
        t.offa1 = (uint32_t)(q1 < a_rows ? q1 : a_rows - 1) * (uint32_t)K + (uint32_t)((c16 ^ q1) << 4);
        const int l = lane & 15;
        t.offsa = act_quant == MOE_ACT_PER_TENSOR ? 0u : (uint32_t)(tc.row0 + (l < a_rows ? l : a_rows - 1)) * 4u;
        t.offsb = w_quant == MOE_W_PER_EXPERT ? (uint32_t)tc.e * 4u
                                              : (uint32_t)((int64_t)tc.e * N + tc.n0 + l) * 4u;
        return t;
    };
    const uint8_t* sa_b = uniform_ptr((const uint8_t*)sa);
    const uint8_t* sb_b = uniform_ptr((const uint8_t*)sb);
    // lane l of a scale group's DMA: 16 bytes at byte 16 (l % 4) of row l / 4's
    // 64 (clamped to the row's last 16 bytes past its end; those are not used)
    const uint32_t e_row = (uint32_t)(lane >> 2) * (uint32_t)(K / 32);
    // issue step k of unit u (descriptor t) into stage s; gi: the scale groups
    // issued so far (the buffer of this step's group is (gi - 1) & 1 after a
    // group start). Returns the number of DMA instructions issued.
    auto issue = [&](const S4Unit& t, int u, int k, int s, int& gi) {
        const uint32_t st = lds0 + (uint32_t)(s * kS4Stage);
        const uint8_t* bb = uniform_ptr(t.b_g + k * (S4K / 2));
        const uint8_t* ab = uniform_ptr(t.a_g + k * S4K);
        if (t.shared_b) {  // read again by the expert's other row blocks: keep in L2
            dma16(bb, t.offb0, __builtin_amdgcn_readfirstlane(st));
            dma16(bb, t.offb1, __builtin_amdgcn_readfirstlane(st + 1024));
        } else {
            dma16_nt(bb, t.offb0, __builtin_amdgcn_readfirstlane(st));
            dma16_nt(bb, t.offb1, __builtin_amdgcn_readfirstlane(st + 1024));
        }
        dma16(ab, t.offa0, __builtin_amdgcn_readfirstlane(st + kS4StageB));
        dma16(ab, t.offa1, __builtin_amdgcn_readfirstlane(st + kS4StageB + 1024));
        int n = 4;
        if (k % S4G == 0) {
            const int byte = (k / S4G) * (S4G * 8) + (lane & 3) * 16;
            const int last = K / 32 - 16;
            dma16(uniform_ptr(t.e_g), e_row + (uint32_t)(byte < last ? byte : last),
                  __builtin_amdgcn_readfirstlane(lds_e8 + (uint32_t)((gi & 1) * kS4Group)));
            ++gi;
            ++n;
        }
        if (k == 0) {
            const uint32_t sc = lds_sc + (uint32_t)((u & 1) * 128 * 4);
            dma4(sa_b, t.offsa, __builtin_amdgcn_readfirstlane(sc));
            dma4(sb_b, t.offsb, __builtin_amdgcn_readfirstlane(sc + 64 * 4));
            n += 2;
        }
        return n;
    };

    // issue cursor: unit ui, step ki, ji steps and gi scale groups issued;
    // n_last / n_prev: DMA instructions of the last / the one before last issued step
    int ui = 0, ki = 0, ji = 0, gi = 0, n_last = 0, n_prev = 0;
    S4Unit ti = setup(0);
    S4Unit tc = ti;
    for (; ji < S4STAGES - 1 && ji < n_steps; ++ji) {
        n_prev = n_last;
        n_last = issue(ti, ui, ki, ji % S4STAGES, gi);
        if (++ki == nk) { ki = 0; if (++ui < n_units) ti = setup(ui); }
    }
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    int uc = 0, kc = 0;
    const int ra = lane & 7;  // activation row of this lane's MFMA operand (rows 8-15 repeat 0-7)
    for (int j = 0; j < n_steps; ++j) {
        const int later = ji - 1 - j;
        wait_dma4(later >= 2 ? n_last + n_prev : (later == 1 ? n_last : 0));
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the reads of step j - 1 are done
        if (ji < n_steps) {
            n_prev = n_last;
            n_last = issue(ti, ui, ki, ji % S4STAGES, gi);
            ++ji;
            if (++ki == nk) { ki = 0; if (++ui < n_units) ti = setup(ui); }
        }
        const uint8_t* lb = &lds[wid][(j % S4STAGES) * kS4Stage];
        const uint8_t* la = lb + kS4StageB;
        // this step's scale group: the (uc * gpu + kc / S4G)-th of this wave
        const uint8_t* le = &s_e8[wid][(uc * gpu + kc / S4G) & 1][(kc % S4G) * 8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // two 128-deep MFMA steps
            const int rb = lane & 15;
            const uint4 q = *(const uint4*)(lb + swz(rb, h * 4 + (lane >> 4)));
            const v8i bo = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            const int scl = (int)le[rb * (S4G * 8) + h * 4 + (lane >> 4)];
            const int c = h * 8 + (lane >> 4);
            const uint4 lo = *(const uint4*)(la + swz256(ra, c));
            const uint4 hi = *(const uint4*)(la + swz256(ra, c + 4));
            const v8i ao = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bo, ao, acc, 4, 0, 0, scl, 0, 127);
        }
        if (++kc == nk) {
            const float* sc = &s_scale[wid][uc & 1][0];
            const int m = tc.row0 + (lane & 15);
            const int nl = 4 * (lane >> 4);
            const float srow = sc[lane & 15];
            float hv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) hv[v] = acc[v] * (srow * sc[64 + nl + v]);
            if (m < tc.row_end)
                *(uint2*)(C + (int64_t)m * N + tc.n0 + nl) =
                    make_uint2(bf16x2_rne(hv[0], hv[1]), bf16x2_rne(hv[2], hv[3]));
            acc = v4f{0.f, 0.f, 0.f, 0.f};
            kc = 0;
            if (++uc < n_units) tc = setup(uc);
        }
    }
    wait_vmcnt<0>();
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
    const bool kdep_modes = act_quant == MOE_ACT_PER_GROUP || w_quant == MOE_W_BLOCK;
    if (!kdep_modes && K % 128 == 0 && K / 128 >= SSTAGES && m_cap <= (int64_t)64 * num_local &&
        (int64_t)K * SM < ((int64_t)1 << 32) && (int64_t)num_local * N * 4 < ((int64_t)1 << 32)) {
        // few rows per expert (at most 64 on average even if every row slot is
        // filled): stream each expert's weights once
        const int64_t upper = (ceil_div(m_cap, SM) + num_local) * ceil_div(N, SC);  // units
        int64_t g = 2 * (int64_t)device_cu_count();
        if (g > ceil_div(upper, 32) * 8) g = ceil_div(upper, 32) * 8;  // four waves per block
        g = ceil_div(g < 8 ? 8 : g, 8) * 8;
        hipLaunchKernelGGL(grouped_gemm_stream_kernel, dim3((unsigned)g), dim3(256), 0, (hipStream_t)stream,
                           a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr, num_local, m_cap, N, K,
                           (uint16_t*)c_bf16);
        return launch_status();
    }
    if (kdep_modes && K % 128 == 0 && (int64_t)K * GT < ((int64_t)1 << 32) && m_cap >= (int64_t)128 * num_local) {
        // block-scaled modes with segments that could average 128 rows or more
        // per local expert (chosen from the sizes alone; M stays on the device):
        // 256 x 256 tiles
        const int64_t upper = (ceil_div(m_cap, GT) + num_local) * ceil_div(N, GT);
        int64_t g = (int64_t)device_cu_count();
        if (g > ceil_div(upper, 8) * 8) g = ceil_div(upper, 8) * 8;
        g = ceil_div(g < 8 ? 8 : g, 8) * 8;
        hipLaunchKernelGGL((grouped_gemm_256_kernel<true>), dim3((unsigned)g), dim3(kDThreads), 0,
                           (hipStream_t)stream, a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr,
                           num_local, m_cap, N, K, (uint16_t*)c_bf16);
        return launch_status();
    }
    if (K % DBK == 0 && (int64_t)K * DBN < ((int64_t)1 << 32)) {
        // large tiles, LDS-DMA pipeline: one block per CU
        const int64_t upper = (ceil_div(m_cap, DBM) + num_local) * ceil_div(N, DBN);
        int64_t g = (int64_t)device_cu_count();
        if (g > ceil_div(upper, 8) * 8) g = ceil_div(upper, 8) * 8;
        g = ceil_div(g < 8 ? 8 : g, 8) * 8;
        hipStream_t st = (hipStream_t)stream;
        const uint8_t* no_e8m0 = nullptr;
        if (act_quant == MOE_ACT_PER_GROUP || w_quant == MOE_W_BLOCK)
            hipLaunchKernelGGL((grouped_gemm_dma_kernel<true, false>), dim3((unsigned)g), dim3(kDThreads), 0, st,
                               a_q, a_scale, act_quant, b_q, no_e8m0, b_scale, w_quant, seg_indptr,
                               num_local, m_cap, N, K, (uint16_t*)c_bf16);
        else
            hipLaunchKernelGGL((grouped_gemm_dma_kernel<false, false>), dim3((unsigned)g), dim3(kDThreads), 0, st,
                               a_q, a_scale, act_quant, b_q, no_e8m0, b_scale, w_quant, seg_indptr,
                               num_local, m_cap, N, K, (uint16_t*)c_bf16);
        return launch_status();
    }
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

extern "C" int moe_grouped_gemm_mxfp4(const uint8_t* a_q, const float* a_scale, int64_t a_scale_numel,
                                      int32_t act_quant, const uint8_t* b_fp4, const uint8_t* b_e8m0,
                                      const float* b_scale, int64_t b_scale_numel, int32_t w_quant,
                                      const int32_t* seg_indptr, int32_t num_local, int64_t m_cap,
                                      int32_t N, int32_t K, void* c_bf16, void* stream) {
    using namespace moe;
    if (num_local < 0 || m_cap < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
    if (act_quant < MOE_ACT_PER_TENSOR || act_quant > MOE_ACT_PER_GROUP) return MOE_ERR_INVALID_ARG;
    if (w_quant < MOE_W_PER_EXPERT || w_quant > MOE_W_BLOCK) return MOE_ERR_INVALID_ARG;
    if (act_quant == MOE_ACT_PER_GROUP || w_quant == MOE_W_BLOCK) return MOE_ERR_UNSUPPORTED;
    if (K % DBK != 0 || N % 16 != 0 || num_local > kMaxLocal) return MOE_ERR_UNSUPPORTED;
    if (m_cap > INT32_MAX / 2 || (int64_t)K * DBN >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    const int64_t want_a = act_quant == MOE_ACT_PER_TENSOR ? 1 : m_cap;
    const int64_t want_b = w_quant == MOE_W_PER_EXPERT ? num_local : (int64_t)num_local * N;
    if (a_scale_numel != want_a || b_scale_numel != want_b) return MOE_ERR_SHAPE;
    if (!seg_indptr) return MOE_ERR_NULL;
    if (num_local == 0 || m_cap == 0) return MOE_OK;  // no rows can exist
    if (!a_q || !a_scale || !b_fp4 || !b_e8m0 || !b_scale || !c_bf16) return MOE_ERR_NULL;
    if (!aligned16(a_q) || !aligned16(b_fp4) || !aligned16(c_bf16) || ((uintptr_t)b_e8m0 & 3u) != 0)
        return MOE_ERR_INVALID_ARG;

    (void)hipGetLastError();
    // (the scale groups of eight steps: every group, a unit's last included, has
    // at least three steps, so a group's buffer is refilled only after its last
    // step has been read)
    const int s4_tail = (K / S4K) % S4G;
    if (K % 512 == 0 && K / S4K >= S4STAGES && (s4_tail == 0 || s4_tail >= 3) && ((uintptr_t)b_e8m0 & 15u) == 0 &&
        m_cap <= (int64_t)64 * num_local && num_local <= kS4MaxLocal &&
        (int64_t)K * SC < ((int64_t)1 << 32) && (int64_t)num_local * N * (K / 32) < ((int64_t)1 << 32)) {
        // few rows per expert: stream each expert's weights once
        const int64_t units = (ceil_div(m_cap, S4M) + num_local) * ceil_div(N, SC);
        int64_t g = 2 * (int64_t)device_cu_count();
        if (g > ceil_div(units, 32) * 8) g = ceil_div(units, 32) * 8;  // four waves per block
        g = ceil_div(g < 8 ? 8 : g, 8) * 8;
        hipLaunchKernelGGL(grouped_gemm_stream_fp4_kernel, dim3((unsigned)g), dim3(256), 0, (hipStream_t)stream,
                           a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant, seg_indptr, num_local, m_cap,
                           N, K, (uint16_t*)c_bf16);
        return launch_status();
    }
    const int64_t upper = (ceil_div(m_cap, DBM) + num_local) * ceil_div(N, DBN);
    int64_t g = (int64_t)device_cu_count();
    if (g > ceil_div(upper, 8) * 8) g = ceil_div(upper, 8) * 8;
    g = ceil_div(g < 8 ? 8 : g, 8) * 8;
    if (K % F4K == 0)  // full cache lines of weights per K step
        hipLaunchKernelGGL(grouped_gemm_fp4_kernel, dim3((unsigned)g), dim3(kDThreads), 0,
                           (hipStream_t)stream, a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant,
                           seg_indptr, num_local, m_cap, N, K, (uint16_t*)c_bf16);
    else
        hipLaunchKernelGGL((grouped_gemm_dma_kernel<false, true>), dim3((unsigned)g), dim3(kDThreads), 0,
                           (hipStream_t)stream, a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant,
                           seg_indptr, num_local, m_cap, N, K, (uint16_t*)c_bf16);
    return launch_status();
}
