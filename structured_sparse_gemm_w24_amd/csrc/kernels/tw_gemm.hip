// Tile-wise sparse GEMM for gfx950.
//
// "Accelerating Sparse DNN Models without Hardware-Support via Tile-Wise
// Sparsity" (Guo et al.): each G-column tile t of W keeps its own rows
// (offset_k, global k) and columns (offset_n, tile-local) and runs as a
// condensed dense block V_t [N_t x K_t]; the run-time GEMM reads A through
// offset_k and writes C through offset_n (run-time slide).  The slides
// transpose A so that the picked rows are contiguous; this kernel takes the
// K-major At [K][M].
//
// One workgroup (8 waves) handles one work item: a block of BM = 128 tokens
// of one tile.
//   * The tile's offset_k list is copied to LDS (KCAP entries at a time);
//     every stage of BK picked rows is then gathered global -> LDS with
//     direct-to-LDS loads: a picked row of At is 256 contiguous bytes for the
//     block's tokens, so 16 lanes fetch one row.  V_t's rows for the stage
//     are copied the same way.  Padding rows (N_t rounded up to 16) and the
//     K_t tail read a zero page, so both operands are zero there.  Stages
//     live in a ring of NB buffers handed over with one counter wait and one
//     barrier per stage.
//   * The At stage stays K-major in LDS ([k][token], 16-byte chunks XOR
//     swizzled by row).  The matrix instruction wants 8 consecutive k of one
//     token per lane; gfx950's transposing LDS read gives exactly that:
//     within a 16-lane group, lane i receives element i%4 of the 8-byte run
//     read by lane 4e + i/4 (e = 0..3), so lanes aimed at rows k0 + j/4,
//     tokens 4(j%4).. return 4 consecutive k per token; two reads give 8.
//   * v_mfma_f32_16x16x32_f16 accumulates D[j][token] = sum_k V_t[j][k] At[k][token];
//     each wave owns 16 tokens and all NJ = ceil(N_t/16) column blocks of the
//     tile (NJ is a template parameter: one instantiation per value).
//   * Epilogue: the tile's G-wide output window for the 128 tokens is built in
//     LDS (zeros, then accumulators rounded to nearest even and scattered to
//     column offset_n[j]) and stored with 16-byte coalesced nontemporal
//     writes, so pruned columns of C come out as +0 without a separate fill.
//   * The production shape (32-row stages, three buffers, 512-entry index
//     chunks) needs 52 KiB of LDS and under 85 VGPRs, so three workgroups
//     share a CU: one workgroup's epilogue stores and index loads overlap the
//     others' main loops.
// Work items are ordered token-block-major with tiles heaviest first (the
// packer's tile_order), and block ids are remapped so each XCD owns a
// contiguous range of items: the tiles that share a token block share its At
// rows in one L2.
#include "common.h"
#include "launch.h"
#include "tw_common.h"

namespace ssg {

// A zero page: the source of padding rows and K tails.
__device__ __attribute__((aligned(256))) uint16_t g_tw_zero[128];

namespace {

using namespace tw_detail;

// Column operand of two k32 steps: four transposing reads at byte offsets
// 0, 1024 (k + 4), 8192 (k + 32) and 9216 (k + 36) from addr, waited for in
// the same statement so no result register is live while its load is in
// flight.
__device__ __forceinline__ void tw_read_b(uint32_t addr, u32x2 &b0, u32x2 &b1, u32x2 &b2, u32x2 &b3) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:1024\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:8192\n\t"
        "ds_read_b64_tr_b16 %3, %4 offset:9216\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(addr)
        : "memory");
}

// Column operand of one k32 step: two transposing reads (k and k + 4).
__device__ __forceinline__ void tw_read_b2(uint32_t addr, u32x2 &b0, u32x2 &b1) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(b0), "=&v"(b1)
        : "v"(addr)
        : "memory");
}

}  // namespace

// BK picked rows per stage (32 or 64), NB stage buffers, KCAP offset_k
// entries held in LDS at a time, WPE waves per SIMD the register allocation
// must allow (two workgroups per CU need 4), GMAX the widest tile, NTMAX the
// most kept columns of a tile (rows of a stage's V_t part).
template <int BK_, int NB_, int KCAP_, int WPE_, int GMAX_ = 128, int NTMAX_ = GMAX_>
struct TwCfg {
    static constexpr int NW = 8, NT = NW * 64;
    static constexpr int BM = 128;   // tokens per work item (8 blocks of 16)
    static constexpr int BK = BK_;
    static constexpr int KS = BK / 32;  // k32 steps per stage
    static constexpr int NB = NB_;
    static constexpr int KCAP = KCAP_;
    static constexpr int WPE = WPE_;
    static constexpr int GMAX = GMAX_;    // widest supported tile
    static constexpr int NTMAX = NTMAX_;  // most kept columns per tile
    static constexpr int A_STAGE = BK * BM * 2;     // [BK][BM] halves
    static constexpr int W_STAGE = NTMAX * BK * 2;  // [NTMAX][BK] halves
    static constexpr int STAGE = A_STAGE + W_STAGE;
    static constexpr int LA = A_STAGE / 1024 / NW;  // A loads per wave per stage
    static constexpr int WROWS = 1024 / (BK * 2);   // V_t rows per direct-to-LDS load
    static constexpr int WIN_ROW = GMAX * 2 + 16;   // output window row stride (bytes)
    static constexpr int IDX_OFF = NB * STAGE;       // offset_k chunk, KCAP ints
    static constexpr int OFFN_OFF = IDX_OFF + KCAP * 4;  // offset_n of the tile, GMAX ints
    static constexpr int SMEM = OFFN_OFF + GMAX * 4;
    static_assert(BK == 32 || BK == 64, "stage depth");
    static_assert(LA >= 1 && LA * NW * 1024 == A_STAGE, "A stage must split over the waves");
    static_assert(KCAP % NT == 0, "index chunk must split over the threads");
    // the output window may extend over the index chunk, which the epilogue no longer reads
    static_assert(BM * WIN_ROW <= NB * STAGE + KCAP * 4, "output window must fit in the stage ring");
    static_assert(NTMAX % 16 == 0 && NTMAX <= GMAX, "kept-column capacity");
    static_assert(NB >= 2 && NB <= 4, "ring depth");
};

// At stage: row r (picked k), 16-byte chunk c (8 tokens) -> stored chunk.  The
// four rows one transposing read touches land in distinct 32-byte bank groups.
__device__ __forceinline__ int tw_swz_a(int r, int c) { return c ^ (2 * (r & 3)); }
// V_t stage: row j (channel), 16-byte chunk c (8 k) of a BK-wide row -> stored
// chunk; the 8 rows read by 8 consecutive lanes cover all banks.
template <int BK>
__device__ __forceinline__ int tw_swz_w(int j, int c) {
    if constexpr (BK == 64) return c ^ ((j ^ (j >> 3)) & 7);
    else return c ^ ((j >> 1) & 3);
}

// How the At stage reaches LDS.
//   A_DMA    K-major At [K][M], M a multiple of 8: 16-byte direct-to-LDS loads;
//   A_ROW    row-major A [M][K] (the slides' "without transpose" case): the
//            picked k of a token are scattered 2-byte elements of its row, so
//            each stage is gathered through registers, 8 elements per thread,
//            into the same K-major LDS layout; every element is its own
//            memory request;
//   A_KGATH  K-major At with M not a multiple of 8: a picked row's 16-byte
//            pieces are not 16-byte aligned, so each thread gathers 8
//            consecutive tokens of one picked row through registers (2-byte
//            loads, bounds-checked against M) into the same LDS layout.
enum AMode { A_DMA = 0, A_ROW = 1, A_KGATH = 2 };

// OUTT: write C transposed, Ct [N][M] (token-contiguous rows), which is the
// K-major input of a following tile-wise layer (the transpose fused into the
// producing GEMM); otherwise C [M][N].  Cw points at the tile's first output
// column (row, for OUTT).
template <class CF, int NJ, bool OUTT, int AM>
__device__ __forceinline__ void tw_item(uint8_t *smem, const uint16_t *__restrict__ At,
                                        const uint16_t *__restrict__ vt, const int32_t *__restrict__ offk,
                                        const int32_t *__restrict__ offn, int kt, int nt, int G, int m0,
                                        uint16_t *__restrict__ Cw, int M, int N, int K) {
    constexpr int NW = CF::NW, NT = CF::NT, BM = CF::BM, BK = CF::BK, NB = CF::NB, KCAP = CF::KCAP;
    constexpr int A_STAGE = CF::A_STAGE, STAGE = CF::STAGE, LA = CF::LA, KS = CF::KS, WROWS = CF::WROWS;
    constexpr int WIN_ROW = CF::WIN_ROW;
    int32_t *s_idx = reinterpret_cast<int32_t *>(smem + CF::IDX_OFF);
    int32_t *s_offn = reinterpret_cast<int32_t *>(smem + CF::OFFN_OFF);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ld = (kt + 7) & ~7;
    // V_t loads per stage: NJ*16 rows of 2*BK bytes = NJ*KS KiB, round-robin over waves
    const int lw = (NJ * KS - wave + NW - 1) / NW;
    const int per_stage = (AM == A_DMA ? LA : 0) + lw;  // direct-to-LDS loads per stage

    // A loads: instruction j of the wave covers stage rows 4q .. 4q+3 (q = j*NW + wave);
    // lane -> row 4q + lane/16, stored chunk lane%16.
    const int a_sub = lane >> 4, a_pos = lane & 15;
    // W loads: rows WROWS*q ..; lane -> row WROWS*q + lane/(8*KS), stored chunk lane%(4*KS).
    const int w_sub = lane / (4 * KS), w_pos = lane % (4 * KS);

    floatx4 acc[NJ > 0 ? NJ : 1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int tok_mb = wave * 16;  // this wave's 16 tokens inside the block
    const int g16 = lane >> 4, j16 = lane & 15;
    // transposing-read address inside a stage: row 8*g16 + j16/4, tokens tok_mb + 4*(j16%4)
    const int rb = 8 * g16 + (j16 >> 2);
    const int tokl = tok_mb + 4 * (j16 & 3);
    const uint32_t b_off = rb * (BM * 2) + tw_swz_a(rb, tokl >> 3) * 16 + (tokl & 7) * 2;
    const uint32_t smem_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

    if (tid < nt && tid < CF::GMAX) s_offn[tid] = offn[tid];  // read back after the barriers below
    if constexpr (NJ > 0) {
        for (int cb = 0; cb < kt; cb += KCAP) {
            const int ck = min(KCAP, kt - cb);  // picked rows in this chunk
            if (cb > 0) __syncthreads();        // every wave is done with the previous list
            {
                // all loads first (clamped to the last entry), then the guarded LDS writes
                constexpr int PER = KCAP / NT;
                int32_t v[PER];
#pragma unroll
                for (int p = 0; p < PER; ++p) v[p] = offk[cb + min(tid + p * NT, ck - 1)];
#pragma unroll
                for (int p = 0; p < PER; ++p)
                    if (tid + p * NT < ck) s_idx[tid + p * NT] = v[p];
            }
            __syncthreads();
            const int S = (ck + BK - 1) / BK;

            auto issue = [&](int s) {
                uint8_t *base = smem + (s % NB) * STAGE;
                if constexpr (AM == A_KGATH) {
                    static_assert(BK * BM == NT * 8, "gather mapping: one 8-token piece per thread");
                    // thread -> picked row r, stored 16-byte chunk p (source chunk tw_swz_a(r, p))
                    const int r = tid / (BM / 8), p = tid % (BM / 8);
                    const int kk = s * BK + r;
                    const int tok = m0 + tw_swz_a(r, p) * 8;
                    const bool row_ok = kk < ck;
                    const int64_t rb = row_ok ? int64_t(s_idx[kk]) * M : 0;
                    uint16_t v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (row_ok && tok + e < M) ? At[rb + tok + e] : uint16_t(0);
                    u32x4 w;
                    w.x = uint32_t(v[0]) | (uint32_t(v[1]) << 16);
                    w.y = uint32_t(v[2]) | (uint32_t(v[3]) << 16);
                    w.z = uint32_t(v[4]) | (uint32_t(v[5]) << 16);
                    w.w = uint32_t(v[6]) | (uint32_t(v[7]) << 16);
                    *reinterpret_cast<u32x4 *>(base + r * (BM * 2) + p * 16) = w;
                }
                if constexpr (AM == A_ROW) {
                    static_assert(BK == 32 && NT == 4 * BM, "gather mapping: 4 threads x 8 picked rows per token");
                    const int tok = tid >> 2, kg = (tid & 3) * 8;
                    const int m = m0 + tok;
                    uint16_t v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kk = s * BK + kg + e;
                        v[e] = (kk < ck && m < M) ? At[int64_t(m) * K + s_idx[kk]] : uint16_t(0);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = kg + e;
                        *reinterpret_cast<uint16_t *>(base + r * (BM * 2) + tw_swz_a(r, tok >> 3) * 16 + (tok & 7) * 2) =
                            v[e];
                    }
                }
#pragma unroll
                for (int j = 0; j < (AM == A_DMA ? LA : 0); ++j) {
                    const int q = j * NW + wave;
                    const int r = 4 * q + a_sub;  // stage row
                    const int kk = s * BK + r;    // picked row inside the chunk
                    const int tok = m0 + tw_swz_a(r, a_pos) * 8;
                    const void *src = g_tw_zero;
                    if (kk < ck && tok < M) src = At + int64_t(s_idx[kk]) * M + tok;
                    tw_dma16(src, base + q * 1024);
                }
                for (int j = 0; j < lw; ++j) {
                    const int q = j * NW + wave;
                    const int row = WROWS * q + w_sub;
                    const int k = cb + s * BK + tw_swz_w<BK>(row, w_pos) * 8;
                    const void *src = g_tw_zero;
                    if (row < nt && k < ld) src = vt + int64_t(row) * ld + k;
                    tw_dma16(src, base + A_STAGE + q * 1024);
                }
            };

            for (int s = 0; s < NB - 1 && s < S; ++s) issue(s);
            for (int s = 0; s < S; ++s) {
                // stage s complete; the younger stages already issued may stay in flight
                tw_wait_barrier(min(NB - 2, S - 1 - s) * per_stage);
                // the buffer of stage s-1 is free: refill it with stage s+NB-1
                if (s + NB - 1 < S) issue(s + NB - 1);
                const uint32_t stage_off = (s % NB) * STAGE;
                const uint8_t *bW = smem + stage_off + A_STAGE;
                u32x2 b[2 * KS];
                if constexpr (KS == 2) tw_read_b(smem_addr + stage_off + b_off, b[0], b[1], b[2], b[3]);
                else tw_read_b2(smem_addr + stage_off + b_off, b[0], b[1]);
#pragma unroll
                for (int k32 = 0; k32 < KS; ++k32) {
                    const half8 bf = __builtin_bit_cast(
                        half8, __builtin_shufflevector(b[2 * k32], b[2 * k32 + 1], 0, 1, 2, 3));
                    // V_t fragments in batches of at most 8 column blocks (register budget of wide tiles)
                    constexpr int JC = NJ > 8 ? 8 : NJ;
#pragma unroll
                    for (int j0 = 0; j0 < NJ; j0 += JC) {
                        u32x4 wf[JC];
#pragma unroll
                        for (int jj = 0; jj < JC; ++jj) {
                            const int row = (j0 + jj) * 16 + j16;
                            if (j0 + jj < NJ)
                                wf[jj] = *reinterpret_cast<const u32x4 *>(bW + row * (BK * 2) +
                                                                          tw_swz_w<BK>(row, k32 * 4 + g16) * 16);
                        }
#pragma unroll
                        for (int jj = 0; jj < JC; ++jj)
                            if (j0 + jj < NJ)
                                acc[j0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    __builtin_bit_cast(half8, wf[jj]), bf, acc[j0 + jj], 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---- epilogue: G-wide output window in LDS (aliases the stage ring); rows
    // padded by 16 bytes so the 16 tokens (or channels) one scatter instruction
    // writes fall in distinct banks
    __syncthreads();
    uint8_t *win = smem;
    if constexpr (!OUTT) {
        const int wrow_chunks = G / 8;  // 16-byte chunks per window row
        for (int c = tid; c < BM * wrow_chunks; c += NT)
            *reinterpret_cast<u32x4 *>(win + (c / wrow_chunks) * WIN_ROW + (c % wrow_chunks) * 16) =
                u32x4{0, 0, 0, 0};
        __syncthreads();
        // acc[jb] lane (g16, j16) holds D[j = 16jb + 4*g16 + i][token = tok_mb + j16]
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jb * 16 + 4 * g16 + i;
                if (j < nt)
                    *reinterpret_cast<uint16_t *>(win + (tok_mb + j16) * WIN_ROW + s_offn[j] * 2) =
                        __builtin_bit_cast(uint16_t, (_Float16)acc[jb][i]);
            }
        }
        __syncthreads();
        for (int c = tid; c < BM * wrow_chunks; c += NT) {
            const int row = c / wrow_chunks, ch = c % wrow_chunks;
            const int m = m0 + row;
            if (m < M)
                tw_store16(Cw + int64_t(m) * N + ch * 8, *reinterpret_cast<const u32x4 *>(win + row * WIN_ROW + ch * 16));
        }
    } else {
        // transposed window [G][BM]: row = tile-local channel, tokens contiguous
        constexpr int TROW = BM * 2 + 16;
        static_assert(CF::GMAX * TROW <= CF::NB * CF::STAGE + CF::KCAP * 4,
                      "transposed window must fit in the stage ring and index chunk");
        constexpr int TCH = BM / 8;  // 16-byte chunks per row
        for (int c = tid; c < G * TCH; c += NT)
            *reinterpret_cast<u32x4 *>(win + (c / TCH) * TROW + (c % TCH) * 16) = u32x4{0, 0, 0, 0};
        __syncthreads();
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jb * 16 + 4 * g16 + i;
                if (j < nt)
                    *reinterpret_cast<uint16_t *>(win + s_offn[j] * TROW + (tok_mb + j16) * 2) =
                        __builtin_bit_cast(uint16_t, (_Float16)acc[jb][i]);
            }
        }
        __syncthreads();
        if (M % 8 == 0) {
            for (int c = tid; c < G * TCH; c += NT) {
                const int row = c / TCH, ch = c % TCH;
                const int m = m0 + ch * 8;  // a chunk is all in or all out
                if (m < M)
                    tw_store16(Cw + int64_t(row) * M + m,
                               *reinterpret_cast<const u32x4 *>(win + row * TROW + ch * 16));
            }
        } else {
            // rows of Ct are not 16-byte aligned: one 2-byte store per token
            for (int c = tid; c < G * BM; c += NT) {
                const int row = c / BM, tk = c % BM;
                const int m = m0 + tk;
                if (m < M) Cw[int64_t(row) * M + m] = *reinterpret_cast<const uint16_t *>(win + row * TROW + tk * 2);
            }
        }
    }
}

// An item whose tile keeps more columns than the configuration holds (a
// caller that promised narrow tiles and passed a wider one): its whole output
// window is written as quiet NaN, so the broken promise shows in C instead of
// leaving stale values there.
template <class CF, bool OUTT>
__device__ __forceinline__ void tw_nan_window(int G, int m0, uint16_t *__restrict__ Cw, int M, int N) {
    constexpr uint16_t kNaN = 0x7e00;
    const int tid = threadIdx.x;
    const int rows = min(CF::BM, M - m0);
    if constexpr (!OUTT) {
        for (int c = tid; c < rows * G; c += CF::NT) Cw[int64_t(m0 + c / G) * N + c % G] = kNaN;
    } else {
        for (int c = tid; c < G * rows; c += CF::NT) Cw[int64_t(c / rows) * M + m0 + c % rows] = kNaN;
    }
}

// Work items: token block mb x tiles tile_order[t_first .. t_first + t_count).
template <class CF, bool OUTT, int AM>
__global__ void __launch_bounds__(CF::NT) __attribute__((amdgpu_waves_per_eu(CF::WPE)))
tw_gemm_kernel(const uint16_t *__restrict__ At, const uint16_t *__restrict__ vals, const int32_t *__restrict__ offset_k,
               const int32_t *__restrict__ offset_n, const int32_t *__restrict__ v_ptr,
               const int32_t *__restrict__ k_ptr, const int32_t *__restrict__ n_ptr,
               const int32_t *__restrict__ tile_order, int t_first, int t_count, int G, uint16_t *__restrict__ C,
               int M, int N, int K) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[CF::SMEM];
    const int n_mb = (M + CF::BM - 1) / CF::BM;
    const int item = xcd_remap(blockIdx.x, n_mb * t_count);
    const int mb = item / t_count;
    const int t = tile_order[t_first + item % t_count];
    const int kp0 = k_ptr[t], kt = k_ptr[t + 1] - kp0;
    const int np0 = n_ptr[t], nt = n_ptr[t + 1] - np0;
    const uint16_t *vt = vals + v_ptr[t];
    const int32_t *offk = offset_k + kp0;
    const int32_t *offn = offset_n + np0;
    uint16_t *Cw = OUTT ? C + int64_t(t) * G * M : C + int64_t(t) * G;
    const int m0 = mb * CF::BM;
    // (a tile of at most GMAX columns has at most GMAX/16 column blocks)
    switch ((nt + 15) >> 4) {
#define TW_CASE(J) \
    case J:                                                                                  \
        if constexpr (J <= CF::NTMAX / 16)                                                   \
            tw_item<CF, J, OUTT, AM>(smem, At, vt, offk, offn, kt, nt, G, m0, Cw, M, N, K); \
        else                                                                                 \
            tw_nan_window<CF, OUTT>(G, m0, Cw, M, N);                                        \
        break;
        TW_CASE(0) TW_CASE(1) TW_CASE(2) TW_CASE(3) TW_CASE(4) TW_CASE(5) TW_CASE(6) TW_CASE(7) TW_CASE(8)
        TW_CASE(9) TW_CASE(10) TW_CASE(11) TW_CASE(12) TW_CASE(13) TW_CASE(14) TW_CASE(15) TW_CASE(16)
#undef TW_CASE
        default: break;
    }
}

// 32-row stages, three buffers, 512 picked rows per index chunk: 51.7 KiB of
// LDS and at most 85 VGPRs (6 waves per SIMD), so three workgroups share a CU.
using TwProd = TwCfg<32, 3, 512, 6>;
// Tiles wider than 128 columns (up to 256): 75 KiB of LDS (two workgroups per
// CU) and up to 16 column blocks of accumulators per wave.
using TwWide = TwCfg<32, 3, 512, 4, 256>;
// Narrow tiles (at most 64 kept columns, the caller's promise): the stage's
// V_t part holds 64 rows and a wave at most 4 column blocks of accumulators,
// which takes the kernel to 38.5 KiB of LDS and under 64 VGPRs, so four
// workgroups share a CU (BERT-large fc1, 1536 items: 22.7 vs 24.1 us).
using TwNarrow = TwCfg<32, 3, 512, 8, 128, 64>;
// Narrow tiles in launches with at most two items per CU and a long K, where
// each item's chain of K stages sets the time rather than the items sharing a
// CU: 64-row stages halve the chain (two buffers, 50.5 KiB, three workgroups
// per CU; BERT-large fc2, 384 items of 1311 picked rows: 22.0 vs 25.8 us).
// With short chains the single buffer in flight costs more than the halving
// gains (BERT-large fc1 as one 48-item launch per tile: 120 vs 94 us).
using TwNarrowDeep = TwCfg<64, 2, 512, 6, 128, 64>;
constexpr int kTwCUs = 256;  // compute units of an MI355X

template <class CF>
static hipError_t launch_tw_cfg(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                                const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                                const int32_t *tile_order, int t_first, int t_count, int G, bool out_t,
                                bool a_rowmajor, void *C, int M, int N, int K, hipStream_t st) {
    const int n_mb = (M + CF::BM - 1) / CF::BM;
    const int am = a_rowmajor ? A_ROW : (M % 8 ? A_KGATH : A_DMA);
    auto kern = out_t ? tw_gemm_kernel<CF, true, A_DMA> : tw_gemm_kernel<CF, false, A_DMA>;
    if constexpr (CF::BK == 32) {  // the register gathers are written for 32-row stages
        if (am == A_ROW) kern = out_t ? tw_gemm_kernel<CF, true, A_ROW> : tw_gemm_kernel<CF, false, A_ROW>;
        if (am == A_KGATH) kern = out_t ? tw_gemm_kernel<CF, true, A_KGATH> : tw_gemm_kernel<CF, false, A_KGATH>;
    } else if (am != A_DMA) {
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kern, dim3(n_mb * t_count), dim3(CF::NT), 0, st, static_cast<const uint16_t *>(At),
                       static_cast<const uint16_t *>(vals), offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order,
                       t_first, t_count, G, static_cast<uint16_t *>(C), M, N, K);
    return hipGetLastError();
}

hipError_t launch_tw_f16(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                         const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                         const int32_t *tile_order, int t_first, int t_count, int G, bool out_t, bool a_rowmajor,
                         bool narrow, void *C, int M, int N, int K, hipStream_t st) {
    if (narrow && G <= TwNarrow::GMAX) {
        const int64_t items = int64_t((M + TwNarrow::BM - 1) / TwNarrow::BM) * t_count;
        // (the 64-row stages take only the direct-to-LDS gather of 16-byte aligned At rows)
        if (!a_rowmajor && M % 8 == 0 && items <= 2 * kTwCUs && K >= 2048)
            return launch_tw_cfg<TwNarrowDeep>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order,
                                               t_first, t_count, G, out_t, false, C, M, N, K, st);
        return launch_tw_cfg<TwNarrow>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, t_first,
                                       t_count, G, out_t, a_rowmajor, C, M, N, K, st);
    }
    if (G > TwProd::GMAX)
        return launch_tw_cfg<TwWide>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, t_first,
                                     t_count, G, out_t, a_rowmajor, C, M, N, K, st);
    return launch_tw_cfg<TwProd>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, t_first, t_count, G,
                                 out_t, a_rowmajor, C, M, N, K, st);
}

}  // namespace ssg
