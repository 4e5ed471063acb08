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
// One workgroup handles one work item (tile t, block of BM tokens):
//   * the kept rows of At are gathered stage by stage (BK rows per stage);
//     16 lanes read one picked row's 8*16 tokens as 256 contiguous bytes;
//   * every thread owns an 8 (k) x 8 (token) block, transposes it in
//     registers (byte permutes) and writes 8 K-contiguous 16-byte rows to LDS,
//     which is the operand layout of the matrix instruction;
//   * V_t's stage (rows padded with zeros to a multiple of 16) is copied to
//     LDS the same way; K_t tails are zero on both operands;
//   * v_mfma_f32_16x16x32_f16 accumulates D[token][j] in fp32;
//   * the epilogue builds the tile's full G-wide output window in LDS: zeros,
//     then the rounded (nearest-even) accumulators scattered to column
//     offset_n[j]; the window is then stored with 16-byte coalesced writes, so
//     pruned columns of C come out as +0 without a separate fill.
// Index arrays are software-pipelined two stages ahead of the data, so the
// gather never waits on its own index load.  Work items are ordered
// token-block-major with tiles heaviest first (the packer's tile_order), and
// block ids are remapped so that each XCD owns a contiguous range of items:
// the tiles that share a token block share its At rows in one L2.
#include "common.h"
#include "launch.h"

namespace ssg {

namespace tw {
constexpr int NT = 256;  // 4 waves
constexpr int BM = 128;  // tokens per work item
constexpr int BK = 128;  // gathered k per stage
constexpr int ROWB = BK * 2;  // bytes per LDS row (16 chunks)

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 15); }
}  // namespace tw

template <int GMAX>
__global__ void __launch_bounds__(tw::NT)
tw_gemm_kernel(const uint16_t *__restrict__ At, const uint16_t *__restrict__ vals, const int32_t *__restrict__ offset_k,
               const int32_t *__restrict__ offset_n, const int32_t *__restrict__ v_ptr,
               const int32_t *__restrict__ k_ptr, const int32_t *__restrict__ n_ptr,
               const int32_t *__restrict__ tile_order, int T, int G, uint16_t *__restrict__ C, int M, int N) {
    using namespace tw;
    constexpr int NBJ = GMAX / 16;  // max 16-column blocks
    static_assert(BM * GMAX * 2 <= 2 * BM * ROWB, "output window must fit in the A buffers");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][GMAX * ROWB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    const int n_mb = (M + BM - 1) / BM;
    const int item = xcd_remap(blockIdx.x, n_mb * T);
    const int mb = item / T;
    const int t = tile_order[item % T];
    const int m0 = mb * BM;

    const int kp0 = k_ptr[t], kt = k_ptr[t + 1] - kp0;
    const int np0 = n_ptr[t], nt = n_ptr[t + 1] - np0;
    const int vp0 = v_ptr[t];
    const int ld = (kt + 7) & ~7;
    const int nbj = (nt + 15) >> 4;
    const int S = (kt + BK - 1) / BK;
    const int32_t *okt = offset_k + kp0;
    const uint16_t *vt = vals + vp0;

    // gather role: token chunk tc (8 tokens), k group kg (8 picked rows)
    const int tc = tid & 15, kg = tid >> 4;
    const bool tok_ok = (m0 + tc * 8) < M;
    const uint16_t *at_base = At + m0 + tc * 8;

    int ridx[8], rnext[8];
    u32x4 ra[8], rw[NBJ];

    auto load_idx = [&](int s, int *dst) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = s * BK + kg * 8 + j;
            dst[j] = (s < S && kk < kt) ? okt[kk] : -1;
        }
    };
    auto load_data = [&](int s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ra[j] = u32x4{0, 0, 0, 0};
            if (tok_ok && ridx[j] >= 0) ra[j] = ld16(at_base + int64_t(ridx[j]) * M);
        }
        const int kb = s * BK;
#pragma unroll
        for (int i = 0; i < NBJ; ++i) {
            rw[i] = u32x4{0, 0, 0, 0};
            const int row = (tid >> 4) + 16 * i, col = tid & 15;
            const int k = kb + col * 8;
            if (i < nbj && row < nt && k < ld) rw[i] = ld16(vt + int64_t(row) * ld + k);
        }
    };
    auto store_data = [&](int buf) {
        // 8x8 transpose: out[i] holds k = kg*8 .. +7 of token tc*8 + i
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
            u32x4 o;
            o.x = __builtin_amdgcn_perm(ra[1][i >> 1], ra[0][i >> 1], sel);
            o.y = __builtin_amdgcn_perm(ra[3][i >> 1], ra[2][i >> 1], sel);
            o.z = __builtin_amdgcn_perm(ra[5][i >> 1], ra[4][i >> 1], sel);
            o.w = __builtin_amdgcn_perm(ra[7][i >> 1], ra[6][i >> 1], sel);
            const int row = tc * 8 + i;
            *reinterpret_cast<u32x4 *>(&sA[buf][row * ROWB + swz(row, kg) * 16]) = o;
        }
#pragma unroll
        for (int i = 0; i < NBJ; ++i) {
            if (i < nbj) {
                const int row = (tid >> 4) + 16 * i, col = tid & 15;
                *reinterpret_cast<u32x4 *>(&sW[buf][row * ROWB + swz(row, col) * 16]) = rw[i];
            }
        }
    };

    floatx4 acc[2][NBJ];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) acc[a][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (S > 0) {
        load_idx(0, ridx);
        load_idx(1, rnext);
        load_data(0);
        store_data(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) ridx[j] = rnext[j];
        load_idx(2, rnext);
    }
    __syncthreads();

    const int r16 = lane & 15, q = lane >> 4;
    for (int s = 0; s < S; ++s) {
        const int buf = s & 1;
        if (s + 1 < S) load_data(s + 1);
        const uint8_t *bA = sA[buf];
        const uint8_t *bW = sW[buf];
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int chunk = kk * 4 + q;
            half8 af[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int row = wave * 32 + a * 16 + r16;
                af[a] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(bA + row * ROWB + swz(row, chunk) * 16));
            }
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                if (j < nbj) {
                    const int row = j * 16 + r16;
                    const half8 bf =
                        __builtin_bit_cast(half8, *reinterpret_cast<const u32x4 *>(bW + row * ROWB + swz(row, chunk) * 16));
#pragma unroll
                    for (int a = 0; a < 2; ++a)
                        acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf, acc[a][j], 0, 0, 0);
                }
            }
        }
        if (s + 1 < S) {
            store_data(buf ^ 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) ridx[j] = rnext[j];
            load_idx(s + 3, rnext);
        }
        __syncthreads();
    }

    // ---- epilogue: G-wide output window in LDS (aliases the A buffers)
    uint16_t *win = reinterpret_cast<uint16_t *>(&sA[0][0]);
    const int wrow_chunks = G / 8;  // 16-byte chunks per window row
    for (int c = tid; c < BM * wrow_chunks; c += NT)
        *reinterpret_cast<u32x4 *>(win + c * 8) = u32x4{0, 0, 0, 0};
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
        const int jj = j * 16 + r16;
        if (j < nbj && jj < nt) {
            const int col = offset_n[np0 + jj];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wave * 32 + a * 16 + q * 4 + i;
                    win[row * G + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[a][j][i]);
                }
        }
    }
    __syncthreads();
    const int64_t c0 = int64_t(t) * G;
    for (int c = tid; c < BM * wrow_chunks; c += NT) {
        const int row = c / wrow_chunks, ch = c % wrow_chunks;
        const int m = m0 + row;
        if (m < M) st16(C + int64_t(m) * N + c0 + ch * 8, *reinterpret_cast<const u32x4 *>(win + row * G + ch * 8));
    }
}

hipError_t launch_tw_f16(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                         const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                         const int32_t *tile_order, int T, int G, void *C, int M, int N, hipStream_t st) {
    const int n_mb = (M + tw::BM - 1) / tw::BM;
    const dim3 grid(n_mb * T), block(tw::NT);
    hipLaunchKernelGGL((tw_gemm_kernel<128>), grid, block, 0, st, static_cast<const uint16_t *>(At),
                       static_cast<const uint16_t *>(vals), offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G,
                       static_cast<uint16_t *>(C), M, N);
    return hipGetLastError();
}

}  // namespace ssg
