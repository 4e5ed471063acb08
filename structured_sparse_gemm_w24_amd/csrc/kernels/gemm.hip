// Dense and 2:4-sparse GEMM kernels for gfx950 (one skeleton, four kinds).
//
// C[M][N] = A[M][K] . W[K][N].  The 2:4 kinds read W from its compressed
// form (two kept values per group of four along K plus 2-bit positions,
// GPUSQ-ViT "Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", abstract) and feed the gfx950 sparse matrix instructions,
// whose sparse operand is the instruction's row operand.  W's sparsity runs
// along K inside an output column, so the kernels compute the transposed
// product C^T = W^T . A^T: instruction rows are output channels n (sparse
// operand: kept values of W^T row n), instruction columns are tokens m
// (dense operand: a row of A, K contiguous).  The hardware selects, per kept
// value, the matching activation by the 2-bit position; no software gather
// of A is needed.  The dense kinds run the same skeleton with the dense
// instruction so that the sparse-vs-dense comparison isolates the matrix
// instruction.
//
// Work decomposition
//   * workgroup = WM x WN waves; tile = BM tokens x BN channels with
//     BM = WM*TM*32, BN = WN*TN*32; every wave owns TM x TN 32x32 blocks;
//   * K advances in stages of 128 bytes of an A row (f16: 64 k, i8: 128 k);
//     each stage is staged global -> registers -> LDS, double-buffered in LDS
//     with one barrier per stage; the next stage's global loads are in flight
//     while the current one feeds the matrix cores;
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the 32 rows read by
//     one fragment load fall into distinct banks;
//   * block ids are remapped so each XCD works on a contiguous range of tiles
//     (grouped GM tile-rows at a time), which keeps shared A rows and W
//     columns in that XCD's L2.
//
// Instruction operand layouts (64-lane wave, h = lane / 32, r = lane % 32):
//   dense f16 32x32x16 : row-op lane holds k = 8h .. 8h+7 of its row r
//   dense i8  32x32x32 : k = 16h .. 16h+15
//   sparse f16 32x32x32: sparse row-op lane holds the 8 kept values of row r
//                        for k in [16h, 16h+16) (4 groups, ascending), slot c's
//                        two-bit position at bits 2c of the index operand; the
//                        dense column-op lane holds, as elements 0..7 and
//                        8..15, k = 8h .. 8h+7 and k = 16+8h .. 16+8h+7 of
//                        column r (measured on gfx950 with one-wave probes)
//   sparse i8 32x32x64 : sparse lane: 16 kept values for k in [32h, 32h+32),
//                        16 positions = 32 index bits; dense lane: elements
//                        0..15 = k 16h .., elements 16..31 = k 32+16h ..
//   accumulator        : lane holds rows 8*(i/4) + 4h + i%4 (i = 0..15) of
//                        column r
// The compressed pack stores slot j's position at bits 2*(j%16) of word j/16,
// which is exactly the index operand for these ranges, so meta words are fed
// to the instruction as stored (shifted by 16 bits for the upper f16 half).
#include "common.h"
#include "launch.h"

namespace ssg {

enum Kind { DENSE_F16 = 0, W24_F16 = 1, DENSE_I8 = 2, W24_I8 = 3 };
enum Epi { EPI_F16 = 0, EPI_I32 = 1, EPI_F32_SCALE = 2 };

template <int KIND>
struct KindTraits;

template <>
struct KindTraits<DENSE_F16> {
    static constexpr bool kSparse = false, kI8 = false;
    static constexpr int kWB = 128;  // W bytes per row per stage
    static constexpr int kMW = 0;    // meta words per row per stage
    static constexpr int kNI = 4;    // instructions per stage
};
template <>
struct KindTraits<W24_F16> {
    static constexpr bool kSparse = true, kI8 = false;
    static constexpr int kWB = 64, kMW = 2, kNI = 2;
};
template <>
struct KindTraits<DENSE_I8> {
    static constexpr bool kSparse = false, kI8 = true;
    static constexpr int kWB = 128, kMW = 0, kNI = 4;
};
template <>
struct KindTraits<W24_I8> {
    static constexpr bool kSparse = true, kI8 = true;
    static constexpr int kWB = 64, kMW = 4, kNI = 2;
};

// 16-byte chunk swizzles (see header comment).
__device__ __forceinline__ int swz128(int row, int col) { return col ^ ((row ^ (row >> 3)) & 7); }
__device__ __forceinline__ int swz64(int row, int col) { return col ^ (((row >> 1) ^ (row >> 3)) & 3); }
template <int WB>
__device__ __forceinline__ int swzw(int row, int col) {
    if constexpr (WB == 64) return swz64(row, col);
    else return swz128(row, col);
}

template <int KIND>
struct AccOf {
    using T = typename std::conditional<KindTraits<KIND>::kI8, intx16, floatx16>::type;
};

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

template <int KIND>
__device__ __forceinline__ void mma(typename AccOf<KIND>::T &acc, u32x4 w, u32x4 a0, u32x4 a1, uint32_t idx) {
    if constexpr (KIND == W24_F16) {
        union { u32x4 u[2]; half16 h; } b;
        b.u[0] = a0;
        b.u[1] = a1;
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_f16(__builtin_bit_cast(half8, w), b.h, acc, int(idx), 0, 0);
    } else if constexpr (KIND == W24_I8) {
        union { u32x4 u[2]; intx8 v; } b;
        b.u[0] = a0;
        b.u[1] = a1;
        acc = __builtin_amdgcn_smfmac_i32_32x32x64_i8(__builtin_bit_cast(intx4, w), b.v, acc, int(idx), 0, 0);
    } else if constexpr (KIND == DENSE_F16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, w), __builtin_bit_cast(half8, a0),
                                                      acc, 0, 0, 0);
    } else {
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(intx4, w), __builtin_bit_cast(intx4, a0),
                                                     acc, 0, 0, 0);
    }
}

template <int KIND, int EPI, int WM, int WN, int TM, int TN, int GM>
__global__ void __launch_bounds__(WM *WN * 64)
gemm_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ Wv, const uint32_t *__restrict__ meta,
            const float *__restrict__ scale, void *__restrict__ C, int M, int N, int K) {
    using KT = KindTraits<KIND>;
    using Acc = typename AccOf<KIND>::T;
    constexpr int NT = WM * WN * kWave;
    constexpr int BM = WM * TM * 32;
    constexpr int BN = WN * TN * 32;
    constexpr int WB = KT::kWB;
    constexpr int MW = KT::kMW;
    constexpr int SA = KT::kI8 ? 1 : 2;  // bytes per element
    constexpr int A_STAGE = BM * 128;
    constexpr int W_STAGE = BN * WB;
    constexpr int M_STAGE = MW > 0 ? MW * BN * 4 : 16;
    constexpr int CA = BM * 8 / NT;           // A chunks per thread per stage
    constexpr int CW = BN * (WB / 16) / NT;   // W chunks per thread per stage
    static_assert(CA * NT == BM * 8 && CW * NT == BN * (WB / 16), "tile does not split evenly");
    static_assert(BN <= NT || MW == 0, "meta load assumes one row per thread");

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][A_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][W_STAGE];
    __shared__ __attribute__((aligned(16))) uint32_t sM[2][M_STAGE / 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int h = lane >> 5, r = lane & 31;

    // ---- tile assignment: XCD-contiguous ranges, GM tile-rows per group
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int b = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int group = b / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_group = b % (GM * tiles_n);
    const int tile_m = first_m + in_group % gm;
    const int tile_n = in_group / gm;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int64_t a_row = int64_t(K) * SA;                  // bytes per A row
    const int64_t w_row = KT::kSparse ? a_row / 2 : a_row;  // bytes per W row
    const int64_t m_row = K / 32;                            // meta words per row
    const int S = int(a_row / 128);

    // ---- per-thread global source pointers (rows clamped into range)
    const uint8_t *ga[CA];
    int la[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int c = tid + i * NT, row = c >> 3, col = c & 7;
        ga[i] = A + int64_t(min(m0 + row, M - 1)) * a_row + col * 16;
        la[i] = row * 128 + swz128(row, col) * 16;
    }
    const uint8_t *gw[CW];
    int lw[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) {
        constexpr int CPR = WB / 16;
        const int c = tid + i * NT, row = c / CPR, col = c % CPR;
        gw[i] = Wv + int64_t(min(n0 + row, N - 1)) * w_row + col * 16;
        lw[i] = row * WB + swzw<WB>(row, col) * 16;
    }
    const uint32_t *gmeta = nullptr;
    if constexpr (MW > 0) gmeta = meta + int64_t(min(n0 + min(tid, BN - 1), N - 1)) * m_row;

    u32x4 ra[CA], rw[CW];
    uint32_t rm[MW > 0 ? MW : 1];

    auto load_stage = [&](int s) {
#pragma unroll
        for (int i = 0; i < CA; ++i) ra[i] = ld16(ga[i] + s * 128);
#pragma unroll
        for (int i = 0; i < CW; ++i) rw[i] = ld16(gw[i] + s * WB);
        if constexpr (MW == 2) {
            u32x2 v = ld8(gmeta + s * 2);
            rm[0] = v.x;
            rm[1] = v.y;
        } else if constexpr (MW == 4) {
            u32x4 v = ld16(gmeta + s * 4);
            rm[0] = v.x;
            rm[1] = v.y;
            rm[2] = v.z;
            rm[3] = v.w;
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4 *>(&sA[buf][la[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < CW; ++i) *reinterpret_cast<u32x4 *>(&sW[buf][lw[i]]) = rw[i];
        if constexpr (MW > 0) {
            if (tid < BN) {
#pragma unroll
                for (int w = 0; w < MW; ++w) sM[buf][w * BN + tid] = rm[w];
            }
        }
    };

    Acc acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = Acc{};

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int s = 0; s < S; ++s) {
        const int buf = s & 1;
        if (s + 1 < S) load_stage(s + 1);
        const uint8_t *bA = sA[buf];
        const uint8_t *bW = sW[buf];
        const uint32_t *bM = sM[buf];
#pragma unroll
        for (int kk = 0; kk < KT::kNI; ++kk) {
            u32x4 wf[TN];
            uint32_t idx[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int row = wn * TN * 32 + tn * 32 + r;
                wf[tn] = lds16(bW + row * WB + swzw<WB>(row, 2 * kk + h) * 16);
                if constexpr (KIND == W24_F16) idx[tn] = bM[kk * BN + row] >> (16 * h);
                else if constexpr (KIND == W24_I8) idx[tn] = bM[(2 * kk + h) * BN + row];
                else idx[tn] = 0;
            }
            u32x4 af0[TM], af1[TM];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const int row = wm * TM * 32 + tm * 32 + r;
                if constexpr (KT::kSparse) {
                    // two 16-byte pieces of the 64-byte window: bytes 16h.. and 32+16h..
                    af0[tm] = lds16(bA + row * 128 + swz128(row, 4 * kk + h) * 16);
                    af1[tm] = lds16(bA + row * 128 + swz128(row, 4 * kk + 2 + h) * 16);
                } else {
                    af0[tm] = lds16(bA + row * 128 + swz128(row, 2 * kk + h) * 16);
                    af1[tm] = af0[tm];
                }
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) mma<KIND>(acc[tn][tm], wf[tn], af0[tm], af1[tm], idx[tn]);
        }
        if (s + 1 < S) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds, per block and q = i/4, channels n..n+3 of token m
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int m = m0 + wm * TM * 32 + tm * 32 + r;
        if (m >= M) continue;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * TN * 32 + tn * 32 + q * 8 + h * 4;
                if (n >= N) continue;
                const int64_t off = int64_t(m) * N + n;
                if constexpr (EPI == EPI_F16) {
                    const floatx16 &v = acc[tn][tm];
                    u32x2 o;
                    o.x = pack_half2_rne(v[4 * q + 0], v[4 * q + 1]);
                    o.y = pack_half2_rne(v[4 * q + 2], v[4 * q + 3]);
                    st8(reinterpret_cast<uint16_t *>(C) + off, o);
                } else if constexpr (EPI == EPI_I32) {
                    const intx16 &v = acc[tn][tm];
                    u32x4 o;
                    o.x = uint32_t(v[4 * q + 0]);
                    o.y = uint32_t(v[4 * q + 1]);
                    o.z = uint32_t(v[4 * q + 2]);
                    o.w = uint32_t(v[4 * q + 3]);
                    st16(reinterpret_cast<int32_t *>(C) + off, o);
                } else {
                    const intx16 &v = acc[tn][tm];
                    const floatx4 sc = *reinterpret_cast<const floatx4 *>(scale + n);
                    floatx4 f;
                    f.x = __fmul_rn(float(v[4 * q + 0]), sc.x);
                    f.y = __fmul_rn(float(v[4 * q + 1]), sc.y);
                    f.z = __fmul_rn(float(v[4 * q + 2]), sc.z);
                    f.w = __fmul_rn(float(v[4 * q + 3]), sc.w);
                    st16(reinterpret_cast<float *>(C) + off, __builtin_bit_cast(u32x4, f));
                }
            }
        }
    }
}

template <int KIND, int EPI, int WM, int WN, int TM, int TN, int GM>
static hipError_t launch(const void *A, const void *Wv, const uint32_t *meta, const float *scale, void *C,
                         int M, int N, int K, hipStream_t st) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const int nb = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_kernel<KIND, EPI, WM, WN, TM, TN, GM>), dim3(nb), dim3(WM * WN * kWave), 0, st,
                       static_cast<const uint8_t *>(A), static_cast<const uint8_t *>(Wv), meta, scale, C, M, N, K);
    return hipGetLastError();
}

// Tile shape: 128 tokens x 256 channels, 4 waves of 64 tokens x 128 channels.
hipError_t launch_dense_f16(const void *A, const void *Wt, void *C, int M, int N, int K, hipStream_t st) {
    return launch<DENSE_F16, EPI_F16, 2, 2, 2, 4, 8>(A, Wt, nullptr, nullptr, C, M, N, K, st);
}

hipError_t launch_w24_f16(const void *A, const void *vals, const uint32_t *meta, void *C, int M, int N, int K,
                          hipStream_t st) {
    return launch<W24_F16, EPI_F16, 2, 2, 2, 4, 8>(A, vals, meta, nullptr, C, M, N, K, st);
}

hipError_t launch_dense_i8(const void *A, const void *Wt, const float *scale, void *C, int M, int N, int K,
                           hipStream_t st) {
    if (scale) return launch<DENSE_I8, EPI_F32_SCALE, 2, 2, 2, 4, 8>(A, Wt, nullptr, scale, C, M, N, K, st);
    return launch<DENSE_I8, EPI_I32, 2, 2, 2, 4, 8>(A, Wt, nullptr, nullptr, C, M, N, K, st);
}

hipError_t launch_w24_i8(const void *A, const void *vals, const uint32_t *meta, const float *scale, void *C,
                         int M, int N, int K, hipStream_t st) {
    if (scale) return launch<W24_I8, EPI_F32_SCALE, 2, 2, 2, 4, 8>(A, vals, meta, scale, C, M, N, K, st);
    return launch<W24_I8, EPI_I32, 2, 2, 2, 4, 8>(A, vals, meta, nullptr, C, M, N, K, st);
}

}  // namespace ssg
