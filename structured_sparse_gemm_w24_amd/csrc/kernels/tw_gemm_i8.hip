// Tile-wise sparse GEMM, int8 in, int32 accumulate, for gfx950.
//
// The tile-wise format of "Accelerating Sparse DNN Models without
// Hardware-Support via Tile-Wise Sparsity" (condensed G-column tiles read
// through offset_k, written through offset_n) with the integer deployment of
// GPUSQ-ViT ("Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", abstract): int8 activations and weights, exact int32
// accumulation, then y = float(acc) * scale[n] (+ bias[n]) stored as fp32,
// fp16 or saturated int8 (or the raw int32 accumulators).
//
// Same structure as the fp16 kernel (one 8-wave workgroup per token block of
// 128 x tile, picked rows of the K-major At gathered by direct-to-LDS loads,
// a ring of stages, an LDS output window), with these int8 specifics:
//   * a stage is 64 picked rows (one v_mfma_i32_16x16x64_i8 k-step) of 128
//     bytes; 16-byte chunks are XOR-swizzled by row so that the 8 rows one
//     transposing read touches, and the 4 row groups of a wave, hit distinct
//     banks;
//   * the column operand comes from gfx950's 8-bit transposing LDS read:
//     within a 16-lane group, lane i receives byte i%8 of the 8-byte run read
//     by lane 2e + i/8 (e = 0..7).  Lanes aimed at rows k0 + j/2, tokens
//     8(j%2).. return 8 consecutive k of one token; two reads give the 16
//     bytes the instruction takes per lane;
//   * the instruction pairs byte j of lane 16g + r of both operands, so any
//     k labelling shared by the two operands is valid: lane (g, r) carries
//     k = 16g .. 16g+15 of the stage in both;
//   * every column of the tile window is written: pruned columns get the
//     epilogue of a zero accumulator (0 * scale[n] + bias[n]), kept columns
//     the tile product.
#include "common.h"
#include "launch.h"
#include "tw_common.h"

namespace ssg {

// A zero page: the source of padding rows and K tails.
__device__ __attribute__((aligned(256))) uint8_t g_tw8_zero[128];

namespace {

using namespace tw_detail;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Column operand of one 64-k step: two 8-bit transposing reads (k and k + 8
// rows, i.e. 1024 bytes apart), waited for in the same statement.
__device__ __forceinline__ void tw8_read_b(uint32_t addr, u32x2 &b0, u32x2 &b1) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %2\n\t"
        "ds_read_b64_tr_b8 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(b0), "=&v"(b1)
        : "v"(addr)
        : "memory");
}

// At stage: row r, 16-byte chunk c (16 tokens) -> stored chunk.
__device__ __forceinline__ int tw8_swz_a(int r, int c) { return c ^ ((r ^ (r >> 4)) & 7); }
// V_t stage: row j (channel), 16-byte chunk c (16 k) of a 64-byte row.
__device__ __forceinline__ int tw8_swz_w(int j, int c) { return c ^ ((j >> 1) & 3); }

// GMAX: widest tile; WPE: waves per SIMD the register allocation must allow.
template <int GMAX_, int WPE_>
struct Tw8Cfg {
    static constexpr int NW = 8, NT = NW * 64;
    static constexpr int BM = 128;   // tokens per work item (8 blocks of 16)
    static constexpr int BK = 64;    // picked rows per stage
    static constexpr int NB = 3;     // stage buffers
    static constexpr int KCAP = 512;  // offset_k entries held in LDS at a time
    static constexpr int GMAX = GMAX_;
    static constexpr int WPE = WPE_;
    static constexpr int A_STAGE = BK * BM;     // bytes
    static constexpr int W_STAGE = GMAX * BK;   // bytes
    static constexpr int STAGE = A_STAGE + W_STAGE;
    static constexpr int LA = A_STAGE / 1024 / NW;  // 1
    static constexpr int RING = NB * STAGE;
    static constexpr int IDX_OFF = RING;
    static constexpr int OFFN_OFF = IDX_OFF + KCAP * 4;
    static constexpr int SCALE_OFF = OFFN_OFF + GMAX * 4;  // scale of each kept column
    static constexpr int BIAS_OFF = SCALE_OFF + GMAX * 4;  // bias of each kept column
    static constexpr int FILL_OFF = BIAS_OFF + GMAX * 4;   // one window row of zero-accumulator outputs
    static constexpr int SMEM = FILL_OFF + GMAX * 4;
    static_assert(LA == 1, "one A load per wave per stage");
    static_assert(KCAP % NT == 0, "index chunk must split over the threads");
};

// fp32 y -> output bits of width OB (raw accumulators when EPI == OUT_I32).
template <int EPI>
__device__ __forceinline__ uint32_t tw8_out(float y) {
    if constexpr (EPI == OUT_F32) {
        return __builtin_bit_cast(uint32_t, y);
    } else if constexpr (EPI == OUT_F16) {
        return uint32_t(__builtin_bit_cast(uint16_t, (_Float16)y));
    } else {
        const float r = fminf(fmaxf(__builtin_rintf(y), -128.0f), 127.0f);
        return uint32_t(int32_t(r)) & 0xffu;
    }
}

// KGATH: M is not a multiple of 16, so a picked row's 16-byte pieces are not
// 16-byte aligned; each thread then gathers 16 consecutive tokens of one
// picked row through registers (byte loads, bounds-checked against M) into
// the LDS layout the direct-to-LDS loads produce.
template <class CF, int NJ, int EPI, bool KGATH>
__device__ __forceinline__ void tw8_item(uint8_t *smem, const int8_t *__restrict__ At, const int8_t *__restrict__ vt,
                                         const int32_t *__restrict__ offk, const int32_t *__restrict__ offn,
                                         const float *__restrict__ scale, const float *__restrict__ bias, int kt,
                                         int nt, int t, int G, int m0, uint8_t *__restrict__ Cw, int M, int N) {
    constexpr int NW = CF::NW, NT = CF::NT, BM = CF::BM, BK = CF::BK, NB = CF::NB, KCAP = CF::KCAP;
    constexpr int A_STAGE = CF::A_STAGE, STAGE = CF::STAGE;
    constexpr int OB = (EPI == OUT_F16) ? 2 : (EPI == OUT_I8 ? 1 : 4);  // output bytes
    int32_t *s_idx = reinterpret_cast<int32_t *>(smem + CF::IDX_OFF);
    int32_t *s_offn = reinterpret_cast<int32_t *>(smem + CF::OFFN_OFF);
    float *s_scale = reinterpret_cast<float *>(smem + CF::SCALE_OFF);
    float *s_bias = reinterpret_cast<float *>(smem + CF::BIAS_OFF);
    uint8_t *s_fill = smem + CF::FILL_OFF;  // packed output of a zero accumulator, G * OB bytes

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ld = (kt + 15) & ~15;
    const int lw = (NJ - wave + NW - 1) / NW;  // V_t loads per stage for this wave (NJ KiB in all)
    const int per_stage = (KGATH ? 0 : 1) + lw;  // direct-to-LDS loads per stage

    // per-column epilogue data: kept columns' scale and bias, and the output of a
    // zero accumulator for every window column
    if (tid < nt && tid < CF::GMAX) {
        const int n = t * G + offn[tid];
        s_offn[tid] = offn[tid];
        if constexpr (EPI != OUT_I32) {
            s_scale[tid] = scale[n];
            s_bias[tid] = bias ? bias[n] : 0.0f;
        }
    }
    if (tid < G) {
        uint32_t f = 0;
        if constexpr (EPI != OUT_I32) {
            float y = __fmul_rn(0.0f, scale[t * G + tid]);
            if (bias) y = __fadd_rn(y, bias[t * G + tid]);
            f = tw8_out<EPI>(y);
        }
        if constexpr (OB == 4) *reinterpret_cast<uint32_t *>(s_fill + tid * 4) = f;
        else if constexpr (OB == 2) *reinterpret_cast<uint16_t *>(s_fill + tid * 2) = uint16_t(f);
        else s_fill[tid] = uint8_t(f);
    }

    // A loads: rows 8*wave .. +7 of the stage; lane -> row 8*wave + lane/8, stored chunk lane%8.
    const int a_row = 8 * wave + (lane >> 3), a_pos = lane & 7;
    // W loads: rows 16q .. 16q+15; lane -> row 16q + lane/4, stored chunk lane%4.
    const int w_sub = lane >> 2, w_pos = lane & 3;

    i32x4 acc[NJ > 0 ? NJ : 1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = i32x4{0, 0, 0, 0};

    const int tok_mb = wave * 16;  // this wave's 16 tokens: chunk `wave` of every row
    const int g16 = lane >> 4, j16 = lane & 15;
    // transposing-read address in a stage: row 16*g16 + j16/2, byte 8*(j16%2) of chunk `wave`
    const int rb = 16 * g16 + (j16 >> 1);
    const uint32_t b_off = rb * BM + tw8_swz_a(rb, wave) * 16 + 8 * (j16 & 1);
    const uint32_t smem_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

    if constexpr (NJ > 0) {
        for (int cb = 0; cb < kt; cb += KCAP) {
            const int ck = min(KCAP, kt - cb);
            if (cb > 0) __syncthreads();
            {
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
                if constexpr (KGATH) {
                    static_assert(BK * BM == NT * 16, "gather mapping: one 16-token piece per thread");
                    // thread -> picked row r, stored 16-byte chunk p (source chunk tw8_swz_a(r, p))
                    const int r = tid / (BM / 16), p = tid % (BM / 16);
                    const int kk = s * BK + r;
                    const int tok = m0 + tw8_swz_a(r, p) * 16;
                    const bool row_ok = kk < ck;
                    const int64_t rb = row_ok ? int64_t(s_idx[kk]) * M : 0;
                    uint32_t w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t x = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = tok + 4 * q + e;
                            const uint32_t b = (row_ok && m < M) ? uint32_t(uint8_t(At[rb + m])) : 0u;
                            x |= b << (8 * e);
                        }
                        w[q] = x;
                    }
                    *reinterpret_cast<u32x4 *>(base + r * BM + p * 16) = u32x4{w[0], w[1], w[2], w[3]};
                } else {
                    const int kk = s * BK + a_row;
                    const int tok = m0 + tw8_swz_a(a_row, a_pos) * 16;
                    const void *src = g_tw8_zero;
                    if (kk < ck && tok < M) src = At + int64_t(s_idx[kk]) * M + tok;
                    tw_dma16(src, base + wave * 1024);
                }
                for (int j = 0; j < lw; ++j) {
                    const int q = j * NW + wave;
                    const int row = 16 * q + w_sub;
                    const int k = cb + s * BK + tw8_swz_w(row, w_pos) * 16;
                    const void *src = g_tw8_zero;
                    if (row < nt && k < ld) src = vt + int64_t(row) * ld + k;
                    tw_dma16(src, base + A_STAGE + q * 1024);
                }
            };

            for (int s = 0; s < NB - 1 && s < S; ++s) issue(s);
            for (int s = 0; s < S; ++s) {
                tw_wait_barrier(min(NB - 2, S - 1 - s) * per_stage);
                if (s + NB - 1 < S) issue(s + NB - 1);
                const uint32_t stage_off = (s % NB) * STAGE;
                const uint8_t *bW = smem + stage_off + A_STAGE;
                u32x2 b0, b1;
                tw8_read_b(smem_addr + stage_off + b_off, b0, b1);
                const i32x4 bv = __builtin_bit_cast(i32x4, __builtin_shufflevector(b0, b1, 0, 1, 2, 3));
                // V_t fragments in batches of at most 8 column blocks (register budget of wide tiles)
                constexpr int JC = NJ > 8 ? 8 : NJ;
#pragma unroll
                for (int j0 = 0; j0 < NJ; j0 += JC) {
                    i32x4 wv[JC];
#pragma unroll
                    for (int jj = 0; jj < JC; ++jj) {
                        const int row = (j0 + jj) * 16 + j16;
                        if (j0 + jj < NJ)
                            wv[jj] = *reinterpret_cast<const i32x4 *>(bW + row * BK + tw8_swz_w(row, g16) * 16);
                    }
#pragma unroll
                    for (int jj = 0; jj < JC; ++jj)
                        if (j0 + jj < NJ)
                            acc[j0 + jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[jj], bv, acc[j0 + jj], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: output window [tokens][G] in LDS (aliases the stage ring),
    // rows padded by 16 bytes; fp32 / int32 windows take two 64-token passes
    constexpr int WROW = CF::GMAX * OB + 16;
    constexpr int PASSES = (BM * WROW <= CF::RING) ? 1 : 2;
    constexpr int PT = BM / PASSES;  // tokens per pass
    static_assert(PT * WROW <= CF::RING, "output window must fit in the stage ring");
    const int rowc = G * OB / 16;  // 16-byte chunks per window row
    uint8_t *win = smem;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        __syncthreads();
        // prefill every row with the zero-accumulator output row, 16 bytes at a time
        for (int c = tid; c < PT * rowc; c += NT) {
            const int row = c / rowc, ch = c % rowc;
            *reinterpret_cast<u32x4 *>(win + row * WROW + ch * 16) = *reinterpret_cast<const u32x4 *>(s_fill + ch * 16);
        }
        __syncthreads();
        // acc[jb] lane (g16, j16) holds D[j = 16jb + 4*g16 + i][token = tok_mb + j16]
        if (tok_mb / PT == ps) {
            const int wr = tok_mb % PT + j16;  // window row
#pragma unroll
            for (int jb = 0; jb < NJ; ++jb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = jb * 16 + 4 * g16 + i;
                    if (j < nt) {
                        uint8_t *p = win + wr * WROW + s_offn[j] * OB;
                        if constexpr (EPI == OUT_I32) {
                            *reinterpret_cast<int32_t *>(p) = acc[jb][i];
                        } else {
                            float y = __fmul_rn(float(acc[jb][i]), s_scale[j]);
                            if (bias) y = __fadd_rn(y, s_bias[j]);
                            const uint32_t o = tw8_out<EPI>(y);
                            if constexpr (OB == 4) *reinterpret_cast<uint32_t *>(p) = o;
                            else if constexpr (OB == 2) *reinterpret_cast<uint16_t *>(p) = uint16_t(o);
                            else *p = uint8_t(o);
                        }
                    }
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < PT * rowc; c += NT) {
            const int row = c / rowc, ch = c % rowc;
            const int m = m0 + ps * PT + row;
            if (m < M)
                tw_store16(Cw + (int64_t(m) * N) * OB + ch * 16,
                           *reinterpret_cast<const u32x4 *>(win + row * WROW + ch * 16));
        }
    }
}

template <class CF, int EPI, bool KGATH>
__global__ void __launch_bounds__(CF::NT) __attribute__((amdgpu_waves_per_eu(CF::WPE)))
tw_gemm_i8_kernel(const int8_t *__restrict__ At, const int8_t *__restrict__ vals, const int32_t *__restrict__ offset_k,
                  const int32_t *__restrict__ offset_n, const int32_t *__restrict__ v_ptr,
                  const int32_t *__restrict__ k_ptr, const int32_t *__restrict__ n_ptr,
                  const int32_t *__restrict__ tile_order, int T, int G, const float *__restrict__ scale,
                  const float *__restrict__ bias, uint8_t *__restrict__ C, int M, int N) {
    constexpr int OB = (EPI == OUT_F16) ? 2 : (EPI == OUT_I8 ? 1 : 4);
    __shared__ __attribute__((aligned(1024))) uint8_t smem[CF::SMEM];
    const int n_mb = (M + CF::BM - 1) / CF::BM;
    const int item = xcd_remap(blockIdx.x, n_mb * T);
    const int mb = item / T;
    const int t = tile_order[item % T];
    const int kp0 = k_ptr[t], kt = k_ptr[t + 1] - kp0;
    const int np0 = n_ptr[t], nt = n_ptr[t + 1] - np0;
    const int8_t *vt = vals + v_ptr[t];
    uint8_t *Cw = C + int64_t(t) * G * OB;
    const int m0 = mb * CF::BM;
    // (a tile of at most GMAX columns has at most GMAX/16 column blocks)
    switch ((nt + 15) >> 4) {
#define TW8_CASE(J)                                                                                               \
    case J:                                                                                                       \
        if constexpr (J <= CF::GMAX / 16)                                                                         \
            tw8_item<CF, J, EPI, KGATH>(smem, At, vt, offset_k + kp0, offset_n + np0, scale, bias, kt, nt, t, G, \
                                        m0, Cw, M, N);                                                            \
        break;
        TW8_CASE(0) TW8_CASE(1) TW8_CASE(2) TW8_CASE(3) TW8_CASE(4) TW8_CASE(5) TW8_CASE(6) TW8_CASE(7) TW8_CASE(8)
        TW8_CASE(9) TW8_CASE(10) TW8_CASE(11) TW8_CASE(12) TW8_CASE(13) TW8_CASE(14) TW8_CASE(15) TW8_CASE(16)
#undef TW8_CASE
        default: break;
    }
}

// Tiles up to 128 columns: 52 KiB of LDS and at most 85 VGPRs, three
// workgroups per CU.  Wider tiles (up to 256 columns): 78 KiB, two per CU.
using Tw8Prod = Tw8Cfg<128, 6>;
using Tw8Wide = Tw8Cfg<256, 4>;

template <class CF, bool KGATH>
hipError_t launch_i8_cfg(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                         const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr, const int32_t *tile_order,
                         int T, int G, const float *scale, const float *bias, void *C, int out, int M, int N,
                         hipStream_t st) {
    const int n_mb = (M + CF::BM - 1) / CF::BM;
    auto kern = out == OUT_I32 ? tw_gemm_i8_kernel<CF, OUT_I32, KGATH>
              : out == OUT_F32 ? tw_gemm_i8_kernel<CF, OUT_F32, KGATH>
              : out == OUT_F16 ? tw_gemm_i8_kernel<CF, OUT_F16, KGATH>
                               : tw_gemm_i8_kernel<CF, OUT_I8, KGATH>;
    hipLaunchKernelGGL(kern, dim3(n_mb * T), dim3(CF::NT), 0, st, static_cast<const int8_t *>(At),
                       static_cast<const int8_t *>(vals), offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G,
                       scale, bias, static_cast<uint8_t *>(C), M, N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tw_i8(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                        const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr, const int32_t *tile_order,
                        int T, int G, const float *scale, const float *bias, void *C, int out, int M, int N,
                        hipStream_t st) {
    const bool gath = M % 16 != 0;
    if (G > Tw8Prod::GMAX) {
        if (gath)
            return launch_i8_cfg<Tw8Wide, true>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G,
                                                scale, bias, C, out, M, N, st);
        return launch_i8_cfg<Tw8Wide, false>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G,
                                             scale, bias, C, out, M, N, st);
    }
    if (gath)
        return launch_i8_cfg<Tw8Prod, true>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G,
                                            scale, bias, C, out, M, N, st);
    return launch_i8_cfg<Tw8Prod, false>(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G, scale,
                                         bias, C, out, M, N, st);
}

}  // namespace ssg
