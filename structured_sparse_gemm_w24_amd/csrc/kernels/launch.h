// Internal launch entry points of the gfx950 kernels (not exported).
// Arguments are validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssg {

// int8 GEMM output kinds (the values of the C-ABI's SSG_OUT_* constants)
enum OutKind { OUT_I32 = 0, OUT_F32 = 1, OUT_F16 = 2, OUT_I8 = 3 };

hipError_t launch_dense_f16(const void *A, const void *Wt, void *C, int M, int N, int K, hipStream_t st);
hipError_t launch_dense_i8(const void *A, const void *Wt, const float *scale, const float *bias, void *C,
                           int out, int M, int N, int K, hipStream_t st);
hipError_t launch_w24_f16(const void *A, const void *vals, const uint32_t *meta, void *C, int M, int N,
                          int K, hipStream_t st);
hipError_t launch_w24_i8(const void *A, const void *vals, const uint32_t *meta, const float *scale,
                         const float *bias, void *C, int out, int M, int N, int K, hipStream_t st);
// Tiles tile_order[t_first .. t_first + t_count); out_t: C is written
// transposed, Ct [N][M]; a_rowmajor: the A operand is row-major [M][K]
// instead of K-major At [K][M]; narrow: every tile keeps at most 64 columns
// (the narrow-tile configurations; a wider tile's window comes out NaN).
hipError_t launch_tw_f16(const void *At, const void *vals, const int32_t *offset_k,
                         const int32_t *offset_n, const int32_t *v_ptr, const int32_t *k_ptr,
                         const int32_t *n_ptr, const int32_t *tile_order, int t_first, int t_count,
                         int G, bool out_t, bool a_rowmajor, bool narrow, void *C, int M, int N, int K,
                         hipStream_t st);
// int8 tile-wise GEMM (K-major int8 At, condensed int8 tiles), epilogue as
// the int8 GEMMs' OUT_* kinds.
hipError_t launch_tw_i8(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                        const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                        const int32_t *tile_order, int T, int G, const float *scale, const float *bias,
                        void *C, int out, int M, int N, hipStream_t st);
hipError_t launch_transpose_f16(const void *A, void *At, int M, int K, hipStream_t st);

// Split K: kind is a GEMM kind (0 dense fp16, 1 2:4 fp16, 2 dense int8, 3 2:4
// int8).  The split launch writes split s's raw accumulators (fp32 / int32)
// to slice s of ws ([splits][M][N], 4 bytes each); the reduce launch sums the
// slices in split order and applies the kind's epilogue (out: OUT_* for int8).
hipError_t launch_gemm_partials(int kind, const void *A, const void *W, const uint32_t *meta, void *ws, int M,
                                int N, int K, int splits, hipStream_t st);
hipError_t launch_splitk_reduce(const void *ws, int splits, bool i8, const float *scale, const float *bias,
                                void *C, int out, int M, int N, hipStream_t st);
// K splits worth taking for a kind and shape (1 = do not split); a host-only
// rule from the tile choice, the resident workgroups per CU and the K stages.
int suggest_splits(int kind, int M, int N, int K);
// tile rows x columns the GEMM launchers pick for a kind (0-3) and shape
void tile_choice(int kind, int M, int N, int K, int *bm, int *bn);
// K stages (one per 128 bytes of an A row) for a kind and K.
inline int gemm_k_stages(int kind, int K) { return (kind == 2 || kind == 3) ? K / 128 : K / 64; }

}  // namespace ssg
