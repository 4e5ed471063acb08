// Explicit transpose At[k][m] = A[m][k] (fp16) -- the "explicit transpose"
// variant in the tile-wise slides ("Accelerating Sparse DNN Models without
// Hardware-Support via Tile-Wise Sparsity", transpose optimisation), which
// makes the rows picked by offset_k contiguous.
//
// A wave owns a 64 (m) x 64 (k) block; lane (mb, kb) = (lane / 8, lane % 8)
// loads the 8x8 sub-block at rows m0 + 8*mb .. +7, columns k0 + 8*kb .. +7
// (eight 16-byte loads; the 8 lanes of one mb read a full 128-byte line of a
// row), transposes it in registers with byte permutes and stores eight
// 16-byte rows of At (the 8 lanes of one kb write a full 128-byte line).
// HBM-bound: 2 * M * K * 2 bytes per call.
#include "common.h"
#include "launch.h"

namespace ssg {

__global__ void __launch_bounds__(256) transpose_f16_kernel(const uint16_t *__restrict__ A, uint16_t *__restrict__ At,
                                                            int M, int K) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // workgroup block: 128 (m) x 128 (k), waves in a 2 x 2 arrangement
    const int m0 = blockIdx.y * 128 + (wave & 1) * 64 + (lane >> 3) * 8;
    const int k0 = blockIdx.x * 128 + (wave >> 1) * 64 + (lane & 7) * 8;
    if (m0 >= M || k0 >= K) return;
    u32x4 r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (m0 + j < M) ? ld16(A + int64_t(m0 + j) * K + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (k0 + i >= K) break;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
        o.x = __builtin_amdgcn_perm(r[1][i >> 1], r[0][i >> 1], sel);
        o.y = __builtin_amdgcn_perm(r[3][i >> 1], r[2][i >> 1], sel);
        o.z = __builtin_amdgcn_perm(r[5][i >> 1], r[4][i >> 1], sel);
        o.w = __builtin_amdgcn_perm(r[7][i >> 1], r[6][i >> 1], sel);
        st16(At + int64_t(k0 + i) * M + m0, o);
    }
}

hipError_t launch_transpose_f16(const void *A, void *At, int M, int K, hipStream_t st) {
    const dim3 grid((K + 127) / 128, (M + 127) / 128), block(256);
    hipLaunchKernelGGL(transpose_f16_kernel, grid, block, 0, st, static_cast<const uint16_t *>(A),
                       static_cast<uint16_t *>(At), M, K);
    return hipGetLastError();
}

}  // namespace ssg
