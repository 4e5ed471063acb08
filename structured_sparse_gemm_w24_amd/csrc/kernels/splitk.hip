// Split-K reduction for the GEMMs of gemm.hip.
//
// A split launch leaves, for split s = 0 .. splits-1, the raw accumulators of
// K-stage range s in slice s of the workspace ([splits][M][N], 4 bytes per
// element: fp32 for the fp16 kinds, int32 for the int8 kinds).  This kernel
// sums the slices in split order and applies the epilogue of the unsplit
// kernels:
//   * fp16 kinds: the fp32 sum rounded to fp16 (nearest even);
//   * int8 kinds: the int32 sum (exact: it is the full accumulator), raw, or
//     y = float(acc) * scale[n] (+ bias[n]), each step rounded to nearest
//     even, stored as fp32, fp16 or int8 (rounded to nearest even, saturated),
//     the same operations in the same order as the GEMM epilogue, so int8
//     results are bit-identical to an unsplit launch.
// Each thread handles 4 consecutive elements of a row (N is a multiple of 64):
// 16-byte loads per split, one 16 / 8 / 4-byte store.  Memory-bound:
// splits * M * N * 4 bytes read, M * N * out_bytes written.
#include "common.h"
#include "launch.h"

namespace ssg {
namespace {

template <bool I8, int OUT>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const uint8_t *__restrict__ ws, int splits, const float *__restrict__ scale,
                     const float *__restrict__ bias, void *__restrict__ C, int64_t groups, int N) {
    const int64_t slice = groups * 16;  // bytes per split slice
    for (int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < groups;
         g += int64_t(gridDim.x) * blockDim.x) {
        const uint8_t *p = ws + g * 16;
        if constexpr (!I8) {
            floatx4 acc = __builtin_bit_cast(floatx4, ld16(p));
            for (int s = 1; s < splits; ++s) {
                const floatx4 v = __builtin_bit_cast(floatx4, ld16(p + s * slice));
                acc.x = __fadd_rn(acc.x, v.x);
                acc.y = __fadd_rn(acc.y, v.y);
                acc.z = __fadd_rn(acc.z, v.z);
                acc.w = __fadd_rn(acc.w, v.w);
            }
            st8(reinterpret_cast<uint8_t *>(C) + g * 8,
                u32x2{pack_half2_rne(acc.x, acc.y), pack_half2_rne(acc.z, acc.w)});
        } else {
            // unsigned adds: two's-complement wrap-around, as the matrix instructions accumulate
            u32x4 sum = ld16(p);
            for (int s = 1; s < splits; ++s) sum += ld16(p + s * slice);
            const intx4 acc = __builtin_bit_cast(intx4, sum);
            if constexpr (OUT == OUT_I32) {
                st16(reinterpret_cast<uint8_t *>(C) + g * 16, __builtin_bit_cast(u32x4, acc));
            } else {
                const int n = int((g * 4) % N);
                const floatx4 sc = *reinterpret_cast<const floatx4 *>(scale + n);
                floatx4 f;
                f.x = __fmul_rn(float(acc.x), sc.x);
                f.y = __fmul_rn(float(acc.y), sc.y);
                f.z = __fmul_rn(float(acc.z), sc.z);
                f.w = __fmul_rn(float(acc.w), sc.w);
                if (bias) {
                    const floatx4 bi = *reinterpret_cast<const floatx4 *>(bias + n);
                    f.x = __fadd_rn(f.x, bi.x);
                    f.y = __fadd_rn(f.y, bi.y);
                    f.z = __fadd_rn(f.z, bi.z);
                    f.w = __fadd_rn(f.w, bi.w);
                }
                if constexpr (OUT == OUT_F32) {
                    st16(reinterpret_cast<uint8_t *>(C) + g * 16, __builtin_bit_cast(u32x4, f));
                } else if constexpr (OUT == OUT_F16) {
                    st8(reinterpret_cast<uint8_t *>(C) + g * 8, u32x2{pack_half2_rne(f.x, f.y), pack_half2_rne(f.z, f.w)});
                } else {
                    auto q8 = [](float y) -> uint32_t {
                        const float r = fminf(fmaxf(__builtin_rintf(y), -128.0f), 127.0f);
                        return uint32_t(int32_t(r)) & 0xffu;
                    };
                    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(C) + g * 4) =
                        q8(f.x) | (q8(f.y) << 8) | (q8(f.z) << 16) | (q8(f.w) << 24);
                }
            }
        }
    }
}

template <bool I8, int OUT>
hipError_t reduce(const void *ws, int splits, const float *scale, const float *bias, void *C, int M, int N,
                  hipStream_t st) {
    const int64_t groups = int64_t(M) * N / 4;
    const int64_t want = (groups + 255) / 256;
    const int blocks = int(want < 4096 ? want : 4096);
    hipLaunchKernelGGL((splitk_reduce_kernel<I8, OUT>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint8_t *>(ws), splits, scale, bias, C, groups, N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_reduce(const void *ws, int splits, bool i8, const float *scale, const float *bias, void *C,
                                int out, int M, int N, hipStream_t st) {
    if (!i8) return reduce<false, OUT_F16>(ws, splits, nullptr, nullptr, C, M, N, st);
    switch (out) {
        case OUT_I32: return reduce<true, OUT_I32>(ws, splits, nullptr, nullptr, C, M, N, st);
        case OUT_F32: return reduce<true, OUT_F32>(ws, splits, scale, bias, C, M, N, st);
        case OUT_F16: return reduce<true, OUT_F16>(ws, splits, scale, bias, C, M, N, st);
        default: return reduce<true, OUT_I8>(ws, splits, scale, bias, C, M, N, st);
    }
}

}  // namespace ssg
