// Test-only probe: runs single matrix instructions with caller-chosen lane
// inputs so the tests can check the operand, index and accumulator layouts
// that the GEMM kernels assume.  Each block is one wave and one experiment:
// lane l of experiment e reads its A elements at a[(e*64 + l)*NA ..], its B
// elements at b[(e*64 + l)*NB ..], its index word at idx[e*64 + l], and
// writes its accumulator registers to d[(e*64 + l)*ND ..].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef int i16v __attribute__((ext_vector_type(16)));

#define PROBE_API extern "C" __attribute__((visibility("default")))

// op 0: smfmac f32 32x32x32 f16   (A 8 halves, B 16 halves, D 16 floats)
// op 1: smfmac i32 32x32x64 i8    (A 16 bytes, B 32 bytes, D 16 ints)
// op 2: mfma f32 32x32x16 f16     (A 8 halves, B 8 halves, D 16 floats)
// op 3: mfma f32 16x16x32 f16     (A 8 halves, B 8 halves, D 4 floats)
// op 4: mfma i32 32x32x32 i8      (A 16 bytes, B 16 bytes, D 16 ints)
__global__ void __launch_bounds__(64) probe_kernel(int op, const void *a, const void *b, const int *idx, void *d) {
    const int g = blockIdx.x * 64 + threadIdx.x;
    if (op == 0) {
        const h8 av = reinterpret_cast<const h8 *>(a)[g];
        const h16 bv = reinterpret_cast<const h16 *>(b)[g];
        f16v acc = {};
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_f16(av, bv, acc, idx[g], 0, 0);
        reinterpret_cast<f16v *>(d)[g] = acc;
    } else if (op == 1) {
        const i4 av = reinterpret_cast<const i4 *>(a)[g];
        const i8v bv = reinterpret_cast<const i8v *>(b)[g];
        i16v acc = {};
        acc = __builtin_amdgcn_smfmac_i32_32x32x64_i8(av, bv, acc, idx[g], 0, 0);
        reinterpret_cast<i16v *>(d)[g] = acc;
    } else if (op == 2) {
        const h8 av = reinterpret_cast<const h8 *>(a)[g];
        const h8 bv = reinterpret_cast<const h8 *>(b)[g];
        f16v acc = {};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
        reinterpret_cast<f16v *>(d)[g] = acc;
    } else if (op == 3) {
        const h8 av = reinterpret_cast<const h8 *>(a)[g];
        const h8 bv = reinterpret_cast<const h8 *>(b)[g];
        f4 acc = {};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
        reinterpret_cast<f4 *>(d)[g] = acc;
    } else if (op == 4) {
        const i4 av = reinterpret_cast<const i4 *>(a)[g];
        const i4 bv = reinterpret_cast<const i4 *>(b)[g];
        i16v acc = {};
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc, 0, 0, 0);
        reinterpret_cast<i16v *>(d)[g] = acc;
    }
}

// Launches `experiments` one-wave experiments of instruction `op` on `stream`
// and waits for them.  Buffers are device memory sized for the op (see above).
PROBE_API int probe_run(int op, int experiments, const void *a, const void *b, const int *idx, void *d,
                        void *stream) {
    if (op < 0 || op > 4 || experiments <= 0 || !a || !b || !idx || !d) return 1;
    hipLaunchKernelGGL(probe_kernel, dim3(experiments), dim3(64), 0, hipStream_t(stream), op, a, b, idx, d);
    if (hipGetLastError() != hipSuccess) return 2;
    return hipStreamSynchronize(hipStream_t(stream)) == hipSuccess ? 0 : 3;
}
