// Matrix-core rate probe for the bench (a separate library; libssg never
// loads it).  The roofline fractions of the MFMA-bound GEMMs are quoted against
// MI355X's published dense peaks, which assume the nominal 2.4 GHz shader
// clock; the clock is power-managed, so the bench also measures the rate this
// device actually sustains for each matrix instruction the GEMMs use, and
// quotes the fractions against that as well.
//
// Every wave issues the same instruction back to back on four independent
// accumulators (enough independent chains per SIMD that the issue rate, not
// the dependency latency, sets the time), with four waves per SIMD on every CU.
// The operand values do not matter to the rate; the accumulators are summed
// into `out` so the work is not dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));

// 2-bit positions (0, 1) in every group of four: a valid sparse index operand
constexpr int kIdx = 0x44444444;
constexpr int kAcc = 4;

// KIND 0: dense fp16 32x32x16; 1: 2:4 fp16 32x32x32; 2: dense int8 32x32x32;
// 3: 2:4 int8 32x32x64 (the instructions of the library's GEMM kinds).
template <int KIND>
__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float *__restrict__ out) {
    const int t = threadIdx.x;
    float s = 0.f;
    if constexpr (KIND == 0 || KIND == 1) {
        half16 b;
        for (int e = 0; e < 16; ++e) b[e] = (_Float16)(float((t + e) & 7) * 0.125f);
        const half8 a = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
        floatx16 acc[kAcc];
        for (int j = 0; j < kAcc; ++j) acc[j] = floatx16{};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j) {
                if constexpr (KIND == 0) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[j], 0, 0, 0);
                else acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, acc[j], kIdx, 0, 0);
            }
        }
        for (int j = 0; j < kAcc; ++j)
            for (int e = 0; e < 16; ++e) s += acc[j][e];
    } else {
        intx8 b;
        for (int e = 0; e < 8; ++e) b[e] = (t + e) & 0x01010101;
        const intx4 a = __builtin_shufflevector(b, b, 0, 1, 2, 3);
        intx16 acc[kAcc];
        for (int j = 0; j < kAcc; ++j) acc[j] = intx16{};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j) {
                if constexpr (KIND == 2) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[j], 0, 0, 0);
                else acc[j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc[j], kIdx, 0, 0);
            }
        }
        for (int j = 0; j < kAcc; ++j)
            for (int e = 0; e < 16; ++e) s += float(acc[j][e]);
    }
    out[blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads, each wave issuing iters * 4
// instructions of `kind` (0..3, as above); `out` holds blocks * 256 floats of
// device memory.  Returns the HIP status of the launch.  Dense-equivalent
// operations per instruction: 32768 (kind 0), 65536 (1, 2), 131072 (3).
extern "C" __attribute__((visibility("default"))) int ssg_bench_mfma_peak(int kind, int iters, int blocks,
                                                                         float *out, void *stream) {
    if (kind < 0 || kind > 3 || iters < 1 || blocks < 1 || !out) return int(hipErrorInvalidValue);
    const hipStream_t st = hipStream_t(stream);
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(256), 0, st, iters, out); break;
        case 1: hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(256), 0, st, iters, out); break;
        case 2: hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(256), 0, st, iters, out); break;
        default: hipLaunchKernelGGL(mfma_peak_kernel<3>, dim3(blocks), dim3(256), 0, st, iters, out); break;
    }
    return int(hipGetLastError());
}
