// Device helpers shared by the gfx950 kernels of libssg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte global load / store through plain vector memory instructions.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }

// fp32 -> fp16 with round-to-nearest-even (the default rounding mode of the
// conversion instruction; not the round-toward-zero packed variant).
__device__ __forceinline__ uint32_t pack_half2_rne(float lo, float hi) {
    _Float16 a = (_Float16)lo;
    _Float16 b = (_Float16)hi;
    return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Maps a linear block id so that each of the 8 XCDs (which receive block ids
// round-robin) works on one contiguous range of the logical tile order, which
// keeps the operands a range shares inside that XCD's private L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
    constexpr int kXcd = 8;
    const int q = nblocks / kXcd, r = nblocks % kXcd;
    const int x = b % kXcd, s = b / kXcd;
    return x * q + (x < r ? x : r) + s;
}

}  // namespace ssg
