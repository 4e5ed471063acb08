// Helpers shared by the tile-wise kernels (fp16 and int8).
#pragma once

#include "common.h"

namespace ssg {
namespace tw_detail {

typedef __attribute__((address_space(3))) void *tw_lds_ptr;

// Direct-to-LDS load: lane i writes its 16 bytes to wave_base + 16*i.
__device__ __forceinline__ void tw_dma16(const void *g, uint8_t *wave_base) {
    __builtin_amdgcn_global_load_lds(g, (tw_lds_ptr)wave_base, 16, 0, 0);
}

// Output stores are nontemporal: C is written once and not read back by the
// kernel, and streaming it past L2 avoids write-backs at the kernel's end.
__device__ __forceinline__ void tw_store16(void *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Wait until at most n of this wave's direct-to-LDS loads are outstanding and
// its LDS reads have completed, then synchronise the workgroup.
__device__ __forceinline__ void tw_wait_barrier(int n) {
    switch (n) {
#define TW_WAIT(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        TW_WAIT(1) TW_WAIT(2) TW_WAIT(3) TW_WAIT(4) TW_WAIT(5) TW_WAIT(6) TW_WAIT(7)
        TW_WAIT(8) TW_WAIT(9) TW_WAIT(10) TW_WAIT(11) TW_WAIT(12)
#undef TW_WAIT
        default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    }
}

}  // namespace tw_detail
}  // namespace ssg
