// lds_ring.h -- device helpers shared by the kernels whose K stages are copied
// global -> LDS by the load units (global_load_lds) into rings (gfx950).
#pragma once
#include "common.h"

// an LDS (address space 3) pointer, the destination operand of global_load_lds
#define FT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

namespace ft {

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
// the same with a run-time count (capped at N)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm_upto(int n) {
    if constexpr (N <= 0) {
        wait_vm_lgkm<0>();
    } else {
        if (n >= N) wait_vm_lgkm<N>();
        else wait_vm_lgkm_upto<N - 1>(n);
    }
}

}  // namespace ft
