// attend_common.h -- helpers shared by the attention kernels (bf16, MXFP8
// entries, FP8 arithmetic): LDS address space, explicit vmcnt waits, the
// block barrier without a memory fence, and lane-half exchanges.
#pragma once
#include "common.h"

namespace csa {

#define CSA_LDS __attribute__((address_space(3)))

// Maximum / sum of a value over lanes l and l ^ 32 (a VALU lane swap, so it
// does not queue behind LDS reads)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// vmcnt wait (other counters untouched) leaving n copies in flight (n <= 63)
#define CSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x3f70 | ((n) & 15) | (((n) >> 4) << 14))

// Block barrier without a memory fence: LDS writes are drained explicitly
// and the copies each wave waited for are complete, so no outstanding copy
// into another stage is waited for here.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// vmcnt wait leaving n (wave-uniform, 0 .. 63) copies in flight; larger n
// waits for every copy
__device__ __forceinline__ void wait_vm_leaving(int n) {
    switch (n) {
#define CSA_WCASE(x) case x: CSA_WAIT_VM(x); break;
#define CSA_WCASE8(x) CSA_WCASE(x) CSA_WCASE(x + 1) CSA_WCASE(x + 2) CSA_WCASE(x + 3) \
        CSA_WCASE(x + 4) CSA_WCASE(x + 5) CSA_WCASE(x + 6) CSA_WCASE(x + 7)
        CSA_WCASE(1) CSA_WCASE(2) CSA_WCASE(3) CSA_WCASE(4) CSA_WCASE(5) CSA_WCASE(6)
        CSA_WCASE(7) CSA_WCASE8(8) CSA_WCASE8(16) CSA_WCASE8(24) CSA_WCASE8(32)
        CSA_WCASE8(40) CSA_WCASE8(48) CSA_WCASE8(56)
#undef CSA_WCASE8
#undef CSA_WCASE
        default: CSA_WAIT_VM(0); break;
    }
}

}  // namespace csa
