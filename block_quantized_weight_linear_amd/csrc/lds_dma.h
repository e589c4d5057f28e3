// Direct-to-LDS copies and explicit vector-memory waits (gfx950), shared by the
// kernels that stage activations through LDS while weights stream into registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8k {

// s_waitcnt with only vmcnt limited to n (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One wave-wide direct-to-LDS copy: lane l copies 16 bytes from its src to
// lds + 16*l (lds wave-uniform, taken from M0 when the load issues).  Written as inline
// assembly so that the compiler does not serialize it against LDS reads of the other
// buffer: the caller waits for it with wait_vmcnt (it counts as one vector-memory load,
// retired in order) and a barrier.  M0 is saved and restored around it; a write of M0
// needs one wait state before an LDS-DMA load reads it.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base));
}

}  // namespace q8k
