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

// The same wait with a compiler memory barrier: nothing is moved across it, so LDS reads
// after it see what direct-to-LDS copies older than the limit wrote.
template <int N>
__device__ __forceinline__ void wait_vmcnt_mem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt_mem() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// 4352 contiguous bytes (4 x 1 KB with 16 bytes a lane, then 256 B with 4 bytes a lane)
// from src to lds .. lds + 4351, as five direct-to-LDS loads (five vmcnt events).  Only
// the first len bytes (len >= 16, a multiple of 4) are read: a lane whose bytes lie past
// them reads the last 16 (or 4) bytes instead, and what it writes is never used.  NT: the
// loads carry the non-temporal hint (streamed data that is read once).
constexpr int kLdsItemBytes = 4352;
template <bool NT = false>
__device__ __forceinline__ void lds_copy_4352(const uint8_t* src, int len, uint32_t lds, int lane) {
    const uint8_t* p[5];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int off = 1024 * c + 16 * lane;
        p[c] = src + (off <= len - 16 ? off : len - 16);
    }
    const int off4 = 4096 + 4 * lane;
    p[4] = src + (off4 <= len - 4 ? off4 : len - 4);
    uint32_t saved;
#define Q8K_LDS_COPY_4352(H)                                                                                 \
    asm volatile(                                                                                              \
        "s_mov_b32 %0, m0\n\t"                                                                                 \
        "s_mov_b32 m0, %6\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %1, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %7\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %2, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %8\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %3, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %9\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %4, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %10\n\t"                                                                                \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dword %5, off" H "\n\t"                                                               \
        "s_mov_b32 m0, %0"                                                                                     \
        : "=&s"(saved)                                                                                         \
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "s"(lds), "s"(lds + 1024), "s"(lds + 2048),    \
          "s"(lds + 3072), "s"(lds + 4096)                                                                     \
        : "memory")
    if constexpr (NT)
        Q8K_LDS_COPY_4352(" nt");
    else
        Q8K_LDS_COPY_4352("");
#undef Q8K_LDS_COPY_4352
}

// 4352 bytes into lds .. lds + 4351 from per-lane sources, as the same five direct-to-LDS
// loads (five vmcnt events): copy c < 4 moves 16 bytes from p[c] to lds + 1024c + 16*lane,
// copy 4 moves 4 bytes from p[4] to lds + 4096 + 4*lane.  The caller maps each destination
// to its source (a gather: the bytes may come from different rows).
template <bool NT = false>
__device__ __forceinline__ void lds_copy_4352_gather(const uint8_t* const (&p)[5], uint32_t lds) {
    uint32_t saved;
#define Q8K_LDS_GATHER_4352(H)                                                                               \
    asm volatile(                                                                                              \
        "s_mov_b32 %0, m0\n\t"                                                                                 \
        "s_mov_b32 m0, %6\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %1, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %7\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %2, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %8\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %3, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %9\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %4, off" H "\n\t"                                                             \
        "s_mov_b32 m0, %10\n\t"                                                                                \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dword %5, off" H "\n\t"                                                               \
        "s_mov_b32 m0, %0"                                                                                     \
        : "=&s"(saved)                                                                                         \
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "s"(lds), "s"(lds + 1024), "s"(lds + 2048),    \
          "s"(lds + 3072), "s"(lds + 4096)                                                                     \
        : "memory")
    if constexpr (NT)
        Q8K_LDS_GATHER_4352(" nt");
    else
        Q8K_LDS_GATHER_4352("");
#undef Q8K_LDS_GATHER_4352
}

// The gather above with the source given as one wave-uniform base (an SGPR pair) and five
// 32-bit per-lane byte offsets from it: no per-lane 64-bit address arithmetic.
template <bool NT = false>
__device__ __forceinline__ void lds_copy_4352_gather_s(const uint8_t* base, const uint32_t (&off)[5], uint32_t lds) {
    uint32_t saved;
#define Q8K_LDS_GATHER_4352_S(H)                                                                             \
    asm volatile(                                                                                              \
        "s_mov_b32 %0, m0\n\t"                                                                                 \
        "s_mov_b32 m0, %7\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %1, %6" H "\n\t"                                                              \
        "s_mov_b32 m0, %8\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %2, %6" H "\n\t"                                                              \
        "s_mov_b32 m0, %9\n\t"                                                                                 \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %3, %6" H "\n\t"                                                              \
        "s_mov_b32 m0, %10\n\t"                                                                                \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dwordx4 %4, %6" H "\n\t"                                                              \
        "s_mov_b32 m0, %11\n\t"                                                                                \
        "s_nop 0\n\t"                                                                                          \
        "global_load_lds_dword %5, %6" H "\n\t"                                                                \
        "s_mov_b32 m0, %0"                                                                                     \
        : "=&s"(saved)                                                                                         \
        : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds), "s"(lds + 1024), \
          "s"(lds + 2048), "s"(lds + 3072), "s"(lds + 4096)                                                    \
        : "memory")
    if constexpr (NT)
        Q8K_LDS_GATHER_4352_S(" nt");
    else
        Q8K_LDS_GATHER_4352_S("");
#undef Q8K_LDS_GATHER_4352_S
}

}  // namespace q8k
