// Asynchronous global -> LDS copies and the waits and barriers that go with them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pakv_dev {

// One instruction copies 16 bytes per active lane; lane i writes LDS byte
// address m0 + 16*i.  M0 is saved and restored around it (the compiler keeps
// its own values there), with the one wait state the hardware needs between
// writing M0 and an LDS-DMA instruction.  The compiler does not track these
// copies: completion is awaited explicitly (wait_vm) before a barrier.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gaddr)
        : "memory");
}

// Same copy from a wave-uniform base address plus a per-lane 32-bit byte
// offset (the scalar-base form keeps one VGPR per copy instead of two).
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(base)
        : "memory");
}

// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier for LDS traffic only: waits for this wave's LDS reads/writes (not
// for global->LDS copies in flight) and orders the compiler around it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) { return (uint32_t)(uintptr_t)p; }

}  // namespace pakv_dev
