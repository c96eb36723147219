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

// A wave-uniform pointer as the scalar operand of a copy: when the compiler
// cannot prove the value uniform it would otherwise hand the asm a VGPR pair.
// (Both halves go through uint32_t so the high half is not sign-extended.)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<const void*>((uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo));
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
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(base))
        : "memory");
}

// The same copy marked non-temporal (nt): for bytes read once per call, such
// as a decode's K/V pages, so that streaming them does not push out of the
// caches the small data that every workgroup reads (schedule, Q, partials).
__device__ __forceinline__ void dma16_s_nt(const void* base, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(base))
        : "memory");
}

// Runs of copies from one wave-uniform base with M0 written once: copy i
// reads base + voff_i + 1024 i into LDS [lds_addr + 1024 i, +1024) (the
// instruction's immediate offset is added to both the global and the LDS
// address).  A wavefront runs one instruction at a time, so a copy costs as
// many issue slots as the scalar work around it; this keeps it to two per
// copy.
__device__ __forceinline__ void dma16_s_x4(const void* base, uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                           uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "global_load_lds_dwordx4 %3, %6 offset:1024\n\t"
        "global_load_lds_dwordx4 %4, %6 offset:2048\n\t"
        "global_load_lds_dwordx4 %5, %6 offset:3072\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(uniform_ptr(base))
        : "memory");
}
__device__ __forceinline__ void dma16_s_x2(const void* base, uint32_t v0, uint32_t v1, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %4\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:1024\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(v0), "v"(v1), "s"(uniform_ptr(base))
        : "memory");
}

// One copy of such a run: copy I reads base + voff + 1024 I into LDS
// [lds_addr + 1024 I, +1024), as a single instruction, so that copies can be
// spread one at a time between other work.
template <int I>
__device__ __forceinline__ void dma16_s_at(const void* base, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3 offset:%4\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(base)), "i"(1024 * I)
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
