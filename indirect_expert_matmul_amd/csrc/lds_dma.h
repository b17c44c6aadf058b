// Direct global -> LDS copies for gfx950 (global_load_lds_*), shared by the grouped
// GEMM and the decode GEMV.
//
// Lane i of the wave reads 4 or 16 bytes and writes them to LDS at
// lds_base + size * i. The copies are issued as inline asm so that the waits are the
// caller's: the compiler cannot see them and would otherwise drain every outstanding
// load at each barrier. They count in the wave's vmcnt like any vector load, and loads
// complete in issue order, so "s_waitcnt vmcnt(N)" with N = copies issued after a
// given one means that copy has landed in LDS. M0 (the LDS base operand) is saved and
// restored around each copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// LDS byte address of a shared-memory pointer.
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A pointer all lanes agree on, held in scalar registers.
static __device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// base: wave-uniform 64-bit address; voff: per-lane 32-bit byte offset. NT marks
// the lines as not expected to be read again (streamed weights), so the caches
// replace them before lines that are (activation rows, scales).
template <bool NT = false>
static __device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
    uint32_t tmp;
    if constexpr (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "global_load_lds_dwordx4 %2, %3 nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(tmp)
            : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "global_load_lds_dwordx4 %2, %3\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(tmp)
            : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base)
            : "memory");
}
static __device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_base) {
    uint32_t tmp;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dword %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(tmp)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base)
        : "memory");
}
// Per-lane 64-bit addresses (lanes may read different tensors).
static __device__ __forceinline__ void dma4v(const void* addr, uint32_t lds_base) {
    uint32_t tmp;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(tmp)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(addr)
        : "memory");
}
static __device__ __forceinline__ void dma16v(const void* addr, uint32_t lds_base) {
    uint32_t tmp;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(tmp)
        : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(addr)
        : "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
static __device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same plus this wave's LDS reads, then meet the other waves at the barrier: the
// copies of every wave up to that point landed, and no wave still reads a buffer
// about to be refilled.
template <int N>
static __device__ __forceinline__ void wait_stage_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace moe
