// Device helpers shared by the MFMA decode kernels: asynchronous
// global -> LDS copies, scalar loads of wave-uniform values, and an opaque
// copy of a per-lane value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// One asynchronous 1 KiB copy: global_load_lds_dwordx4 writes lane i's 16
// bytes to LDS at M0 + 16 i.  Issued as inline asm so that the compiler's
// wait-count pass does not see an LDS writer in flight (it would otherwise
// drain every LDS read with lgkmcnt(0)); completion is awaited explicitly
// (vmcnt + barrier) before a stage is read.  VMEM loads complete in order, so
// the compiler's own vmcnt waits stay correct: unseen extra loads can only
// make them over-wait.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, const uint8_t *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(src)
                 : "memory", "m0");
}

// One asynchronous 4-byte copy by lane 0 only: to LDS at M0 (the block scale
// of an 8-bit stage).  Same wait discipline as dma16.
__device__ __forceinline__ void dma4_lane0(uint32_t lds_addr, const uint8_t *src, int lane) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    if (lane == 0)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                     :: "s"(m0), "v"(0u), "s"(src) : "memory", "m0");
}

// One asynchronous 4-byte copy by every lane of the same source word: 64
// copies at M0 + 4 i (a wave-uniform value without an exec-mask branch).
// Same wait discipline as dma16.
__device__ __forceinline__ void dma4_all(uint32_t lds_addr, const uint8_t *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(0u), "s"(src) : "memory", "m0");
}

// Loads of wave-uniform values (plan, block table, lengths) through the
// constant address space become scalar loads, which never wait on the
// vector-memory counter of the asynchronous stage copies.
__device__ __forceinline__ int32_t sload(const int32_t *p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// An opaque copy of a per-lane value: offsets derived from it are computed
// where they are used and die there, instead of being held in registers
// across a stage loop.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

}  // namespace mla
