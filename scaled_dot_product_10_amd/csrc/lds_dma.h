// Tile DMA into LDS and the barrier that publishes a tile, shared by the fused
// forward kernels (bf16, fp8) and the backward dQ sweep.
#pragma once

#include "common.h"

namespace attn {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One global_load_lds_dwordx4: 64 lanes x 16 bytes from global memory into 1 KB
// of LDS at lds (wave-uniform), lane L filling bytes [16L, 16L+16); lane L
// fetches base + off (base wave-uniform, off per lane).  Issued as inline
// assembly so the compiler does not treat every later LDS read as dependent on
// it; completion is awaited explicitly (s_waitcnt vmcnt(0)) before the barrier
// that publishes the tile.  M0 is a reserved register that the compiler loads
// right before each of its own uses, so setting it here is safe.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory");
}

// Workgroup barrier between phases.  Inline assembly so that the compiler adds
// no fence of its own (its fence would wait for every outstanding load,
// including the tile DMA that is meant to stay in flight across the barrier);
// the "memory" clobber keeps LDS accesses from moving across it.  LDS reads
// are drained first; with wait_dma, this wave's tile DMA as well.
// The sched_barrier(0) fences keep the compiler from moving any instruction
// (matrix products and exponentials included) from one phase into the next.
__device__ __forceinline__ void phase_barrier(bool wait_dma) {
    __builtin_amdgcn_sched_barrier(0);
    if (wait_dma)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace attn
