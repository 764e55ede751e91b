// Direct global -> LDS loads (global_load_lds_*) for the attention kernels.
//
// They are issued as inline asm so that the compiler neither tracks them nor inserts
// its own waits for them (its LDS-DMA alias tracking is lost across a tile loop and
// would drain every tile in flight); a kernel waits for them explicitly with vmcnt,
// which counts vector-memory operations in issue order.  The LDS destination of lane i
// is m0 + 16*i (dwordx4) or m0 + 4*i (dword); m0 must be wave-uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sad {

template <typename T>
__device__ inline uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}

__device__ inline void dma_x4(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_wave_base), "v"(src) : "memory", "m0");
}
// Same with an immediate byte offset on the global address.  The instruction adds its
// offset to the LDS address as well, so M0 is lowered by the same amount.
template <int OFF>
__device__ inline void dma_x4_off(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
               :: "s"(lds_wave_base - OFF), "v"(src), "n"(OFF) : "memory", "m0");
}
__device__ inline void dma_x1(const void* src, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_wave_base), "v"(src) : "memory", "m0");
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ inline void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// wait until every LDS (and scalar-load) operation of this wave has completed
__device__ inline void wait_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace sad
