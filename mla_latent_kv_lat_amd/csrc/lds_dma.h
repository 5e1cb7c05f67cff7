// Direct-to-LDS staging helpers of the decode kernels that stream cache tiles into LDS by
// global_load_lds (gfx950), with the waits they need.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mla {

// Direct-to-LDS load of 16 bytes per lane: lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).
// Written as inline assembly so that the compiler does not treat every later LDS read as
// dependent on it; completion is awaited explicitly (wait_vm) before the step's barrier.
// The base address and the LDS address are wave-uniform (made scalar here; each 32-bit half
// goes through an unsigned value, so the low half is zero-extended).  The compiler does not
// insert wait states inside inline assembly, so the block carries the ones the hardware
// needs: one between the M0 write and the LDS-DMA load, and five between a vector-ALU write of
// an SGPR (the read-first-lane above) and a memory instruction reading it (the M0 write plus
// four no-ops).
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
  const uint64_t ps = (uint64_t(hi) << 32) | uint64_t(lo);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ps), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void dma16_v(const void* addr, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(m0)
               : "memory");
}
// Scalar load of one int (a wave-uniform address) and its wait, in one block: the value is
// ready when the block ends.  Used for block-table entries inside the tile loop, where a
// vector load would make the compiler wait for every outstanding vector-memory operation,
// the tile loads in flight included.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  const uint64_t as = (uint64_t(hi) << 32) | uint64_t(lo);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(as) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier after this wave's LDS accesses have completed.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }

__device__ __forceinline__ uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace mla
