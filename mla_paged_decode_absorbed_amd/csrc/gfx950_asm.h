// The few gfx950 instructions the decode kernel issues from inline assembly,
// kept in one place: HBM -> LDS copies (global_load_lds), explicit vmcnt
// waits, the workgroup barrier and two register-placement hints.
//
// The copies are inline assembly because the compiler, seeing an LDS write it
// cannot order, would wait for every copy in flight before each LDS read; the
// kernel orders them itself with the vmcnt waits below.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_PTR(T) T __attribute__((address_space(3)))*

namespace mla {

// 32-bit LDS address of a shared-memory object (the form M0 takes).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(LDS_PTR(const char))p;
}

// HBM -> LDS copy of 16 (or 4) bytes per lane: LDS destination = lds_base +
// 16 (4) * lane, source = sbase + voff.  M0 is saved and restored.
__device__ __forceinline__ void lds_dma_x4(uint32_t lds_base, int voff, const void* sbase) {
  int tmp;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(tmp)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}
__device__ __forceinline__ void lds_dma_x1(uint32_t lds_base, int voff, const void* sbase) {
  int tmp;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3 offset:0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(tmp)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
// The "memory" clobber keeps later LDS reads after the wait.
#define MLA_VM_WAIT(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")

// Workgroup barrier that also completes this wave's LDS operations first, so
// LDS stores (and the reads of a ring stage about to be refilled) are done
// for every wave after it.
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// An opaque copy of x: the compiler cannot hoist arithmetic on the result out
// of the loop it sits in (such hoisted values would pin VGPRs for the loop).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "=v"(x) : "0"(x));
  return x;
}

// An opaque copy of a wave-uniform value, kept in an SGPR: conditions on it
// are evaluated where they are used (a few scalar instructions) rather than
// hoisted out of the loop, where each would hold a register.
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "=s"(x) : "0"(x));
  return x;
}

// Store `value` to the LDS word at p once this wave's earlier LDS operations
// have completed, so that a wave that sees the value also sees those writes.
__device__ __forceinline__ void lds_publish(LDS_PTR(int) p, int value) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  *(volatile LDS_PTR(int))p = value;
}

// Wait until the LDS word at p, which another wave of the workgroup raises
// with lds_publish, holds at least `target`; later LDS reads stay after the
// wait.  The polls are bounded (about 2^20 of them, tens of milliseconds), so
// that a kernel whose invariant broke returns with wrong results instead of
// holding the GPU.
__device__ __forceinline__ void lds_wait_at_least(const LDS_PTR(int) p, int target) {
  for (int n = 0; n < (1 << 20); ++n) {
    if (__builtin_amdgcn_readfirstlane(*(const volatile LDS_PTR(int))p) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// Require v to be resident in VGPRs here (the compiler then places its wait
// for the load that produced v at this point).
template <typename T>
__device__ __forceinline__ void require_vgpr(const T& v) {
  asm volatile("" ::"v"(v));
}

}  // namespace mla
