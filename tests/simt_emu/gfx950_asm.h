// Emulator version of the kernel's inline-assembly helpers (same names and
// signatures as the library's gfx950_asm.h): LDS-DMA copies are queued per
// lane and land at the vmcnt waits; the barrier is a workgroup rendezvous; a
// wait on an LDS word another wave publishes blocks the lane until it does.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef EMU_LDS_TRACE
#include "lds_trace.h"
#define LDS_PTR(T) emu::LdsP<T>
#else
#define LDS_PTR(T) T*
#endif

namespace emu {
uint32_t lds_address(const void* p);
void lds_dma(uint32_t lds_base, int voff, const void* sbase, int bytes);
void vm_wait(int n);
void block_barrier();
void flag_wait(const int* p, int target);
void flag_publish(int* p, int value);
}  // namespace emu

namespace mla {
inline uint32_t lds_address(const void* p) { return emu::lds_address(p); }
inline void lds_dma_x4(uint32_t lds_base, int voff, const void* sbase) {
  emu::lds_dma(lds_base, voff, sbase, 16);
}
inline void lds_dma_x1(uint32_t lds_base, int voff, const void* sbase) {
  emu::lds_dma(lds_base, voff, sbase, 4);
}
#define MLA_VM_WAIT(N) emu::vm_wait(N)
inline void barrier() { emu::block_barrier(); }
// the wave's lanes meet first (on the GPU the store follows all of the
// wave's earlier LDS writes), then the word is stored
inline void lds_publish(int* p, int value) { emu::flag_publish(p, value); }
// the lane sleeps (is not resumed) until the word reaches the target
inline void lds_wait_at_least(const int* p, int target) { emu::flag_wait(p, target); }
inline int opaque(int x) { return x; }
inline int opaque_s(int x) { return x; }
template <typename T>
inline void require_vgpr(const T&) {}
}  // namespace mla
