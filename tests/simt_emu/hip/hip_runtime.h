// Host stand-in for <hip/hip_runtime.h>: runs the decode library's kernel
// sources on the CPU, one std::thread per lane, for memory-safety and parity
// checks without a GPU (built with AddressSanitizer by tests/simt_emu/build.py).
//
// Wave-level operations (MFMA, transposing LDS reads, lane permutes, shuffles,
// ballots) are rendezvous points of the 64 lane threads of a wave; LDS-DMA
// copies are queued per lane and land at the kernel's vmcnt waits, so a read
// of a ring stage before its wait sees stale data, as on the hardware.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct EmuIdx {
  unsigned x, y, z;
};
extern thread_local EmuIdx threadIdx;
extern thread_local EmuIdx blockIdx;
extern thread_local EmuIdx gridDim;

typedef int hipError_t;
enum : int { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorLaunchFailure = 2 };
typedef struct ihipStream_t* hipStream_t;
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 0 };
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device);
hipError_t hipGetLastError();

typedef float emu_f32x2 __attribute__((ext_vector_type(2)));
typedef float emu_f32x4 __attribute__((ext_vector_type(4)));
typedef float emu_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 emu_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 emu_bf16x4 __attribute__((ext_vector_type(4)));
typedef int emu_i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned emu_u32x2 __attribute__((ext_vector_type(2)));
typedef int emu_i32x4 __attribute__((ext_vector_type(4)));
typedef int emu_i32x8 __attribute__((ext_vector_type(8)));

namespace emu {
// kernel launch: blocks run one after another, each as block.x lane threads
void run_grid(dim3 grid, dim3 block, void (*body)(void*), void* ctx);
template <typename K, typename... A>
hipError_t launch(K kernel, dim3 grid, dim3 block, A... args) {
  auto fn = [kernel, args...]() { kernel(args...); };
  using F = decltype(fn);
  run_grid(grid, block, [](void* p) { (*static_cast<F*>(p))(); }, &fn);
  return hipSuccess;
}

// wave-level operations (every lane of the wave must call them)
uint32_t readfirstlane(uint32_t v);
uint32_t readlane(uint32_t v, int lane);
int shfl_xor(int v, int mask);
float shfl_xor(float v, int mask);
int any(int pred);
emu_u32x2 permlane16_swap(uint32_t a, uint32_t b);
emu_u32x2 permlane32_swap(uint32_t a, uint32_t b);
emu_f32x4 mfma16x16x32(emu_bf16x8 a, emu_bf16x8 b, emu_f32x4 c);
emu_f32x16 mfma32x32x16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x16 c);
emu_i32x4 mfma_i8_16x16x64(emu_i32x4 a, emu_i32x4 b, emu_i32x4 c);
emu_f32x4 mfma_f8_16x16x128(emu_i32x8 a, emu_i32x8 b, emu_f32x4 c, int fmt_a, int fmt_b,
                            int scale_a, int scale_b);
emu_bf16x4 ds_read_tr16_b64(const emu_bf16x4* p);
emu_i32x2 ds_read_tr8_b64(const emu_i32x2* p);
emu_f32x2 cvt_pk_f32_fp8(int v, bool hi);
// fp32 -> OCP e4m3fn, round to nearest with ties to even.  The model covers
// the range the kernels use, |x| <= 448; anything else stops the run.
uint32_t e4m3_rne(float x);
inline int cvt_pk_fp8_f32(float a, float b, int old, bool hi) {
  const uint32_t w = e4m3_rne(a) | (e4m3_rne(b) << 8), o = uint32_t(old);
  return int(hi ? (o & 0xFFFFu) | (w << 16) : (o & 0xFFFF0000u) | w);
}
inline unsigned long long memtime() {
  static unsigned long long t = 0;
  return ++t;
}
}  // namespace emu

#define hipLaunchKernelGGL(K, G, B, SH, ST, ...) emu::launch(K, dim3(G), dim3(B), __VA_ARGS__)
namespace emu {
void block_barrier();
}
#define __syncthreads() emu::block_barrier()
#define __builtin_amdgcn_readfirstlane(x) emu::readfirstlane((uint32_t)(x))
#define __builtin_amdgcn_readlane(x, l) emu::readlane((uint32_t)(x), (l))
#define __shfl_xor(v, m) emu::shfl_xor((v), (m))
#define __any(p) emu::any((p))
#define __builtin_amdgcn_permlane16_swap(a, b, fi, bc) emu::permlane16_swap((a), (b))
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) emu::permlane32_swap((a), (b))
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) emu::mfma16x16x32((a), (b), (c))
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) emu::mfma32x32x16((a), (b), (c))
#define __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, x, y, z) emu::mfma_i8_16x16x64((a), (b), (c))
#define __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fa, fb, oa, sa, ob, sb) \
  emu::mfma_f8_16x16x128((a), (b), (c), (fa), (fb), (sa), (sb))
#define __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p) emu::ds_read_tr16_b64((const emu_bf16x4*)(p))
#define __builtin_amdgcn_ds_read_tr8_b64_v2i32(p) emu::ds_read_tr8_b64((const emu_i32x2*)(p))
#define __builtin_amdgcn_cvt_pk_f32_fp8(v, hi) emu::cvt_pk_f32_fp8((v), (hi))
#define __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, hi) emu::cvt_pk_fp8_f32((a), (b), (old), (hi))
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_sched_group_barrier(a, b, c) ((void)0)
#define __builtin_amdgcn_sched_barrier(a) ((void)0)
#define __log2f(x) log2f(x)
#define __logf(x) logf(x)
#define __expf(x) expf(x)
#define __builtin_amdgcn_s_memtime() emu::memtime()
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipMemcpyFromSymbol(void* dst, const void* sym, size_t n) {
  std::memcpy(dst, sym, n);
  return hipSuccess;
}
inline hipError_t hipMemcpyToSymbol(const void* sym, const void* src, size_t n) {
  std::memcpy(const_cast<void*>(sym), src, n);
  return hipSuccess;
}

inline unsigned __float_as_uint(float x) { return __builtin_bit_cast(unsigned, x); }
inline float __uint_as_float(unsigned x) { return __builtin_bit_cast(float, x); }
inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_RELAXED); }
inline unsigned long long atomicAdd(unsigned long long* p, unsigned long long v) {
  const unsigned long long old = *p;
  *p = old + v;
  return old;
}
inline int atomicMin(int* p, int v) {
  int old = *p;
  if (v < old) *p = v;
  return old;
}
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
