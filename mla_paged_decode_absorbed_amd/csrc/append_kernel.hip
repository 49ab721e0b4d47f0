// Cache append: stores this step's new latent rows (576 wide: 512 latent +
// 64 rope) into their slots of the paged cache, before the decode reads them.
//
// Token t of the q_b new tokens of sequence b sits at position
// kv_len_b - q_b + t (the cache length counts the new tokens), which is slot
// position mod P of page block_table[b][position / P] -- the page/block-table
// layout of the FlashAttention-3 in DeepSeek-R1 page (section 4.1).  A bf16
// cache takes the row as it is.  An e4m3 cache takes the row quantized with
// one symmetric fp32 scale per token, the largest magnitude of the row over
// the largest e4m3 magnitude (448): the per-token absmax calibration of that
// page's section 3.1, with the e4m3 range in place of int8's, for the 8-bit
// KV-cache inference the PaddlePaddle 3.0 inference page lists.  An all-zero
// row gets scale 1 (its codes are all zero either way).
//
// One wave per row: lane l moves 16-byte chunk l (8 bf16 values) and lanes
// 0..7 also chunk 64 + l, so every load and store is a contiguous 1 KB (+128
// B) span.  A bounded grid strides over the rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "append.h"
#include "plan_layout.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                     // waves (rows in flight) per workgroup
constexpr int kRowBytes = kDQK * 2;           // 1152 bytes of a bf16 row
constexpr int kChunks = kRowBytes / 16;       // 72 chunks of 16 bytes
constexpr int kTail = kChunks - 64;           // 8 chunks taken by lanes 0..7
constexpr int kMaxBlocks = 2048;              // 8 workgroups per CU on 256 CUs
constexpr float kE4M3Max = 448.f;

// fp32 -> e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities, largest magnitude 448), round to nearest, ties to even, the
// magnitude clamped to 448 first.
__device__ __forceinline__ uint32_t to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {
    // below 2^-6 the grid is k * 2^-9, k = 0..7; k = 8 is the smallest normal
    code = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const uint32_t v = __float_as_uint(a);
    const uint32_t m = v & 0x7FFFFFu;
    code = (((v >> 23) - 120u) << 3) | (m >> 20);   // exponent rebiased 127 -> 7
    const uint32_t rest = m & 0xFFFFFu;               // the 20 dropped mantissa bits
    // a carry out of the mantissa moves to the next binade, as it should
    code += (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ? 1u : 0u;
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float chunk_amax(u32x4 c) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(c[e])), fabsf(bf16_hi(c[e]))));
  return m;
}

// 8 bf16 values -> 8 e4m3 codes (byte j of the result = value j)
__device__ __forceinline__ u32x2 chunk_codes(u32x4 c, float scale) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t c0 = to_e4m3(bf16_lo(c[2 * w]) / scale);
    const uint32_t c1 = to_e4m3(bf16_hi(c[2 * w]) / scale);
    const uint32_t c2 = to_e4m3(bf16_lo(c[2 * w + 1]) / scale);
    const uint32_t c3 = to_e4m3(bf16_hi(c[2 * w + 1]) / scale);
    r[w] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  return r;
}

template <int KVD>
__global__ __launch_bounds__(kWaves * 64) void mla_kv_append_kernel(const AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = int64_t(a.batch) * a.max_new;
  const int64_t stride = int64_t(gridDim.x) * kWaves;
  const int64_t pmask = (int64_t(1) << a.page_shift) - 1;
  // r is uniform over the wave, so every branch below is too
  for (int64_t r = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6); r < rows; r += stride) {
    const int b = int(r / a.max_new);
    const int t = int(r - int64_t(b) * a.max_new);
    const int n = a.new_lens ? a.new_lens[b] : a.max_new;
    if (t >= n) continue;                                   // padding row
    const int64_t pos = int64_t(a.kv_lens[b]) - n + t;
    int page = -1;
    if (n <= a.max_new && pos >= 0 && pos < (int64_t(a.max_pages) << a.page_shift))
      page = a.block_table[int64_t(b) * a.max_pages + (pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) {
      if (lane == 0 && a.skipped) atomicAdd(a.skipped, 1);
      continue;
    }
    const int64_t slot = (int64_t(page) << a.page_shift) + (pos & pmask);
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src + r * kRowBytes);
    const u32x4 c0 = src[lane];
    const u32x4 c1 = lane < kTail ? src[64 + lane] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (KVD == 0) {
      u32x4* dst = reinterpret_cast<u32x4*>(a.kv + slot * kRowBytes);
      dst[lane] = c0;
      if (lane < kTail) dst[64 + lane] = c1;
    } else {
      float amax = fmaxf(chunk_amax(c0), chunk_amax(c1));   // c1 is zero past the tail
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      float scale = amax / kE4M3Max;
      if (!(scale > 0.f)) scale = 1.f;
      uint8_t* dst = a.kv + slot * kDQK;
      *reinterpret_cast<u32x2*>(dst + 8 * lane) = chunk_codes(c0, scale);
      if (lane < kTail) *reinterpret_cast<u32x2*>(dst + 8 * (64 + lane)) = chunk_codes(c1, scale);
      if (lane == 0) a.kv_scale[slot] = scale;
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv_dtype, hipStream_t stream) {
  const int64_t rows = int64_t(a.batch) * a.max_new;
  if (rows <= 0) return hipSuccess;
  const int blocks = int(std::min<int64_t>((rows + kWaves - 1) / kWaves, kMaxBlocks));
  if (kv_dtype == 0)
    hipLaunchKernelGGL((mla_kv_append_kernel<0>), dim3(blocks), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_kv_append_kernel<1>), dim3(blocks), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
