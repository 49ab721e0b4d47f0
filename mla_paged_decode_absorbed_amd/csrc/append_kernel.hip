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
// A wave takes kRowsPerWave consecutive rows at a time: it issues every
// load of them before any store, so each wave keeps about 4.6 KB of reads in
// flight.  Lane l moves 16-byte chunk l (8 bf16 values) of a row and lanes
// 0..7 also chunk 64 + l, so every load and store is a contiguous 1 KB
// (+128 B) span.  A bounded grid strides over the rows.
//
// e4m3: the codes must be those of the correctly rounded fp32 quotients x / s.
// One correctly rounded reciprocal y = 1/s per row, q0 = |x| * y, then one
// correction step q = q0 + (|x| - q0 * s) * y in fused multiply-adds gives
// that quotient whenever the remainder |x| - q0 * s stays in the normal range
// (Markstein's theorem on division through a reciprocal); where it does not,
// the quotient is below 2^-49 and its code is 0 either way.  A check over
// every pair of bf16 values (|x| <= max|x|) with s >= 2^-64 finds the same
// codes as true division; rows with smaller scales take a true division.
// The rounding to e4m3 itself is the hardware conversion v_cvt_pk_fp8_f32 on
// values clamped to +-448, checked against the format's definition for every
// fp32 value in that range by the GPU check of tests/gpu_checks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "append.h"
#include "plan_layout.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                     // waves per workgroup
constexpr int kRowsPerWave = 4;               // rows a wave loads before it stores any
constexpr int kRowBytes = kDQK * 2;           // 1152 bytes of a bf16 row
constexpr int kChunks = kRowBytes / 16;       // 72 chunks of 16 bytes
constexpr int kTail = kChunks - 64;           // 8 chunks taken by lanes 0..7
constexpr int kMaxBlocks = 2048;              // 8 workgroups per CU on 256 CUs
constexpr float kE4M3Max = 448.f;
static_assert(kRowsPerWave == 4, "the e4m3 path packs the maxima of rows 0-1 and 2-3");

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |x| of this lane's 16 bf16 values of a row, as the bit pattern of
// the magnitude (for finite values, magnitudes order like their patterns).
__device__ __forceinline__ uint32_t row_max_bits(u32x4 c0, u32x4 c1) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, c0[e] & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, c1[e] & 0x7FFF7FFFu));
  }
  return m[0] > m[1] ? m[0] : m[1];
}

// Per-halfword maximum over the 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_max_u16x2(uint32_t w) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    const uint32_t o = uint32_t(__shfl_xor(int(w), k));
    w = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, w),
                                                               __builtin_bit_cast(u16x2, o)));
  }
  return w;
}

// |x| / s as the correctly rounded fp32 quotient, given y = RN(1 / s).
__device__ __forceinline__ float quotient(float ax, float s, float y, bool exact_div) {
  if (exact_div) return ax / s;
  const float q0 = ax * y;
  return fmaf(fmaf(-q0, s, ax), y, q0);
}

// x / s rounded to fp32 (correctly), clamped to [-448, 448], sign of x kept
// (also for -0).  v_cvt_pk_fp8_f32 then rounds it to the nearest e4m3 code,
// ties to even; values within +-448 never reach its overflow handling.
template <bool kExactDiv>
__device__ __forceinline__ float scaled(float x, float s, float y) {
  const float q = fminf(quotient(fabsf(x), s, y, kExactDiv), kE4M3Max);
  return __uint_as_float(__float_as_uint(q) | (__float_as_uint(x) & 0x80000000u));
}

// 8 bf16 values -> 8 e4m3 codes (byte j of the result = value j)
template <bool kExactDiv>
__device__ __forceinline__ u32x2 chunk_codes(u32x4 c, float s, float y) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(scaled<kExactDiv>(bf16_lo(c[2 * w]), s, y),
                                                   scaled<kExactDiv>(bf16_hi(c[2 * w]), s, y),
                                                   0, false);
    r[w] = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(
        scaled<kExactDiv>(bf16_lo(c[2 * w + 1]), s, y),
        scaled<kExactDiv>(bf16_hi(c[2 * w + 1]), s, y), lo, true));
  }
  return r;
}

// Quantize one row (this lane's chunks) and store codes and scale.
template <bool kExactDiv>
__device__ __forceinline__ void store_e4m3_row(uint8_t* dst, float* scale_dst, u32x4 c0, u32x4 c1,
                                               float s, float y, int lane) {
  *reinterpret_cast<u32x2*>(dst + 8 * lane) = chunk_codes<kExactDiv>(c0, s, y);
  if (lane < kTail) *reinterpret_cast<u32x2*>(dst + 8 * (64 + lane)) = chunk_codes<kExactDiv>(c1, s, y);
  if (lane == 0) *scale_dst = s;
}

// Destination row (cache slot) of source row r, or -1 when r is padding;
// counts a row whose slot lies outside the pool and returns -1 for it too.
__device__ __forceinline__ int64_t dest_slot(const AppendArgs& a, int r, int lane) {
  const int b = r / a.max_new;            // B * max_new < 2^31 (checked on the host)
  const int t = r - b * a.max_new;
  const int n = a.new_lens ? a.new_lens[b] : a.max_new;
  if (t >= n) return -1;                                    // padding row
  const int64_t pos = int64_t(a.kv_lens[b]) - n + t;
  int page = -1;
  if (n <= a.max_new && pos >= 0 && pos < (int64_t(a.max_pages) << a.page_shift))
    page = a.block_table[int64_t(b) * a.max_pages + (pos >> a.page_shift)];
  if (page < 0 || page >= a.num_pages) {
    if (lane == 0 && a.skipped) atomicAdd(a.skipped, 1);
    return -1;
  }
  return (int64_t(page) << a.page_shift) + (pos & ((int64_t(1) << a.page_shift) - 1));
}

template <int KVD>
__global__ __launch_bounds__(kWaves * 64) void mla_kv_append_kernel(const AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = int64_t(a.batch) * a.max_new;   // < 2^31 (checked on the host)
  const int64_t stride = int64_t(gridDim.x) * kWaves * kRowsPerWave;
  // every row index below is uniform over the wave, so every branch is too
  for (int64_t r0 = (int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * kRowsPerWave;
       r0 < rows; r0 += stride) {
    int64_t slot[kRowsPerWave];
    u32x4 c0[kRowsPerWave], c1[kRowsPerWave];
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
      slot[u] = r0 + u < rows ? dest_slot(a, int(r0 + u), lane) : -1;
      c0[u] = c1[u] = u32x4{0u, 0u, 0u, 0u};
      if (slot[u] >= 0) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.src + int64_t(r0 + u) * kRowBytes);
        c0[u] = src[lane];
        if (lane < kTail) c1[u] = src[64 + lane];
      }
    }
    if constexpr (KVD == 0) {
#pragma unroll
      for (int u = 0; u < kRowsPerWave; ++u) {
        if (slot[u] < 0) continue;
        u32x4* dst = reinterpret_cast<u32x4*>(a.kv + slot[u] * kRowBytes);
        dst[lane] = c0[u];
        if (lane < kTail) dst[64 + lane] = c1[u];
      }
    } else {
      // max|x| of the four rows: two rows per 32-bit word, reduced over the
      // wave with packed 16-bit maxima (c1 is zero past the tail; rows not
      // written are zero too)
      const uint32_t w01 = row_max_bits(c0[0], c1[0]) | (row_max_bits(c0[1], c1[1]) << 16);
      const uint32_t w23 = row_max_bits(c0[2], c1[2]) | (row_max_bits(c0[3], c1[3]) << 16);
      const uint32_t m01 = wave_max_u16x2(w01), m23 = wave_max_u16x2(w23);
      // lane l works out row (l & 3)'s scale and reciprocal; lane u hands them out
      const int mine = lane & 3;
      const uint32_t mb = ((mine < 2 ? m01 : m23) >> (16 * (mine & 1))) & 0xFFFFu;
      float s = __uint_as_float(mb << 16) / kE4M3Max;
      if (!(s > 0.f)) s = 1.f;
      const float y = 1.f / s;
#pragma unroll
      for (int u = 0; u < kRowsPerWave; ++u) {
        if (slot[u] < 0) continue;
        const float su = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s), u));
        const float yu = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(y), u));
        uint8_t* dst = a.kv + slot[u] * kDQK;
        if (su < 5.421010862427522e-20f)                          // 2^-64: true division
          store_e4m3_row<true>(dst, a.kv_scale + slot[u], c0[u], c1[u], su, yu, lane);
        else
          store_e4m3_row<false>(dst, a.kv_scale + slot[u], c0[u], c1[u], su, yu, lane);
      }
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv_dtype, hipStream_t stream) {
  const int64_t rows = int64_t(a.batch) * a.max_new;
  if (rows <= 0) return hipSuccess;
  const int64_t per_block = int64_t(kWaves) * kRowsPerWave;
  const int blocks = int(std::min<int64_t>((rows + per_block - 1) / per_block, kMaxBlocks));
  if (kv_dtype == 0)
    hipLaunchKernelGGL((mla_kv_append_kernel<0>), dim3(blocks), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_kv_append_kernel<1>), dim3(blocks), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
