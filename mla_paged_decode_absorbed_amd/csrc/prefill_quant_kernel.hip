// Quantization for the SageAttention-style prefill (PaddlePaddle 3.0 inference
// page, long-sequence inference): Q and K to INT8, V to FP8, on the fly.
//
// Q and K: one symmetric scale per (token, head) row of 192, s = max|x| / 127
// (1 for an all-zero row), code = x / s rounded to nearest even, clamped to
// +-127.  Eight lanes take a row (24 values each: three 16-byte loads, three
// 8-byte stores) and reduce its max with three lane swaps; a wave takes 8
// rows.  Q rows come first in the row index, then K rows.
//
// V: one scale per (128-token block of a sequence, head, channel),
// s = max|v| / 448 over the block's tokens (1 if zero), code = the e4m3 value
// nearest to v / s (ties to even; the hardware conversion on the clamped
// quotient, as in the cache append).  A workgroup takes one (block, head):
// 16 threads cover a token's 256 bytes, 16 token groups reduce the channel
// maxima through LDS, and the codes are laid out in LDS transposed, each
// channel's 128 keys in the order the PV matrix instruction takes them (key
// 16 a + 4 g + r at byte 32 g + 4 a + r), then copied out in 16-byte pieces.
//
// Quotients are correctly rounded fp32 divisions (the compiler's default for
// '/').
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "prefill.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQkRowsPerBlock = 32;          // 4 waves x 8 rows
constexpr int kMaxQkBlocks = 8192;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t int8_code(float x, float s) {
  const float c = fminf(fmaxf(rintf(x / s), -127.f), 127.f);
  return uint32_t(int32_t(c)) & 0xFFu;
}

__global__ __launch_bounds__(256) void mla_prefill_quant_qk_kernel(const PrefillQuantArgs a) {
  const int64_t per_tensor = int64_t(a.num_tokens) * a.num_heads;
  const int64_t rows = 2 * per_tensor;
  const int lane = threadIdx.x & 63, j = lane & 7;
  const int64_t stride = int64_t(gridDim.x) * kQkRowsPerBlock;
  // the loop bound is uniform over the wave, so every lane takes part in the
  // lane swaps; rows past the end are computed on zeros and not stored
  for (int64_t base = int64_t(blockIdx.x) * kQkRowsPerBlock + (threadIdx.x >> 6) * 8; base < rows;
       base += stride) {
    const int64_t r = base + (lane >> 3);
    const bool valid = r < rows;
    const bool is_k = r >= per_tensor;
    const int64_t rr = is_k ? r - per_tensor : r;
    u32x4 c[3] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (valid) {
      const u32x4* src = reinterpret_cast<const u32x4*>((is_k ? a.k : a.q) + rr * kPfDQK) + 3 * j;
      c[0] = src[0];
      c[1] = src[1];
      c[2] = src[2];
    }
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(c[w][e])), fabsf(bf16_hi(c[w][e]))));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    if (!valid) continue;
    float s = m / 127.f;
    if (!(s > 0.f)) s = 1.f;
    u32x2* dst = reinterpret_cast<u32x2*>((is_k ? a.kc : a.qc) + rr * kPfDQK + 24 * j);
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      u32x2 out;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = c[w][2 * h], w1 = c[w][2 * h + 1];
        out[h] = int8_code(bf16_lo(w0), s) | (int8_code(bf16_hi(w0), s) << 8) |
                 (int8_code(bf16_lo(w1), s) << 16) | (int8_code(bf16_hi(w1), s) << 24);
      }
      dst[w] = out;
    }
    if (j == 0) (is_k ? a.ks : a.qs)[rr] = s;
  }
}

// e4m3 code of v / s: correctly rounded quotient, clamped to +-448 with the
// sign kept, rounded by the hardware conversion (nearest, ties to even).
__device__ __forceinline__ uint32_t e4m3_code(float x, float s) {
  const float q = fminf(fabsf(x) / s, 448.f);
  const float y = __uint_as_float(__float_as_uint(q) | (__float_as_uint(x) & 0x80000000u));
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false)) & 0xFFu;
}

__global__ __launch_bounds__(256) void mla_prefill_quant_v_kernel(const PrefillQuantArgs a) {
  __shared__ float pmax[16][kPfDV];
  __shared__ float scale[kPfDV];
  __shared__ __attribute__((aligned(16))) uint8_t codes[kPfDV * kPfBlock];
  const int H = a.num_heads;
  const int i = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  PfBlock blk;
  if (!pf_find_block(a.cu, a.num_seqs, a.num_tokens, a.num_blocks, i, &blk)) return;
  const int key0 = blk.kb * kPfBlock;
  const int nk = min(kPfBlock, blk.n - key0);
  const int cc = threadIdx.x & 15;             // channels 8 cc .. 8 cc + 7
  const int rg = threadIdx.x >> 4;             // keys rg + 16 m
  u32x4 x[8];
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int key = rg + 16 * m;
    x[m] = u32x4{0u, 0u, 0u, 0u};
    if (key < nk)
      x[m] = reinterpret_cast<const u32x4*>(
          a.v + (int64_t(blk.t0 + key0 + key) * H + h) * kPfDV)[cc];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx[2 * e] = fmaxf(mx[2 * e], fabsf(bf16_lo(x[m][e])));
      mx[2 * e + 1] = fmaxf(mx[2 * e + 1], fabsf(bf16_hi(x[m][e])));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) pmax[rg][8 * cc + e] = mx[e];
  __syncthreads();
  if (threadIdx.x < kPfDV) {
    float m = 0.f;
    for (int r = 0; r < 16; ++r) m = fmaxf(m, pmax[r][threadIdx.x]);
    float s = m / 448.f;
    if (!(s > 0.f)) s = 1.f;
    scale[threadIdx.x] = s;
    a.vs[(int64_t(i) * H + h) * kPfDV + threadIdx.x] = s;
  }
  __syncthreads();
  float sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sc[e] = scale[8 * cc + e];
  // key rg + 16 m = 16 m + 4 g + r with g = rg / 4, r = rg % 4: byte 32 g + 4 m + r
  const int pos0 = 32 * (rg >> 2) + (rg & 3);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      codes[(8 * cc + 2 * e) * kPfBlock + pos0 + 4 * m] =
          uint8_t(e4m3_code(bf16_lo(x[m][e]), sc[2 * e]));
      codes[(8 * cc + 2 * e + 1) * kPfBlock + pos0 + 4 * m] =
          uint8_t(e4m3_code(bf16_hi(x[m][e]), sc[2 * e + 1]));
    }
  }
  __syncthreads();
  u32x4* dst = reinterpret_cast<u32x4*>(a.vc + (int64_t(i) * H + h) * (kPfDV * kPfBlock));
  const u32x4* src = reinterpret_cast<const u32x4*>(codes);
#pragma unroll
  for (int c = 0; c < (kPfDV * kPfBlock) / (16 * 256); ++c)
    dst[threadIdx.x + 256 * c] = src[threadIdx.x + 256 * c];
}

}  // namespace

hipError_t launch_prefill_quant(const PrefillQuantArgs& a, hipStream_t stream) {
  const int64_t rows = 2 * int64_t(a.num_tokens) * a.num_heads;
  if (rows > 0) {
    const int blocks = int(std::min<int64_t>((rows + kQkRowsPerBlock - 1) / kQkRowsPerBlock,
                                             kMaxQkBlocks));
    hipLaunchKernelGGL(mla_prefill_quant_qk_kernel, dim3(blocks), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t vblocks = int64_t(a.num_blocks) * a.num_heads;
  if (vblocks > 0) {
    hipLaunchKernelGGL(mla_prefill_quant_v_kernel, dim3(unsigned(vblocks)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mla
