// Quantization for the SageAttention-style prefill (PaddlePaddle 3.0 inference
// page, long-sequence inference): Q and K to INT8, V to FP8, on the fly.
//
// Q: one symmetric scale per (token, head) row of 192, s = max|x| / 127 (1
// for an all-zero row), code = x / s rounded to nearest even, clamped to
// +-127.  Eight lanes take a row (24 values each: three 16-byte loads, three
// 8-byte stores) and reduce its max with three lane swaps; a wave takes 8
// rows.
//
// K: the same rule with one scale per (128-token block of a sequence, head),
// the max over the block's 128 x 192 values: a workgroup takes one (block,
// head), each thread 12 16-byte pieces, the max reduced over the wave and
// through LDS.
//
// V: one power-of-two scale per (128-token block, head, channel), the
// smallest 2^e (e >= -127) with max|v| / 2^e <= 448 (2^0 if zero), taken
// exactly from the max's exponent and mantissa; code = the e4m3 value
// nearest to v 2^-e (an exact product; the hardware conversion, nearest
// even).  A workgroup takes one (block, head):
// 16 threads cover a token's 256 bytes, 16 token groups reduce the channel
// maxima through LDS, and the codes are laid out in LDS transposed, each
// channel's 128 keys in the order the PV matrix instruction takes them (key
// 16 a + 4 g + r at byte 32 g + 4 a + r), then copied out in 16-byte pieces.
//
// Q and K quotients are correctly rounded fp32 divisions (the compiler's
// default for '/').
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

__global__ __launch_bounds__(256) void mla_prefill_quant_q_kernel(const PrefillQuantArgs a) {
  const int64_t rows = int64_t(a.num_tokens) * a.num_heads;
  const int lane = threadIdx.x & 63, j = lane & 7;
  const int64_t stride = int64_t(gridDim.x) * kQkRowsPerBlock;
  // the loop bound is uniform over the wave, so every lane takes part in the
  // lane swaps; rows past the end are computed on zeros and not stored
  for (int64_t base = int64_t(blockIdx.x) * kQkRowsPerBlock + (threadIdx.x >> 6) * 8; base < rows;
       base += stride) {
    const int64_t r = base + (lane >> 3);
    const bool valid = r < rows;
    u32x4 c[3] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (valid) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.q + r * kPfDQK) + 3 * j;
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
    u32x2* dst = reinterpret_cast<u32x2*>(a.qc + r * kPfDQK + 24 * j);
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
    if (j == 0) a.qs[r] = s;
  }
}

// K codes with one scale per (block, head): thread t takes pieces t + 256 p
// (p < 12) of the block's 128 x 24 16-byte pieces (key = piece / 24).
__global__ __launch_bounds__(256) void mla_prefill_quant_k_kernel(const PrefillQuantArgs a) {
  __shared__ float wmax[4];
  constexpr int kPieces = kPfBlock * (kPfDQK / 8) / 256;     // 12
  const int H = a.num_heads;
  const int i = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  PfBlock blk;
  if (!pf_find_block(a.cu, a.num_seqs, a.num_tokens, a.num_blocks, i, &blk)) return;
  const int key0 = blk.kb * kPfBlock;
  const int nk = min(kPfBlock, blk.n - key0);
  u32x4 x[kPieces];
  float m = 0.f;
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int c = int(threadIdx.x) + 256 * p;
    const int key = c / 24, part = c - key * 24;
    x[p] = u32x4{0u, 0u, 0u, 0u};
    if (key < nk)
      x[p] = reinterpret_cast<const u32x4*>(a.k + (int64_t(blk.t0 + key0 + key) * H + h) *
                                                      kPfDQK)[part];
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(x[p][e])), fabsf(bf16_hi(x[p][e]))));
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float s = m / 127.f;
  if (!(s > 0.f)) s = 1.f;
  if (threadIdx.x == 0) a.ks[int64_t(i) * H + h] = s;
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int c = int(threadIdx.x) + 256 * p;
    const int key = c / 24, part = c - key * 24;
    if (key >= nk) continue;
    u32x2 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t w0 = x[p][2 * w], w1 = x[p][2 * w + 1];
      out[w] = int8_code(bf16_lo(w0), s) | (int8_code(bf16_hi(w0), s) << 8) |
               (int8_code(bf16_lo(w1), s) << 16) | (int8_code(bf16_hi(w1), s) << 24);
    }
    reinterpret_cast<u32x2*>(a.kc + (int64_t(blk.t0 + key0 + key) * H + h) * kPfDQK)[part] = out;
  }
}

// e4m3 code of v 2^-e (exact; within +-448 by the choice of e, clamped all
// the same), rounded by the hardware conversion (nearest, ties to even).
__device__ __forceinline__ uint32_t e4m3_code(float x, int e) {
  const float y = fminf(fmaxf(ldexpf(x, -e), -448.f), 448.f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false)) & 0xFFu;
}

// Smallest e >= -127 with amax 2^-e <= 448, 0 for amax = 0: with
// amax = f 2^E, f in [0.5, 1), 448 = 0.875 2^9 fits at E - 9 if f <= 0.875.
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = f <= 0.875f ? E - 9 : E - 8;
  return e < -127 ? -127 : e;
}

__global__ __launch_bounds__(256) void mla_prefill_quant_v_kernel(const PrefillQuantArgs a) {
  __shared__ float pmax[16][kPfDV];
  __shared__ int expo[kPfDV];
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
    const int e = pow2_exponent(m);
    expo[threadIdx.x] = e;
    a.vs[(int64_t(i) * H + h) * kPfDV + threadIdx.x] = ldexpf(1.f, e);
  }
  __syncthreads();
  int sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sc[e] = expo[8 * cc + e];
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
  const int64_t rows = int64_t(a.num_tokens) * a.num_heads;
  if (rows > 0) {
    const int blocks = int(std::min<int64_t>((rows + kQkRowsPerBlock - 1) / kQkRowsPerBlock,
                                             kMaxQkBlocks));
    hipLaunchKernelGGL(mla_prefill_quant_q_kernel, dim3(blocks), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t kvblocks = int64_t(a.num_blocks) * a.num_heads;
  if (kvblocks > 0) {
    hipLaunchKernelGGL(mla_prefill_quant_k_kernel, dim3(unsigned(kvblocks)), dim3(256), 0, stream,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_prefill_quant_v_kernel, dim3(unsigned(kvblocks)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mla
