// Tree-shaped drafts: the draft tokens' own part of the attention, merged
// into the result of a decode over the cached prefix.
//
// With EAGLE-style drafts (top-k candidates per step: the Dewu DeepSeek
// deployment slides launch SGLang that way) the q draft tokens of a sequence
// form a tree, verified in one pass (PaddlePaddle 3.0 inference page,
// speculative decoding): token t sees the cached prefix (positions below
// L - q) and the drafts its mask word names (draft k at position L - q + k).
// Attention over a union of key sets is the log-sum-exp merge of attention
// over each part (the split-K merge of the FlashAttention-3 in DeepSeek-R1
// page, chapter 2), so the prefix goes through the ordinary decode kernels
// (non-causal, kv_len L - q) and this kernel adds the at most q <= 8 draft
// keys of each row:
//   s_k = scale * <q, c_k>,  LSE_d = ln sum_k e^(s_k),
//   LSE = ln(e^LSE_p + e^LSE_d),
//   O = e^(LSE_p - LSE) O_p + sum_k e^(s_k - LSE) c_k[0:512].
//
// One workgroup per (sequence, draft token): its visible draft rows go to LDS
// as fp32 (e4m3 rows widened and scaled), and each wave takes every fourth
// head: lane l holds dims l + 64 j of the query for the scores and output
// columns 8l .. 8l + 7.  Draft positions or pages outside the pool are not
// read (that key is dropped).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plan_layout.h"
#include "tree.h"

namespace mla {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kMaxDrafts = 8;   // MLA_MAX_Q_LEN

__device__ __forceinline__ float bf16_at(const uint8_t* p, int64_t i) {
  const uint16_t v = reinterpret_cast<const uint16_t*>(p)[i];
  return __uint_as_float(uint32_t(v) << 16);
}

__global__ __launch_bounds__(kWaves * 64) void mla_tree_kernel(const TreeArgs a) {
  __shared__ float keys[kMaxDrafts][kDQK];
  const int b = blockIdx.x / a.max_q_len, t = blockIdx.x - b * a.max_q_len;
  const int qb = a.q_lens ? a.q_lens[b] : a.max_q_len;
  if (t >= qb) return;                                        // padding token
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = a.kv_lens[b];
  const uint32_t mask = a.tree_mask[int64_t(b) * a.max_q_len + t];
  // visible drafts, in draft order, into LDS (every thread walks the same
  // mask, so nk is the same everywhere)
  int nk = 0;
  for (int k = 0; k < qb && k < kMaxDrafts; ++k) {
    if (!((mask >> k) & 1u)) continue;
    const int64_t pos = int64_t(L) - qb + k;
    if (pos < 0 || pos >= (int64_t(a.max_pages) << a.page_shift)) continue;
    const int page = a.block_table[int64_t(b) * a.max_pages + (pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) continue;
    const int64_t row = (int64_t(page) << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
    for (int d = threadIdx.x; d < kDQK; d += kWaves * 64) {
      float v;
      if (a.kv_dtype == 0) {
        v = bf16_at(a.kv, row * kDQK + d);
      } else {
        const int code = a.kv[row * kDQK + d];
        v = __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0] * a.kv_scale[row];
      }
      keys[nk][d] = v;
    }
    ++nk;
  }
  __syncthreads();
  if (nk == 0) return;                                        // nothing to add

  for (int h = wave; h < a.num_heads; h += kWaves) {
    const int64_t qrow = (int64_t(b) * a.max_q_len + t) * a.num_heads + h;
    // the prefix LSE is read by every lane before lane 0 overwrites it below
    const float lse_p = a.lse[qrow];
    float part[kMaxDrafts];
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) part[k] = 0.f;
    for (int j = 0; j < kDQK / 64; ++j) {
      const int d = lane + 64 * j;
      const float qd = bf16_at(a.q, qrow * kDQK + d);
#pragma unroll
      for (int k = 0; k < kMaxDrafts; ++k)
        if (k < nk) part[k] += qd * keys[k][d];
    }
    float s[kMaxDrafts];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) {
      float v = part[k];
      for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x);
      s[k] = k < nk ? v * a.sm_scale : -INFINITY;
      m = fmaxf(m, s[k]);
    }
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) l += k < nk ? expf(s[k] - m) : 0.f;
    const float lse_d = m + logf(l);
    const float top = fmaxf(lse_p, lse_d);
    const float lse = top + logf(expf(lse_p - top) + expf(lse_d - top));
    const float wp = expf(lse_p - lse);                       // 0 for an empty prefix
    float w[kMaxDrafts];
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) w[k] = k < nk ? expf(s[k] - lse) : 0.f;
    bf16x8* orow = reinterpret_cast<bf16x8*>(a.o + qrow * (kDLatent * 2)) + lane;
    const bf16x8 op = *orow;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lane + e;
      float acc = lse_p == -INFINITY ? 0.f : wp * float(op[e]);
#pragma unroll
      for (int k = 0; k < kMaxDrafts; ++k)
        if (k < nk) acc += w[k] * keys[k][d];
      out[e] = (__bf16)acc;
    }
    *orow = out;
    if (lane == 0) a.lse[qrow] = lse;
  }
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream) {
  const int64_t blocks = int64_t(a.batch) * a.max_q_len;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_tree_kernel, dim3(unsigned(blocks)), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
