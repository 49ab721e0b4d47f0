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
// The work is bound by moving each row's query (1152 B) and prefix output
// (1 KB in, 1 KB out); the draft keys are a few KB per token.  A workgroup
// takes one draft token and 16 heads, each of its 4 waves 4 heads: a wave
// issues the loads of all its heads' query and output chunks before it
// waits for anything, while the workgroup widens the visible draft rows to
// fp32 in LDS (e4m3 rows scaled).  Lane l holds 16-byte chunk l of a row
// (dims 8l .. 8l + 7, which are also output columns 8l .. 8l + 7) and lanes
// 0..7 the rope chunk 64 + l.  The up to 8 partial dot products of a head
// are summed over the wave by a butterfly that halves the values each lane
// carries at every step (10 exchanges instead of 48), after which lane 8k
// holds score k.  Consecutive head groups of one token go to the same XCD
// so its draft rows are fetched into one L2.  Draft positions or pages
// outside the pool are not read (that key is dropped).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gfx950_asm.h"
#include "plan_layout.h"
#include "tree.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kHeadsPerWave = 4;
constexpr int kHeadsPerBlock = kWaves * kHeadsPerWave;
constexpr int kMaxDrafts = 8;                 // MLA_MAX_Q_LEN
constexpr int kChunks = kDQK / 8;             // 72 chunks of 8 values per row
constexpr int kTail = kChunks - 64;           // rope chunks, taken by lanes 0..7
constexpr int kXcds = 8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};                  // round to nearest even
  return __builtin_bit_cast(uint32_t, p);
}

// <8 bf16 values, 8 fp32 values>
__device__ __forceinline__ float dot8(u32x4 q, f32x4 k0, f32x4 k1) {
  float s = bf16_lo(q[0]) * k0[0];
  s = fmaf(bf16_hi(q[0]), k0[1], s);
  s = fmaf(bf16_lo(q[1]), k0[2], s);
  s = fmaf(bf16_hi(q[1]), k0[3], s);
  s = fmaf(bf16_lo(q[2]), k1[0], s);
  s = fmaf(bf16_hi(q[2]), k1[1], s);
  s = fmaf(bf16_lo(q[3]), k1[2], s);
  return fmaf(bf16_hi(q[3]), k1[3], s);
}

// Sums v[0..7] over the 64 lanes; lane 8k ends up with the sum of v[k].
__device__ __forceinline__ float wave_sum8(const float (&v)[kMaxDrafts], int lane) {
  const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
  float a[4], c[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float send = h32 ? v[j] : v[j + 4];
    a[j] = (h32 ? v[j + 4] : v[j]) + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float send = h16 ? a[j] : a[j + 2];
    c[j] = (h16 ? a[j + 2] : a[j]) + __shfl_xor(send, 16);
  }
  float s = (h8 ? c[1] : c[0]) + __shfl_xor(h8 ? c[0] : c[1], 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  return s;
}

__global__ __launch_bounds__(kWaves * 64) void mla_tree_kernel(const TreeArgs a) {
  __shared__ __attribute__((aligned(16))) float keys[kMaxDrafts][kDQK];
  // consecutive blocks of the linear order share an XCD (blocks are dealt
  // to the XCDs round-robin)
  const int G = int(gridDim.x);
  const int lin = G % kXcds == 0 ? int(blockIdx.x % kXcds) * (G / kXcds) + int(blockIdx.x / kXcds)
                                 : int(blockIdx.x);
  const int groups = (a.num_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int bt = lin / groups, hg = lin - bt * groups;
  const int b = bt / a.max_q_len, t = bt - b * a.max_q_len;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every load below depends only on (b, t, head) and stays inside the
  // [B, q_max, ...] arrays even for a padding token, so all of them are in
  // flight before the first wait
  const int qb = a.q_lens ? a.q_lens[b] : a.max_q_len;
  const int L = a.kv_lens[b];
  const uint32_t mask = a.tree_mask[int64_t(b) * a.max_q_len + t];
  // this wave's rows: query chunks, prefix output chunk, prefix LSE
  const int h0 = hg * kHeadsPerBlock + wave * kHeadsPerWave;
  u32x4 qc[kHeadsPerWave], qt[kHeadsPerWave], oc[kHeadsPerWave];
  float lse_p[kHeadsPerWave];
#pragma unroll
  for (int i = 0; i < kHeadsPerWave; ++i) {
    qc[i] = qt[i] = oc[i] = u32x4{0u, 0u, 0u, 0u};
    lse_p[i] = -INFINITY;
    if (h0 + i >= a.num_heads) continue;
    const int64_t row = (int64_t(b) * a.max_q_len + t) * a.num_heads + h0 + i;
    const u32x4* qrow = reinterpret_cast<const u32x4*>(a.q + row * (kDQK * 2));
    qc[i] = qrow[lane];
    if (lane < kTail) qt[i] = qrow[64 + lane];
    oc[i] = reinterpret_cast<const u32x4*>(a.o + row * (kDLatent * 2))[lane];
    lse_p[i] = a.lse[row];
  }
  if (t >= qb) return;                                        // padding token
  // visible drafts with a cache row in the pool (the same bits in every thread)
  uint32_t vis = 0;
  int64_t rowk[kMaxDrafts];
#pragma unroll
  for (int k = 0; k < kMaxDrafts; ++k) {
    rowk[k] = -1;
    if (k >= qb || !((mask >> k) & 1u)) continue;
    const int64_t pos = int64_t(L) - qb + k;
    if (pos < 0 || pos >= (int64_t(a.max_pages) << a.page_shift)) continue;
    const int page = a.block_table[int64_t(b) * a.max_pages + (pos >> a.page_shift)];
    if (page < 0 || page >= a.num_pages) continue;
    rowk[k] = (int64_t(page) << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
    vis |= 1u << k;
  }
  if (vis == 0) return;                                       // nothing to add

  // visible draft rows -> LDS as fp32: item (k, c) is chunk c of draft k
  for (int it = threadIdx.x; it < kMaxDrafts * kChunks; it += kWaves * 64) {
    const int k = it / kChunks, c = it - k * kChunks;
    if (!((vis >> k) & 1u)) continue;
    int64_t row = 0;
#pragma unroll
    for (int j = 0; j < kMaxDrafts; ++j)
      if (j == k) row = rowk[j];
    f32x4 v0, v1;
    if (a.kv_dtype == 0) {
      const u32x4 w = reinterpret_cast<const u32x4*>(a.kv + row * (kDQK * 2))[c];
      v0 = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      v1 = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    } else {
      const u32x2 w = reinterpret_cast<const u32x2*>(a.kv + row * kDQK)[c];
      const float s = a.kv_scale[row];
      const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[0]), false);
      const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[0]), true);
      const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[1]), false);
      const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[1]), true);
      v0 = f32x4{p0[0] * s, p0[1] * s, p1[0] * s, p1[1] * s};
      v1 = f32x4{p2[0] * s, p2[1] * s, p3[0] * s, p3[1] * s};
    }
    LDS_PTR(f32x4) dst = (LDS_PTR(f32x4))(&keys[k][8 * c]);
    dst[0] = v0;
    dst[1] = v1;
  }
  __syncthreads();

  // partial scores: part[i][k] = this lane's share of <q_i, c_k>
  float part[kHeadsPerWave][kMaxDrafts];
#pragma unroll
  for (int k = 0; k < kMaxDrafts; ++k) {
#pragma unroll
    for (int i = 0; i < kHeadsPerWave; ++i) part[i][k] = 0.f;
    if (!((vis >> k) & 1u)) continue;
    const LDS_PTR(f32x4) kr = (const LDS_PTR(f32x4))(&keys[k][8 * lane]);
    const f32x4 k0 = kr[0], k1 = kr[1];
    f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = t0;
    if (lane < kTail) {
      const LDS_PTR(f32x4) tr = (const LDS_PTR(f32x4))(&keys[k][kDLatent + 8 * lane]);
      t0 = tr[0];
      t1 = tr[1];
    }
#pragma unroll
    for (int i = 0; i < kHeadsPerWave; ++i)
      part[i][k] = dot8(qc[i], k0, k1) + dot8(qt[i], t0, t1);
  }

  // merge weights of every head (uniform over the wave)
  float wp[kHeadsPerWave], w[kHeadsPerWave][kMaxDrafts], lse[kHeadsPerWave];
#pragma unroll
  for (int i = 0; i < kHeadsPerWave; ++i) {
    const float tot = wave_sum8(part[i], lane);
    float s[kMaxDrafts];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) {
      s[k] = -INFINITY;
      if ((vis >> k) & 1u)
        s[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(tot), 8 * k)) * a.sm_scale;
      m = fmaxf(m, s[k]);
    }
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) l += (vis >> k) & 1u ? expf(s[k] - m) : 0.f;
    const float lse_d = m + logf(l);
    const float top = fmaxf(lse_p[i], lse_d);
    lse[i] = top + logf(expf(lse_p[i] - top) + expf(lse_d - top));
    wp[i] = expf(lse_p[i] - lse[i]);                          // 0 for an empty prefix
#pragma unroll
    for (int k = 0; k < kMaxDrafts; ++k) w[i][k] = (vis >> k) & 1u ? expf(s[k] - lse[i]) : 0.f;
  }

  // O = wp O_p + sum_k w_k c_k over this lane's 8 columns
  float acc[kHeadsPerWave][8];
#pragma unroll
  for (int i = 0; i < kHeadsPerWave; ++i) {
    // an empty prefix (LSE -inf) contributes nothing, whatever its O holds
    const bool has_p = lse_p[i] != -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[i][2 * e] = has_p ? wp[i] * bf16_lo(oc[i][e]) : 0.f;
      acc[i][2 * e + 1] = has_p ? wp[i] * bf16_hi(oc[i][e]) : 0.f;
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxDrafts; ++k) {
    if (!((vis >> k) & 1u)) continue;
    const LDS_PTR(f32x4) kr = (const LDS_PTR(f32x4))(&keys[k][8 * lane]);
    const f32x4 k0 = kr[0], k1 = kr[1];
#pragma unroll
    for (int i = 0; i < kHeadsPerWave; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[i][e] = fmaf(w[i][k], k0[e], acc[i][e]);
        acc[i][4 + e] = fmaf(w[i][k], k1[e], acc[i][4 + e]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kHeadsPerWave; ++i) {
    if (h0 + i >= a.num_heads) continue;
    const int64_t row = (int64_t(b) * a.max_q_len + t) * a.num_heads + h0 + i;
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = bf16_pack(acc[i][2 * e], acc[i][2 * e + 1]);
    reinterpret_cast<u32x4*>(a.o + row * (kDLatent * 2))[lane] = out;
    if (lane == 0) a.lse[row] = lse[i];
  }
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream) {
  const int64_t groups = (a.num_heads + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int64_t blocks = int64_t(a.batch) * a.max_q_len * groups;
  if (blocks <= 0) return hipSuccess;
  if (blocks > int64_t(0x7FFFFFFF)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_tree_kernel, dim3(unsigned(blocks)), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
