// Merge of key-range partials: for every split row block of the plan,
//   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) * O_s  -> bf16.
// This is the log-sum-exp merge that makes the split-K key partition of the
// FlashAttention-3 in DeepSeek-R1 page (chapter 2) exact up to rounding.
// One workgroup handles 4 query rows of one combine entry; 64 lanes per row,
// 8 output columns per lane (two 16-byte fp32 loads per partial).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "plan_layout.h"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRowsPerCta = 4;

__global__ __launch_bounds__(256) void mla_combine_kernel(const CombineArgs a) {
  // the grid may be a bound (plans for a fixed launch shape): the plan image
  // holds the real number of entries
  if (int(blockIdx.x) >= a.plan[kWNumCombine]) return;
  const int32_t* comb = a.plan + a.plan[kWOffCombine] + blockIdx.x * kCombineWords;
  const int b = comb[0], row0 = comb[1], first = comb[2], n = comb[3];
  const int rb = blockIdx.y * kRowsPerCta + (threadIdx.x >> 6);   // row inside the block
  const int lane = threadIdx.x & 63;
  const int H = a.num_heads;
  const int qb = a.q_lens ? a.q_lens[b] : a.max_q_len;
  const int row = row0 + rb;
  if (row >= qb * H) return;
  const int t = row / H, h = row - t * H;

  float m = -INFINITY;
  for (int s = 0; s < n; ++s) m = fmaxf(m, a.part_lse[(int64_t)(first + s) * kRowsPerBlock + rb]);
  const int64_t orow = (int64_t)(b * a.max_q_len + t) * H + h;
  bf16x8 out;
  if (m == -INFINITY) {
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)0.f;
    if (a.lse && lane == 0) a.lse[orow] = -INFINITY;
  } else {
    f32x4 acc0 = f32x4{}, acc1 = f32x4{};
    float tot = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = __expf(a.part_lse[(int64_t)(first + s) * kRowsPerBlock + rb] - m);
      if (w > 0.f) {
        const f32x4* src = reinterpret_cast<const f32x4*>(
            a.part_o + ((int64_t)(first + s) * kRowsPerBlock + rb) * kDLatent + lane * 8);
        acc0 += w * src[0];
        acc1 += w * src[1];
        tot += w;
      }
    }
    const float inv = 1.f / tot;
    for (int e = 0; e < 4; ++e) {
      out[e] = (__bf16)(acc0[e] * inv);
      out[4 + e] = (__bf16)(acc1[e] * inv);
    }
    if (a.lse && lane == 0) a.lse[orow] = m + __logf(tot);
  }
  *reinterpret_cast<bf16x8*>(a.o + orow * (kDLatent * 2) + lane * 16) = out;
}

// The same merge over bf16 partials (the two-waves-per-SIMD candidate writes
// them: [partials][128][512] bf16 in the first half of the fp32 partial area,
// the LSE where it always is).  Kept apart from mla_combine_kernel, whose
// compiled code stays as validated.
__global__ __launch_bounds__(256) void mla_combine_kernel_bf16(const CombineArgs a) {
  if (int(blockIdx.x) >= a.plan[kWNumCombine]) return;
  const int32_t* comb = a.plan + a.plan[kWOffCombine] + blockIdx.x * kCombineWords;
  const int b = comb[0], row0 = comb[1], first = comb[2], n = comb[3];
  const int rb = blockIdx.y * kRowsPerCta + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int H = a.num_heads;
  const int qb = a.q_lens ? a.q_lens[b] : a.max_q_len;
  const int row = row0 + rb;
  if (row >= qb * H) return;
  const int t = row / H, h = row - t * H;
  const __bf16* part = reinterpret_cast<const __bf16*>(a.part_o);

  float m = -INFINITY;
  for (int s = 0; s < n; ++s) m = fmaxf(m, a.part_lse[(int64_t)(first + s) * kRowsPerBlock + rb]);
  const int64_t orow = (int64_t)(b * a.max_q_len + t) * H + h;
  bf16x8 out;
  if (m == -INFINITY) {
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)0.f;
    if (a.lse && lane == 0) a.lse[orow] = -INFINITY;
  } else {
    float acc[8] = {};
    float tot = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = __expf(a.part_lse[(int64_t)(first + s) * kRowsPerBlock + rb] - m);
      if (w > 0.f) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(
            part + ((int64_t)(first + s) * kRowsPerBlock + rb) * kDLatent + lane * 8);
        for (int e = 0; e < 8; ++e) acc[e] += w * (float)v[e];
        tot += w;
      }
    }
    const float inv = 1.f / tot;
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] * inv);
    if (a.lse && lane == 0) a.lse[orow] = m + __logf(tot);
  }
  *reinterpret_cast<bf16x8*>(a.o + orow * (kDLatent * 2) + lane * 16) = out;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.num_combine <= 0) return hipSuccess;
  const dim3 grid(a.num_combine, kRowsPerBlock / kRowsPerCta), block(256);
  hipLaunchKernelGGL(mla_combine_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t stream) {
  if (a.num_combine <= 0) return hipSuccess;
  const dim3 grid(a.num_combine, kRowsPerBlock / kRowsPerCta), block(256);
  hipLaunchKernelGGL(mla_combine_kernel_bf16, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
