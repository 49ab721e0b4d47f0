// Device-side planner: builds, from device-resident lengths, the same plan
// image as the host planner for a fixed launch shape (mla_decode_plan_fixed),
// so a decode step whose lengths were produced on the GPU (accepted draft
// tokens, for instance) needs no copy of them to the host.
//
// One workgroup of one wave.  All lanes stage the lengths in LDS and check
// them; lane 0 then runs the planner's loops (plan_core.h, the code the host
// planner runs) over LDS arrays and writes the image.  Lengths that the host
// planner would reject yield an empty plan (no items: the decode writes
// nothing) and MLA_ERR_BAD_SHAPE in *status.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode.h"
#include "plan_core.h"
#include "plan_device.h"

namespace mla {
namespace {

__host__ __device__ inline int64_t align16(int64_t x) { return (x + 15) / 16 * 16; }

struct PlanLds {
  int64_t kvl, ql, units, pieces, ufp, slot, comb, total;
};

__host__ __device__ inline PlanLds plan_lds_layout(int64_t B, int64_t MU, int64_t P) {
  PlanLds l;
  l.kvl = 0;
  l.ql = l.kvl + align16(4 * B);
  l.units = l.ql + align16(4 * B);
  l.pieces = l.units + align16(int64_t(sizeof(PlanUnit)) * MU);
  l.ufp = l.pieces + align16(int64_t(sizeof(PlanPiece)) * (MU + P + 1));
  l.slot = l.ufp + align16(4 * (MU + 1));
  l.comb = l.slot + align16(4 * (MU + P + 1));
  l.total = l.comb + align16(4 * kCombineWords * MU);
  return l;
}

__global__ __launch_bounds__(64) void mla_plan_kernel(const PlanDeviceArgs a, int64_t max_units) {
  __shared__ __attribute__((aligned(16))) char lds[kPlanLdsBytes];
  __shared__ int bad;
  const PlanLds l = plan_lds_layout(a.batch, max_units, a.P);
  int32_t* kvl = reinterpret_cast<int32_t*>(lds + l.kvl);
  int32_t* ql = reinterpret_cast<int32_t*>(lds + l.ql);
  const int lane = threadIdx.x;
  if (lane == 0) bad = 0;
  __syncthreads();
  for (int b = lane; b < a.batch; b += 64) {
    const int32_t L = a.kv_lens[b];
    const int32_t q = a.q_lens ? a.q_lens[b] : a.max_q_len;
    kvl[b] = L;
    ql[b] = q;
    // the host planner's length checks
    if (L < 0 || q < 0 || q > a.max_q_len || L > a.cap || (a.causal && q > 0 && L < q)) bad = 1;
  }
  __syncthreads();
  if (lane != 0) return;

  PlanUnit* units = reinterpret_cast<PlanUnit*>(lds + l.units);
  PlanPiece* pieces = reinterpret_cast<PlanPiece*>(lds + l.pieces);
  int32_t* ufp = reinterpret_cast<int32_t*>(lds + l.ufp);
  int32_t* slot = reinterpret_cast<int32_t*>(lds + l.slot);
  int32_t* comb = reinterpret_cast<int32_t*>(lds + l.comb);
  int32_t n_units = 0, n_pieces = 0, C = 0, n_partials = 0;
  if (!bad) {
    for (int32_t b = 0; b < a.batch; ++b)
      n_units += plan_units_of(b, ql[b], kvl[b], a.num_heads, units + n_units);
    const int64_t per_proc = plan_per_proc(units, n_units, a.item_cost, a.P);
    plan_fill(units, n_units, per_proc, a.item_cost, a.P, true, pieces, &n_pieces, ufp);
    plan_slots(units, n_units, ufp, slot, comb, &C, &n_partials);
  }
  // an empty plan when the lengths are bad (no pieces: every workgroup idle)
  const int64_t words = plan_write_image(units, pieces, n_pieces, slot, comb, C, n_partials,
                                         a.PH, a.P * a.PH, a.plan, a.plan_words);
  if (a.status)
    *a.status = bad ? int32_t(MLA_ERR_BAD_SHAPE)
                    : (words < 0 ? int32_t(MLA_ERR_PLAN_TOO_SMALL) : int32_t(MLA_OK));
}

}  // namespace

int64_t plan_lds_bytes(int64_t batch, int64_t max_units, int64_t P) {
  return plan_lds_layout(batch, max_units, P).total;
}

hipError_t launch_plan(const PlanDeviceArgs& a, int64_t max_units, hipStream_t stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(64), 0, stream, a, max_units);
  return hipGetLastError();
}

}  // namespace mla
