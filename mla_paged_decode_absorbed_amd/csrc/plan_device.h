// Internal launcher interface of the device-side planner.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct PlanDeviceArgs {
  const int32_t* kv_lens;   // [B] device
  const int32_t* q_lens;    // [B] device, or nullptr (all max_q_len)
  int32_t* plan;            // plan image, plan_words words
  int32_t* status;          // mla_status of the plan, or nullptr
  int64_t plan_words;
  int32_t batch, num_heads, max_q_len, causal;
  int32_t cap;              // max_pages_per_seq * page_size
  int32_t P, PH, item_cost; // processors, phases, per-piece cost in rounds
};

// LDS the planner needs for a shape (lengths, units, pieces, slots, combine
// entries), in bytes; the launch is refused when it exceeds kPlanLdsBytes.
constexpr int64_t kPlanLdsBytes = 131072;
int64_t plan_lds_bytes(int64_t batch, int64_t max_units, int64_t P);

hipError_t launch_plan(const PlanDeviceArgs& a, int64_t max_units, hipStream_t stream);

}  // namespace mla
