// Internal launcher interface of the debug validation kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct CheckArgs {
  const int32_t* plan;         // plan image, plan_words words
  const int32_t* block_table;  // [batch, max_pages]
  const int32_t* kv_lens;      // [batch]
  const int32_t* q_lens;       // [batch] or nullptr (all max_q_len)
  int32_t* err;                // [2] device: check code, index
  int64_t plan_words;
  int32_t batch, num_heads, max_q_len, causal;
  int32_t page_size, num_pages, max_pages;
  int32_t num_wg, phases, num_partials;   // from the launch info
};

hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

}  // namespace mla
