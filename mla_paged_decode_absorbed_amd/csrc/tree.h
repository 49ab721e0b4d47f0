// Internal launcher interface of the tree-draft merge kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct TreeArgs {
  const uint8_t* q;           // [B, q_max, H, 576] bf16
  const uint8_t* kv;          // [pages, P, 576] bf16 or e4m3
  const float* kv_scale;      // [pages, P] (e4m3 only)
  const int32_t* block_table; // [B, max_pages]
  const int32_t* kv_lens;     // [B] keys, drafts included
  const int32_t* q_lens;      // [B] draft tokens, or nullptr (all q_max)
  const uint32_t* tree_mask;  // [B, q_max]: bit k of word t = token t sees draft k
  uint8_t* o;                 // [B, q_max, H, 512] bf16: prefix result in, merged out
  float* lse;                 // [B, q_max, H]: prefix LSE in, merged out
  float sm_scale;
  int32_t batch, num_heads, max_q_len, page_shift, max_pages, num_pages, kv_dtype;
};

hipError_t launch_tree(const TreeArgs& a, hipStream_t stream);

}  // namespace mla
