// Internal launcher interface of the cache-append kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct AppendArgs {
  const uint8_t* src;         // [B, max_new, 576] bf16 rows of the new tokens
  const int32_t* new_lens;    // [B] new tokens per sequence, or nullptr (all max_new)
  const int32_t* block_table; // [B, max_pages]
  const int32_t* kv_lens;     // [B] cached tokens per sequence, new ones included
  uint8_t* kv;                // [pages, P, 576] bf16 or e4m3
  float* kv_scale;            // [pages, P] (e4m3 only)
  int32_t* skipped;           // rows whose slot lies outside the pool, or nullptr
  int32_t batch;
  int32_t max_new;
  int32_t page_shift;         // log2(page_size)
  int32_t max_pages;
  int32_t num_pages;
};

hipError_t launch_append(const AppendArgs& a, int kv_dtype, hipStream_t stream);

}  // namespace mla
