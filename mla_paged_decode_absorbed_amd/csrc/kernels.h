// Internal launcher interface between the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
  const int32_t* plan;        // device plan image
  const uint8_t* q;           // [B, q_max, H, 576] bf16
  const uint8_t* kv;          // [pages, P, 576] bf16 or e4m3
  const float* kv_scale;      // [pages, P] (fp8 only)
  const int32_t* block_table; // [B, max_pages]
  const int32_t* kv_lens;     // [B]
  const int32_t* q_lens;      // [B] or nullptr
  uint8_t* o;                 // [B, q_max, H, 512] bf16
  float* lse;                 // [B, q_max, H] or nullptr
  float* part_o;              // [partials][128][512]
  float* part_lse;            // [partials][128]
  float scale_log2;           // softmax_scale * log2(e)
  int32_t num_heads;
  int32_t max_q_len;
  int32_t page_shift;         // log2(page_size)
  int32_t max_pages;
  int32_t causal;
  int32_t num_wg;
  int32_t phases;             // waves sharing one row group (1, 2 or 4)
};

struct CombineArgs {
  const int32_t* plan;
  const float* part_o;
  const float* part_lse;
  const int32_t* q_lens;      // [B] or nullptr
  uint8_t* o;
  float* lse;
  int32_t num_heads;
  int32_t max_q_len;
  int32_t num_combine;
};

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// The library's e4m3 decode kernels with the query fragments forced resident
// before the key loop (decode_kernel_qres.hip); chosen only when
// MLA_DECODE_KERNEL=qres, e4m3 caches only.
hipError_t launch_decode_qres(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// Candidate decode kernel with two waves per SIMD (one-phase plans, bf16 or
// e4m3 cache); chosen only when MLA_DECODE_KERNEL=w8.
hipError_t launch_decode_w8(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// Candidate decode kernel with two waves per SIMD sharing each 32-row group
// (decode_split_kernel.hip; one-phase plans, bf16 or e4m3 cache); chosen only when
// MLA_DECODE_KERNEL=split.
hipError_t launch_decode_split(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// The merge over bf16 partials, as the candidate decode kernels write them.
hipError_t launch_combine_bf16(const CombineArgs& a, hipStream_t stream);

}  // namespace mla
