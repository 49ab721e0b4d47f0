// Internal launcher interface of the quantized prefill kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPfDQK = 192;     // Q/K head dim (128 + 64 rope)
constexpr int kPfDV = 128;      // V head dim
constexpr int kPfBlock = 128;   // tokens per block: query tile, key step and V-scale block

struct PrefillQuantArgs {
  const int32_t* cu;            // [S + 1] device
  const uint16_t* q;            // [T, H, 192] bf16
  const uint16_t* k;            // [T, H, 192] bf16
  const uint16_t* v;            // [T, H, 128] bf16
  int8_t* qc;                   // [T, H, 192]
  float* qs;                    // [T, H]
  int8_t* kc;                   // [T, H, 192]
  float* ks;                    // [T, H]
  uint8_t* vc;                  // [blocks, H, 128, 128]
  float* vs;                    // [blocks, H, 128]
  int32_t num_seqs, num_tokens, num_heads, num_blocks;
};

struct PrefillAttnArgs {
  const int32_t* cu;
  const int8_t* qc;
  const float* qs;
  const int8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  uint8_t* o;                   // [T, H, 128] bf16
  float* lse;                   // [T, H]
  float sm_scale;
  int32_t num_seqs, num_tokens, num_heads, num_blocks;
};

hipError_t launch_prefill_quant(const PrefillQuantArgs& a, hipStream_t stream);
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t stream);

// Block i of the packed sequences: its sequence's first token t0 and length
// n, its index kb within the sequence and the sequence's first block b0.
struct PfBlock {
  int32_t t0, n, kb, b0;
};

// Walks cu_seqlens (device data, checked as it goes: it must start at 0, not
// decrease, stay within T, and the blocks must fit num_blocks).  Returns
// false when block i is not a block of a consistent sequence.  Every thread
// reads the same entries, so the result is uniform over the workgroup.
__device__ inline bool pf_find_block(const int32_t* cu, int32_t S, int32_t T, int32_t nblocks,
                                     int32_t i, PfBlock* out) {
  int32_t prev = cu[0];
  if (prev != 0) return false;
  int32_t b0 = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t nxt = cu[s + 1];
    if (nxt < prev || nxt > T) return false;
    const int32_t nb = (nxt - prev + kPfBlock - 1) / kPfBlock;
    if (b0 + nb > nblocks) return false;
    if (i < b0 + nb) {
      *out = PfBlock{prev, nxt - prev, i - b0, b0};
      return true;
    }
    b0 += nb;
    prev = nxt;
  }
  return false;
}

}  // namespace mla
