// Host-side argument checks shared by the C-ABI entry points.
#pragma once
#include <stdint.h>

#include "mla_decode.h"
#include "plan_layout.h"

namespace mla {

inline bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

inline mla_status validate_shape(const mla_shape* s) {
  if (!s) return MLA_ERR_NULL_ARG;
  if (s->batch < 0 || s->num_heads < 1 || s->max_q_len < 1 || s->d_latent < 1 ||
      s->d_rope < 0 || s->page_size < 1 || s->num_pages < 0 || s->max_pages_per_seq < 0 ||
      (s->batch > 0 && (s->max_pages_per_seq < 1 || s->num_pages < 1)))
    return MLA_ERR_BAD_SHAPE;
  if (s->kv_dtype != MLA_KV_BF16 && s->kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (s->d_latent != kDLatent || s->d_rope != kDRope) return MLA_ERR_UNSUPPORTED;
  if (s->max_q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (!is_pow2(s->page_size) || s->page_size < min_page_size_for(s->kv_dtype))
    return MLA_ERR_UNSUPPORTED;
  if (s->causal != 0 && s->causal != 1) return MLA_ERR_BAD_SHAPE;
  // 32-bit row indexing inside the kernels
  if (int64_t(s->num_pages) * s->page_size >= (int64_t(1) << 31)) return MLA_ERR_UNSUPPORTED;
  if (int64_t(s->batch) * s->max_q_len * s->num_heads >= (int64_t(1) << 31))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

inline mla_status validate_lengths(const mla_shape* s, const int32_t* kv_lens,
                                   const int32_t* q_lens) {
  const int64_t cap = int64_t(s->max_pages_per_seq) * s->page_size;
  for (int b = 0; b < s->batch; ++b) {
    const int32_t L = kv_lens[b];
    const int32_t q = q_lens ? q_lens[b] : s->max_q_len;
    if (L < 0 || q < 0 || q > s->max_q_len || L > cap) return MLA_ERR_BAD_SHAPE;
    if (s->causal && q > 0 && L < q) return MLA_ERR_BAD_SHAPE;
  }
  return MLA_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t plan_words_bound(const mla_shape& s, int32_t G);
uint64_t partial_bytes(int64_t n_partials);
mla_status build_plan(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens,
                      int32_t G, int32_t* out, uint64_t out_words, mla_plan_info* info,
                      bool fixed_shape);
// Most 128-row units any lengths of the shape can have.
int64_t max_units(const mla_shape& s);
// Workgroups (MLA_NUM_WORKGROUPS may force them), phases (MLA_PHASES) and the
// per-piece cost (MLA_ITEM_COST_ROUNDS) the planners use.
void plan_launch_params(int32_t* G, int32_t* PH, int32_t* item_cost);
// The launch bounds of a fixed-shape plan (see mla_decode_plan_fixed).
void fixed_launch_info(const mla_shape& s, int32_t G, int32_t PH, mla_plan_info* info);

}  // namespace mla
