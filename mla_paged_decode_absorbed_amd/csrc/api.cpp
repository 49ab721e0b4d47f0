// C-ABI entry points: argument checks, then one launch each.  No allocation,
// no host synchronisation, no mutable global state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>

#include "append.h"
#include "check.h"
#include "kernels.h"
#include "mla_decode.h"
#include "plan_device.h"
#include "plan_layout.h"
#include "prefill.h"
#include "tree.h"
#include "validate.h"

using namespace mla;

namespace {

int ilog2(int32_t x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

mla_status check_info(const mla_shape* s, const mla_plan_info* info) {
  if (!info) return MLA_ERR_NULL_ARG;
  if (info->num_workgroups < 1 || info->num_items < 0 || info->num_partials < 0 ||
      info->num_combine < 0 || info->rows_per_block != kRowsPerBlock ||
      info->tile_tokens != tile_tokens_for(s->kv_dtype) ||
      (info->phases != 1 && info->phases != 2 && info->phases != 4))
    return MLA_ERR_BAD_PLAN;
  return MLA_OK;
}

// MLA_DECODE_KERNEL=w8 selects the two-waves-per-SIMD candidate decode
// kernel for the plans it covers (one phase, either cache type), and with it
// the merge of the bf16 partials it writes; every other plan, and the
// default, runs the library's decode and combine kernels.  mla_decode_fwd and
// mla_combine of one step must see the same setting.
bool candidate_selected(const mla_plan_info* info) {
  const char* variant = std::getenv("MLA_DECODE_KERNEL");
  return variant && std::strcmp(variant, "w8") == 0 && info->phases == 1;
}

// MLA_DECODE_KERNEL=split selects the candidate whose pairs of waves share
// each 32-row group (one-phase plans, either cache type), and with it the
// merge of the bf16 partials it writes; other plans run the library's
// kernels.
bool split_selected(const mla_plan_info* info) {
  const char* variant = std::getenv("MLA_DECODE_KERNEL");
  return variant && std::strcmp(variant, "split") == 0 && info->phases == 1;
}

// MLA_DECODE_KERNEL=qres selects, for e4m3 caches, the library's e4m3
// kernels rebuilt with the query fragments resident before the key loop
// (same plans, same fp32 partials and merge).
bool qres_selected(const mla_shape* shape) {
  const char* variant = std::getenv("MLA_DECODE_KERNEL");
  return variant && std::strcmp(variant, "qres") == 0 && shape->kv_dtype == MLA_KV_FP8_E4M3;
}

// MLA_LOG=1: one line per host plan on stderr (shape, counts, and the keys
// each workgroup takes: the balance the planner reached).  Plan time only.
void log_plan(const mla_shape* shape, const int32_t* plan, const mla_plan_info* info,
              bool fixed_shape) {
  const char* e = std::getenv("MLA_LOG");
  if (!e || std::strcmp(e, "1") != 0) return;
  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  int64_t total = 0, most = 0;
  for (int g = 0; g < info->num_workgroups; ++g) {
    int64_t keys = 0;
    for (int it = wg_start[g]; it < wg_start[g + 1]; ++it)
      keys += items[it * kItemWords + 3] - items[it * kItemWords + 2];
    total += keys;
    most = keys > most ? keys : most;
  }
  const double mean = info->num_workgroups > 0 ? double(total) / info->num_workgroups : 0.0;
  std::fprintf(stderr,
               "mla: plan%s B %d H %d q_max %d page %d %s: %d workgroups, %d items, %d partials, "
               "%d merged blocks, %d phase(s); keys per workgroup max %lld, mean %.1f\n",
               fixed_shape ? " (fixed shape)" : "", shape->batch, shape->num_heads,
               shape->max_q_len, shape->page_size, shape->kv_dtype == MLA_KV_BF16 ? "bf16" : "e4m3",
               info->num_workgroups, info->num_items, info->num_partials, info->num_combine,
               info->phases, static_cast<long long>(most), mean);
}

mla_status host_plan(const mla_shape* shape, const int32_t* kv_lens_host,
                     const int32_t* q_lens_host, int32_t num_workgroups, void* plan_host,
                     uint64_t plan_bytes, mla_plan_info* info, bool fixed_shape) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  if ((shape->batch > 0 && !kv_lens_host) || !plan_host || !info) return MLA_ERR_NULL_ARG;
  if (num_workgroups < 1) return MLA_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(plan_host) & 3u) != 0) return MLA_ERR_MISALIGNED;
  st = validate_lengths(shape, kv_lens_host, q_lens_host);
  if (st != MLA_OK) return st;
  st = build_plan(*shape, kv_lens_host, q_lens_host, num_workgroups,
                  static_cast<int32_t*>(plan_host), plan_bytes / sizeof(int32_t), info,
                  fixed_shape);
  if (st == MLA_OK) log_plan(shape, static_cast<const int32_t*>(plan_host), info, fixed_shape);
  return st;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case MLA_ERR_BAD_SHAPE: return "inconsistent shape or lengths";
    case MLA_ERR_UNSUPPORTED: return "shape or dtype has no built kernel";
    case MLA_ERR_MISALIGNED: return "device pointer is not 16-byte aligned";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the plan needs";
    case MLA_ERR_PLAN_TOO_SMALL: return "plan buffer smaller than the plan needs";
    case MLA_ERR_BAD_PLAN: return "plan info does not match the shape";
    case MLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
  }
  return "unknown status";
}

uint64_t mla_plan_bytes_bound(const mla_shape* shape, int32_t num_workgroups) {
  if (validate_shape(shape) != MLA_OK || num_workgroups < 1) return 0;
  return plan_words_bound(*shape, num_workgroups) * sizeof(int32_t);
}

uint64_t mla_workspace_bytes_bound(const mla_shape* shape, int32_t num_workgroups) {
  if (validate_shape(shape) != MLA_OK || num_workgroups < 1) return 0;
  return partial_bytes(2 * int64_t(num_workgroups));
}

int32_t mla_device_num_cus(int32_t device) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return -int32_t(MLA_ERR_HIP);
  return n;
}

mla_status mla_decode_plan(const mla_shape* shape, const int32_t* kv_lens_host,
                           const int32_t* q_lens_host, int32_t num_workgroups, void* plan_host,
                           uint64_t plan_bytes, mla_plan_info* info) {
  return host_plan(shape, kv_lens_host, q_lens_host, num_workgroups, plan_host, plan_bytes, info,
                   false);
}

mla_status mla_decode_plan_fixed(const mla_shape* shape, const int32_t* kv_lens_host,
                                 const int32_t* q_lens_host, int32_t num_workgroups,
                                 void* plan_host, uint64_t plan_bytes, mla_plan_info* info) {
  return host_plan(shape, kv_lens_host, q_lens_host, num_workgroups, plan_host, plan_bytes, info,
                   true);
}

mla_status mla_decode_plan_device(const mla_shape* shape, int32_t num_workgroups,
                                  const int32_t* kv_lens, const int32_t* q_lens, void* plan_dev,
                                  uint64_t plan_bytes, int32_t* status, mla_plan_info* info,
                                  mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  if (!plan_dev || !info || (shape->batch > 0 && !kv_lens)) return MLA_ERR_NULL_ARG;
  if (num_workgroups < 1) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(plan_dev) || (status && (reinterpret_cast<uintptr_t>(status) & 3u)))
    return MLA_ERR_MISALIGNED;
  int32_t G = num_workgroups, PH = 1, item_cost = 0;
  plan_launch_params(&G, &PH, &item_cost);
  mla_plan_info bounds{};
  fixed_launch_info(*shape, G, PH, &bounds);
  if (plan_bytes < bounds.plan_bytes) return MLA_ERR_PLAN_TOO_SMALL;
  const int64_t P = bounds.num_workgroups / PH;
  if (plan_lds_bytes(shape->batch, max_units(*shape), P) > kPlanLdsBytes) return MLA_ERR_UNSUPPORTED;
  PlanDeviceArgs a{};
  a.kv_lens = kv_lens;
  a.q_lens = q_lens;
  a.plan = static_cast<int32_t*>(plan_dev);
  a.status = status;
  a.plan_words = int64_t(bounds.plan_bytes / sizeof(int32_t));
  a.batch = shape->batch;
  a.num_heads = shape->num_heads;
  a.max_q_len = shape->max_q_len;
  a.causal = shape->causal;
  a.cap = shape->max_pages_per_seq * shape->page_size;
  a.P = int32_t(P);
  a.PH = PH;
  a.item_cost = item_cost;
  if (launch_plan(a, max_units(*shape), reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  *info = bounds;
  return MLA_OK;
}

mla_status mla_decode_fwd(const mla_shape* shape, const mla_plan_info* info, const void* plan_dev,
                          const void* q, const void* kv_cache, const float* kv_scale,
                          const int32_t* block_table, const int32_t* kv_lens,
                          const int32_t* q_lens, float softmax_scale, void* o, float* lse,
                          void* workspace, uint64_t workspace_bytes, mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  st = check_info(shape, info);
  if (st != MLA_OK) return st;
  if (shape->batch == 0 || info->num_items == 0) return MLA_OK;
  if (!plan_dev || !q || !kv_cache || !block_table || !kv_lens || !o) return MLA_ERR_NULL_ARG;
  if (shape->kv_dtype == MLA_KV_FP8_E4M3 && !kv_scale) return MLA_ERR_NULL_ARG;
  if (info->num_partials > 0 && !workspace) return MLA_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(o) || !aligned16(plan_dev) ||
      (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) ||
      (kv_scale && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return MLA_ERR_MISALIGNED;
  if (workspace_bytes < info->workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (!std::isfinite(softmax_scale)) return MLA_ERR_BAD_SHAPE;

  DecodeArgs a{};
  a.plan = static_cast<const int32_t*>(plan_dev);
  a.q = static_cast<const uint8_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.q_lens = q_lens;
  a.o = static_cast<uint8_t*>(o);
  a.lse = lse;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    uint64_t(info->num_partials) * kRowsPerBlock *
                                                        kDLatent * sizeof(float))
                         : nullptr;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.num_heads = shape->num_heads;
  a.max_q_len = shape->max_q_len;
  a.page_shift = ilog2(shape->page_size);
  a.max_pages = shape->max_pages_per_seq;
  a.causal = shape->causal;
  a.num_wg = info->num_workgroups;
  a.phases = info->phases;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (candidate_selected(info))
    return launch_decode_w8(a, shape->kv_dtype, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  if (split_selected(info))
    return launch_decode_split(a, shape->kv_dtype, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  if (qres_selected(shape))
    return launch_decode_qres(a, shape->kv_dtype, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  return launch_decode(a, shape->kv_dtype, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_check(const mla_shape* shape, const mla_plan_info* info,
                            const void* plan_dev, const int32_t* block_table,
                            const int32_t* kv_lens, const int32_t* q_lens, int32_t* err,
                            mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  st = check_info(shape, info);
  if (st != MLA_OK) return st;
  if (!plan_dev || !err || (shape->batch > 0 && (!block_table || !kv_lens)))
    return MLA_ERR_NULL_ARG;
  if (!aligned16(plan_dev) || (reinterpret_cast<uintptr_t>(err) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3u) || (reinterpret_cast<uintptr_t>(q_lens) & 3u))
    return MLA_ERR_MISALIGNED;
  if (info->plan_bytes < uint64_t(kHeaderWords) * sizeof(int32_t)) return MLA_ERR_BAD_PLAN;
  CheckArgs a{};
  a.plan = static_cast<const int32_t*>(plan_dev);
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.q_lens = q_lens;
  a.err = err;
  a.plan_words = int64_t(info->plan_bytes / sizeof(int32_t));
  a.batch = shape->batch;
  a.num_heads = shape->num_heads;
  a.max_q_len = shape->max_q_len;
  a.causal = shape->causal;
  a.page_size = shape->page_size;
  a.num_pages = shape->num_pages;
  a.max_pages = shape->max_pages_per_seq;
  a.num_wg = info->num_workgroups;
  a.phases = info->phases;
  a.num_partials = info->num_partials;
  return launch_check(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK
                                                                                : MLA_ERR_HIP;
}

mla_status mla_combine(const mla_shape* shape, const mla_plan_info* info, const void* plan_dev,
                       const void* workspace, uint64_t workspace_bytes, const int32_t* q_lens,
                       void* o, float* lse, mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  st = check_info(shape, info);
  if (st != MLA_OK) return st;
  if (info->num_combine == 0 || shape->batch == 0) return MLA_OK;
  if (!plan_dev || !workspace || !o) return MLA_ERR_NULL_ARG;
  if (!aligned16(o) || !aligned16(plan_dev) || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return MLA_ERR_MISALIGNED;
  if (workspace_bytes < info->workspace_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;

  CombineArgs a{};
  a.plan = static_cast<const int32_t*>(plan_dev);
  a.part_o = static_cast<const float*>(workspace);
  a.part_lse = reinterpret_cast<const float*>(static_cast<const char*>(workspace) +
                                              uint64_t(info->num_partials) * kRowsPerBlock *
                                                  kDLatent * sizeof(float));
  a.q_lens = q_lens;
  a.o = static_cast<uint8_t*>(o);
  a.lse = lse;
  a.num_heads = shape->num_heads;
  a.max_q_len = shape->max_q_len;
  a.num_combine = info->num_combine;
  const hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
  const bool bf16_partials = candidate_selected(info) || split_selected(info);
  const hipError_t e = bf16_partials ? launch_combine_bf16(a, cs) : launch_combine(a, cs);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_kv_append(const mla_shape* shape, int32_t max_new_tokens, const void* new_rows,
                         const int32_t* new_lens, const int32_t* block_table,
                         const int32_t* kv_lens, void* kv_cache, float* kv_scale,
                         int32_t* skipped, mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  if (max_new_tokens < 1) return MLA_ERR_BAD_SHAPE;
  if (int64_t(shape->batch) * max_new_tokens >= (int64_t(1) << 31)) return MLA_ERR_UNSUPPORTED;
  if (shape->batch == 0) return MLA_OK;
  if (!new_rows || !block_table || !kv_lens || !kv_cache) return MLA_ERR_NULL_ARG;
  if (shape->kv_dtype == MLA_KV_FP8_E4M3 && !kv_scale) return MLA_ERR_NULL_ARG;
  if (!aligned16(new_rows) || !aligned16(kv_cache) ||
      (kv_scale && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)) ||
      (skipped && (reinterpret_cast<uintptr_t>(skipped) & 3u)))
    return MLA_ERR_MISALIGNED;

  AppendArgs a{};
  a.src = static_cast<const uint8_t*>(new_rows);
  a.new_lens = new_lens;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.kv = static_cast<uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.skipped = skipped;
  a.batch = shape->batch;
  a.max_new = max_new_tokens;
  a.page_shift = ilog2(shape->page_size);
  a.max_pages = shape->max_pages_per_seq;
  a.num_pages = shape->num_pages;
  return launch_append(a, shape->kv_dtype, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status mla_tree_attend(const mla_shape* shape, const void* q, const void* kv_cache,
                           const float* kv_scale, const int32_t* block_table,
                           const int32_t* kv_lens, const int32_t* q_lens,
                           const uint32_t* tree_mask, float softmax_scale, void* o, float* lse,
                           mla_stream_t stream) {
  mla_status st = validate_shape(shape);
  if (st != MLA_OK) return st;
  if (shape->batch == 0) return MLA_OK;
  if (!q || !kv_cache || !block_table || !kv_lens || !tree_mask || !o || !lse)
    return MLA_ERR_NULL_ARG;
  if (shape->kv_dtype == MLA_KV_FP8_E4M3 && !kv_scale) return MLA_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(tree_mask) & 3u) ||
      (kv_scale && (reinterpret_cast<uintptr_t>(kv_scale) & 3u)))
    return MLA_ERR_MISALIGNED;
  if (!std::isfinite(softmax_scale)) return MLA_ERR_BAD_SHAPE;
  TreeArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.q_lens = q_lens;
  a.tree_mask = tree_mask;
  a.o = static_cast<uint8_t*>(o);
  a.lse = lse;
  a.sm_scale = softmax_scale;
  a.batch = shape->batch;
  a.num_heads = shape->num_heads;
  a.max_q_len = shape->max_q_len;
  a.page_shift = ilog2(shape->page_size);
  a.max_pages = shape->max_pages_per_seq;
  a.num_pages = shape->num_pages;
  a.kv_dtype = shape->kv_dtype;
  return launch_tree(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK
                                                                             : MLA_ERR_HIP;
}

// Shape checks shared by the two prefill entry points.
static mla_status validate_prefill(const mla_prefill_shape* s) {
  if (!s) return MLA_ERR_NULL_ARG;
  if (s->num_seqs < 0 || s->num_tokens < 0 || s->num_heads < 1 || s->num_blocks < 0)
    return MLA_ERR_BAD_SHAPE;
  if (s->d_qk != kPfDQK || s->d_v != kPfDV) return MLA_ERR_UNSUPPORTED;
  // a sequence holds at least one token per block it counts, and the packed
  // row and block indices stay in 32 bits inside the kernels
  if (int64_t(s->num_blocks) > int64_t(s->num_tokens) ||
      int64_t(s->num_tokens) * s->num_heads >= (int64_t(1) << 31) ||
      int64_t(s->num_blocks) * s->num_heads >= (int64_t(1) << 31))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int32_t mla_prefill_num_blocks(const int32_t* seqlens, int32_t num_seqs) {
  if (num_seqs < 0 || (num_seqs > 0 && !seqlens)) return -1;
  int64_t n = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (seqlens[s] < 0) return -1;
    n += (int64_t(seqlens[s]) + kPfBlock - 1) / kPfBlock;
    if (n > INT32_MAX) return -1;
  }
  return int32_t(n);
}

mla_status mla_prefill_quantize(const mla_prefill_shape* shape, const int32_t* cu_seqlens,
                                const void* q, const void* k, const void* v, int8_t* q_codes,
                                float* q_scale, int8_t* k_codes, float* k_scale,
                                uint8_t* v_codes, float* v_scale, mla_stream_t stream) {
  mla_status st = validate_prefill(shape);
  if (st != MLA_OK) return st;
  if (shape->num_tokens == 0) return MLA_OK;
  if (!cu_seqlens || !q || !k || !v || !q_codes || !q_scale || !k_codes || !k_scale ||
      (shape->num_blocks > 0 && (!v_codes || !v_scale)))
    return MLA_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_codes) ||
      !aligned16(k_codes) || (v_codes && !aligned16(v_codes)) ||
      ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
        reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(cu_seqlens)) & 3u))
    return MLA_ERR_MISALIGNED;
  PrefillQuantArgs a{};
  a.cu = cu_seqlens;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.qc = q_codes;
  a.qs = q_scale;
  a.kc = k_codes;
  a.ks = k_scale;
  a.vc = v_codes;
  a.vs = v_scale;
  a.num_seqs = shape->num_seqs;
  a.num_tokens = shape->num_tokens;
  a.num_heads = shape->num_heads;
  a.num_blocks = shape->num_blocks;
  return launch_prefill_quant(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

mla_status mla_prefill_attn(const mla_prefill_shape* shape, const int32_t* cu_seqlens,
                            const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                            const float* k_scale, const uint8_t* v_codes, const float* v_scale,
                            float softmax_scale, void* o, float* lse, mla_stream_t stream) {
  mla_status st = validate_prefill(shape);
  if (st != MLA_OK) return st;
  if (shape->num_tokens == 0 || shape->num_blocks == 0) return MLA_OK;
  if (!cu_seqlens || !q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale ||
      !o || !lse)
    return MLA_ERR_NULL_ARG;
  if (!aligned16(q_codes) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(o) ||
      ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
        reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(lse) |
        reinterpret_cast<uintptr_t>(cu_seqlens)) & 3u))
    return MLA_ERR_MISALIGNED;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_BAD_SHAPE;
  PrefillAttnArgs a{};
  a.cu = cu_seqlens;
  a.qc = q_codes;
  a.qs = q_scale;
  a.kc = k_codes;
  a.ks = k_scale;
  a.vc = v_codes;
  a.vs = v_scale;
  a.o = static_cast<uint8_t*>(o);
  a.lse = lse;
  a.sm_scale = softmax_scale;
  a.num_seqs = shape->num_seqs;
  a.num_tokens = shape->num_tokens;
  a.num_heads = shape->num_heads;
  a.num_blocks = shape->num_blocks;
  return launch_prefill_attn(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

}  // extern "C"
