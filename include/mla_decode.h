/*
 * mla_decode.h -- C ABI of the gfx950 weight-absorbed MLA decode library.
 *
 * The operation (weight-absorbed Multi-head Latent Attention decode over a
 * paged latent cache):
 *
 *   For sequence b with kv_len L_b keys and q_len q_b query tokens, every query
 *   row (token t, head h) holds an absorbed query q of width d_latent + d_rope
 *   (512 + 64).  Keys are the cached latent rows c_j = [latent_j | rope_j]
 *   gathered through the block table; values are the latent part latent_j
 *   (d_latent wide).  With vis = L_b - q_b + t + 1 when causal, else L_b:
 *
 *     s_j = softmax_scale * <q, c_j>            j < vis
 *     O   = sum_j softmax(s)_j * latent_j        (d_latent wide, bf16 out)
 *     LSE = ln sum_j exp(s_j)                    (fp32 out)
 *
 *   Sources: the decode-only weight-absorbed MLA path of the KsanaLLM 0.6.0
 *   page (prefill/decode disaggregation section); several draft tokens per
 *   sequence verified in one decode pass at the original batch size, from the
 *   PaddlePaddle 3.0 inference page (speculative decoding section); the
 *   softmax_lse output and the split-K key partition of the "FlashAttention-3
 *   in DeepSeek-R1" page (chapter 2); its per-token KV-cache scale (section
 *   3.1) and block table (section 4.1).
 *
 * Calling sequence (all device work is stream-ordered, no host sync inside):
 *
 *   1. mla_decode_plan   host only: split-KV schedule from host-side lengths.
 *   2. copy the plan image (plan_host, info.plan_bytes) to device memory.
 *      The caller copies: the planner makes no HIP call (it runs, and is
 *      tested, without a GPU), and one plan serves every layer of a decode
 *      step, so the caller decides when and on which stream it travels
 *      (from pinned memory with hipMemcpyAsync, keeping the host buffer alive
 *      until the stream passes the copy, or synchronously).  Plans built on
 *      the GPU need no copy: mla_decode_plan_device.
 *   3. mla_decode_fwd    main kernel: writes O/LSE for unsplit row blocks and
 *                        partial (O, LSE) into the workspace for split ones.
 *   4. mla_combine       merges the partials of split row blocks into O/LSE.
 *
 * mla_kv_append writes the step's new tokens into the cache; on the stream it
 * goes before mla_decode_fwd of the same step.
 *
 * Ownership: the caller allocates and owns every buffer; the library
 * allocates no memory and keeps no mutable state.  Buffers must stay alive
 * until the stream has passed the work that uses them.
 *
 * Errors: every call returns an mla_status; nothing throws across the ABI.
 * Values that live in device memory (block-table entries, device lengths) are
 * not validated: they must agree with the host lengths given to the planner
 * and index pages inside the pool, otherwise behaviour is undefined.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

/* hipStream_t; NULL means the null stream of the current device. */
typedef struct ihipStream_t* mla_stream_t;

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = 1,           /* a required pointer is NULL                 */
  MLA_ERR_BAD_SHAPE = 2,          /* sizes or host lengths are inconsistent     */
  MLA_ERR_UNSUPPORTED = 3,        /* valid, but no kernel is built for it       */
  MLA_ERR_MISALIGNED = 4,         /* a device pointer is not 16-byte aligned    */
  MLA_ERR_WORKSPACE_TOO_SMALL = 5,
  MLA_ERR_PLAN_TOO_SMALL = 6,     /* plan buffer smaller than needed            */
  MLA_ERR_BAD_PLAN = 7,           /* plan info does not match the shape         */
  MLA_ERR_HIP = 8                 /* a HIP runtime call or launch failed        */
} mla_status;

typedef enum mla_kv_dtype {
  MLA_KV_BF16 = 0,                /* cache rows are bf16, 2 * (d_latent + d_rope) bytes            */
  MLA_KV_FP8_E4M3 = 1             /* OCP e4m3fn rows plus one fp32 scale per cached token          */
} mla_kv_dtype;

/* Problem shape.  Built kernels: d_latent 512, d_rope 64, page_size a power of
 * two >= 16 (bf16) or >= 64 (fp8), 1 <= max_q_len <= MLA_MAX_Q_LEN, any
 * num_heads >= 1. */
typedef struct mla_shape {
  int32_t batch;              /* B sequences                                       */
  int32_t num_heads;          /* H query heads per token                           */
  int32_t max_q_len;          /* padded query tokens per sequence                  */
  int32_t d_latent;           /* value width = latent width (512)                  */
  int32_t d_rope;             /* rope width (64); query/key width = d_latent+d_rope */
  int32_t page_size;          /* cached tokens per page                            */
  int32_t num_pages;          /* pages in the pool                                 */
  int32_t max_pages_per_seq;  /* row length of the block table                     */
  int32_t kv_dtype;           /* mla_kv_dtype                                       */
  int32_t causal;             /* 1: token t sees keys j <= kv_len - q_len + t      */
} mla_shape;

#define MLA_MAX_Q_LEN 8

/* What a plan holds, returned by the planner and passed back to fwd/combine. */
typedef struct mla_plan_info {
  int32_t num_workgroups;     /* grid of the main kernel                           */
  int32_t num_items;          /* (sequence, row block, key range) work items       */
  int32_t num_partials;       /* partial (O, LSE) slots written to the workspace   */
  int32_t num_combine;        /* row blocks whose partials need merging            */
  int32_t tile_tokens;        /* keys per pipeline tile (16)                       */
  int32_t rows_per_block;     /* query rows per planner unit / partial slot (128)  */
  int32_t phases;             /* workgroups sharing a unit's keys: 1, 2 or 4       */
  uint64_t plan_bytes;        /* bytes of the plan image                           */
  uint64_t workspace_bytes;   /* workspace bytes this plan needs                   */
} mla_plan_info;

/* Library ABI version (MLA_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status status);

/* Upper bounds, for allocating before the lengths are known (the exact sizes
 * of a plan are info->plan_bytes and info->workspace_bytes, known once it is
 * built; hence "_bound").  num_workgroups as passed to mla_decode_plan (0 is
 * not accepted here: pass the CU count). */
uint64_t mla_plan_bytes_bound(const mla_shape* shape, int32_t num_workgroups);
uint64_t mla_workspace_bytes_bound(const mla_shape* shape, int32_t num_workgroups);

/* Number of compute units of a HIP device (the default workgroup count), or a
 * negative mla_status on failure.  Needs a GPU. */
int32_t mla_device_num_cus(int32_t device);

/*
 * Split-KV planner (host only, no HIP call).
 *
 * Splits sum_b ceil(q_b * H / 128) row blocks x ceil(L_b / 64) key rounds into
 * work items and deals them to num_workgroups persistent workgroups so that
 * each gets about the same number of rounds (a fixed per-item cost included).
 * A row block whose key range is cut gets one partial slot per piece and a
 * combine entry.  Key splitting with a log-sum-exp merge follows the split-K
 * remark of the FlashAttention-3 page (chapter 2).  By default every row block
 * is taken by one workgroup (info->phases = 1).  MLA_PHASES=2 or 4 (when it
 * divides num_workgroups) instead lets groups of 2 or 4 workgroups on one XCD
 * share a block (each takes 64 or 32 of its rows over the same keys, which then
 * come from HBM once); MLA_NUM_WORKGROUPS forces the workgroup count.  Both are
 * for tuning and tests.  MLA_LOG=1 prints one line per plan on stderr: the
 * shape, the counts of info, and the largest and mean number of keys a
 * workgroup takes (the hot path itself never logs).
 *
 *   kv_lens_host [B]  keys per sequence, including this step's q_b tokens.
 *   q_lens_host  [B]  query tokens per sequence (0..max_q_len); NULL means
 *                     every sequence has max_q_len tokens.
 *   num_workgroups    > 0; normally the device's CU count.
 *   plan_host         caller buffer of plan_bytes bytes (>= the bound above),
 *                     receives the plan image (int32 words, layout in the
 *                     library source; treat it as opaque).
 *   info              receives the plan summary.
 *
 * Errors: NULL_ARG; BAD_SHAPE if a length is negative, q_b > max_q_len,
 * L_b > max_pages_per_seq * page_size, or (causal) 0 < L_b < q_b;
 * UNSUPPORTED for shapes with no built kernel; PLAN_TOO_SMALL.
 */
mla_status mla_decode_plan(const mla_shape* shape, const int32_t* kv_lens_host,
                           const int32_t* q_lens_host, int32_t num_workgroups,
                           void* plan_host, uint64_t plan_bytes, mla_plan_info* info);

/*
 * Planner for a fixed launch shape, for callers that capture mla_decode_fwd +
 * mla_combine once (a HIP graph) and replay them with new lengths.
 *
 * Same arguments, errors and split as mla_decode_plan, with two differences:
 *   - the plan image always has num_workgroups workgroups (rounded down to a
 *     multiple of info->phases); those the split does not need get no items;
 *   - *info holds launch bounds that every lengths of this shape satisfy, not
 *     this plan's counts: num_workgroups as above, num_partials =
 *     2 * num_workgroups (each processor boundary cuts at most one unit, and
 *     a cut unit has one partial per piece), num_combine = B * ceil(max_q_len
 *     * H / 128), workspace_bytes and plan_bytes for those bounds.
 * The plan image records its real counts, and the kernels read them on the
 * device.  So one info, one plan buffer of info->plan_bytes and one workspace
 * serve every call of the shape: before each replay copy info->plan_bytes
 * bytes of the new plan_host into the same device buffer (words past the
 * image are never read), and keep kv_lens/q_lens in the same device buffers.
 * phases come from MLA_PHASES as for mla_decode_plan and must not change
 * between the capture and the replays.
 */
mla_status mla_decode_plan_fixed(const mla_shape* shape, const int32_t* kv_lens_host,
                                 const int32_t* q_lens_host, int32_t num_workgroups,
                                 void* plan_host, uint64_t plan_bytes, mla_plan_info* info);

/*
 * Device-side planner: the plan mla_decode_plan_fixed would make, built on the
 * GPU from device-resident lengths (for lengths produced on the GPU, such as
 * accepted draft tokens, so that they need not be copied to the host).
 *
 *   kv_lens, q_lens  [B] int32 device arrays as for mla_decode_fwd (q_lens may
 *                    be NULL: every sequence has max_q_len tokens).
 *   plan_dev         device buffer of plan_bytes >= the info->plan_bytes this
 *                    call returns (mla_plan_bytes_bound), 16-byte aligned;
 *                    receives the plan image (stream-ordered).
 *   status           optional int32 device word: MLA_OK, or MLA_ERR_BAD_SHAPE
 *                    when a length fails the checks of mla_decode_plan (then
 *                    the plan has no items and the decode writes nothing).
 *   info             receives the fixed-shape launch bounds (host side, at
 *                    once), identical to mla_decode_plan_fixed's.
 *
 * One workgroup runs the host planner's loops, so the image equals the host
 * one bit for bit.  Its time grows with the number of 128-row units (tens of
 * microseconds at a few hundred); a decode step plans once for all layers.
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED, PLAN_TOO_SMALL, UNSUPPORTED (the
 * shape's lengths, units and pieces exceed the planner's 128 KB of LDS:
 * about 2000 units), HIP.
 */
mla_status mla_decode_plan_device(const mla_shape* shape, int32_t num_workgroups,
                                  const int32_t* kv_lens, const int32_t* q_lens, void* plan_dev,
                                  uint64_t plan_bytes, int32_t* status, mla_plan_info* info,
                                  mla_stream_t stream);

/*
 * Main decode kernel launch: the attention of the formula at the top of this
 * file for every valid query row, over the keys of its work items.  The
 * operation is the decode-time weight-absorbed MLA of the KsanaLLM 0.6.0 page
 * (prefill/decode disaggregation section: the query arrives absorbed, O
 * leaves in latent space); q_len > 1 is the draft verification of the
 * PaddlePaddle 3.0 inference page (speculative decoding section), token t
 * seeing keys j <= L_b - q_b + t; the natural-log LSE output is the
 * softmax_lse of the FlashAttention-3 in DeepSeek-R1 page (chapter 2), whose
 * split-K partition this kernel applies to row blocks the plan cut; fp8
 * caches carry that page's per-token scale (section 3.1).
 *
 *   plan_dev     device copy of the plan image described by *info.
 *   q            [B, max_q_len, H, d_latent + d_rope] bf16, row-major.  Rows
 *                t >= q_lens[b] are never read.
 *   kv_cache     [num_pages, page_size, d_latent + d_rope] bf16, or e4m3 bytes
 *                for MLA_KV_FP8_E4M3.  Slots past kv_len and pages not in the
 *                sequence's first ceil(kv_len / page_size) block-table entries
 *                never influence the result.
 *   kv_scale     [num_pages, page_size] fp32 per-token scales (fp8 only, else
 *                ignored; may be NULL for bf16).
 *   block_table  [B, max_pages_per_seq] int32 physical page ids.
 *   kv_lens, q_lens  [B] int32 device copies of the planner's lengths
 *                (q_lens may be NULL: every sequence has max_q_len tokens).
 *   softmax_scale    multiplies <q, c_j>.
 *   o            [B, max_q_len, H, d_latent] bf16 output; rows t >= q_b untouched.
 *   lse          [B, max_q_len, H] fp32 natural-log LSE, or NULL.
 *   workspace    >= info->workspace_bytes, 256-byte aligned; holds partials:
 *                fp32 O [num_partials][128][d_latent], then fp32 LSE
 *                [num_partials][128].
 *
 * Kernel choice: the environment variable MLA_DECODE_KERNEL=w8 selects, for
 * one-phase plans, a candidate kernel with two waves per SIMD and 16 query
 * rows per wave (not yet run on a GPU).  It writes the partial O as bf16
 * [num_partials][128][d_latent] in the first half of the same area (the LSE
 * where it always is), and mla_combine, seeing the same setting, merges that
 * layout: both calls of a step must see the same value.
 * MLA_DECODE_KERNEL=split selects, for one-phase plans, a second
 * two-waves-per-SIMD candidate in which each pair of waves shares 32 query
 * rows (half the dimensions and half the output columns each); it writes and
 * merges the same bf16 partials, and is not yet run on a GPU either.  Both
 * take bf16 and e4m3 caches.  MLA_DECODE_KERNEL=qres selects, for e4m3
 * caches, the library's e4m3 kernels rebuilt with the query fragments
 * resident before the key loop (same partials, same merge; not yet run on a
 * GPU either).
 *
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, BAD_PLAN,
 * WORKSPACE_TOO_SMALL, HIP (launch failure).
 */
mla_status mla_decode_fwd(const mla_shape* shape, const mla_plan_info* info,
                          const void* plan_dev, const void* q, const void* kv_cache,
                          const float* kv_scale, const int32_t* block_table,
                          const int32_t* kv_lens, const int32_t* q_lens,
                          float softmax_scale, void* o, float* lse,
                          void* workspace, uint64_t workspace_bytes, mla_stream_t stream);

/*
 * Merge of split row blocks (the log-sum-exp combination that makes the
 * split-K key partition of the FlashAttention-3 in DeepSeek-R1 page, chapter
 * 2, exact up to rounding): for each combine entry of the plan,
 *   LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) * O_s  -> bf16,
 * reading the workspace partials laid out as described for mla_decode_fwd
 * (bf16 O under MLA_DECODE_KERNEL=w8 or MLA_DECODE_KERNEL=split for
 * one-phase plans, fp32 otherwise).
 * A row whose partials are all empty (LSE_s = -inf) gets O = 0, LSE = -inf.
 * No-op when info->num_combine == 0.  Must run after mla_decode_fwd on the
 * same stream (or after the caller filled the partials itself).
 */
mla_status mla_combine(const mla_shape* shape, const mla_plan_info* info,
                       const void* plan_dev, const void* workspace,
                       uint64_t workspace_bytes, const int32_t* q_lens,
                       void* o, float* lse, mla_stream_t stream);

/*
 * Debug validation of the device-resident inputs mla_decode_fwd and
 * mla_combine take on trust (a checked mode for callers that assemble block
 * tables, lengths and plans on the device, or replay a captured launch with a
 * plan image of their own).  Nothing here is needed on the fast path; the
 * Python binding runs it before every decode when MLA_DEBUG_CHECK=1.
 *
 * The decode kernels read pages through the block table (the page layout of
 * the FlashAttention-3 in DeepSeek-R1 page, section 4.1) and key ranges from
 * the split-K plan (same page, chapter 2) without checking them: a plan built
 * for other lengths (a stale image after the lengths changed) or a page id
 * outside the pool makes them read outside the cache.  This call checks, on
 * the device and in one workgroup, with every read bounded by sizes it has
 * already checked:
 *
 *   MLA_CHECK_PLAN         the image's header matches *info (magic, version,
 *                          workgroups, phases, partials within the workspace
 *                          layout) and its tables fit info->plan_bytes; the
 *                          workgroup item ranges are ordered and cover the items;
 *   MLA_CHECK_LENGTHS      every kv_lens[b], q_lens[b] passes the planner's
 *                          checks (0 <= q_b <= max_q_len, 0 <= L_b <=
 *                          max_pages_per_seq * page_size, causal: L_b >= q_b
 *                          when q_b > 0);
 *   MLA_CHECK_BLOCK_TABLE  block_table[b][j] is in [0, num_pages) for every
 *                          page j < ceil(L_b / page_size) a sequence uses;
 *   MLA_CHECK_ITEM         every work item names a sequence of the batch, keys
 *                          0 <= k0 <= k1 <= L_b with k0 on a 64-key boundary,
 *                          a first row below q_b * H and a partial slot the
 *                          plan has; and the items together cover every
 *                          (key, query row) pair of the lengths exactly as
 *                          often as a plan for them does (index = the item
 *                          count).  A stale plan fails here;
 *   MLA_CHECK_COMBINE      every combine entry names rows that exist and
 *                          partial slots the plan has.
 *
 *   err   int32[2] device (4-byte aligned): receives the lowest failing check
 *         code (MLA_CHECK_OK = 0 if all pass) and the index it concerns (the
 *         sequence for LENGTHS and BLOCK_TABLE, the item or combine entry, the
 *         workgroup for a broken item range; saturated at 2^24 - 1).  Written
 *         stream-ordered; the caller reads it after the stream passes it.
 *
 * Other arguments as for mla_decode_fwd (plan_dev holds info->plan_bytes
 * bytes).  Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, BAD_PLAN (the
 * info itself is inconsistent with the shape), HIP.
 */
typedef enum mla_check_code {
  MLA_CHECK_OK = 0,
  MLA_CHECK_PLAN = 1,
  MLA_CHECK_LENGTHS = 2,
  MLA_CHECK_BLOCK_TABLE = 3,
  MLA_CHECK_ITEM = 4,
  MLA_CHECK_COMBINE = 5
} mla_check_code;

mla_status mla_decode_check(const mla_shape* shape, const mla_plan_info* info,
                            const void* plan_dev, const int32_t* block_table,
                            const int32_t* kv_lens, const int32_t* q_lens, int32_t* err,
                            mla_stream_t stream);

/*
 * Tree-shaped drafts: the draft tokens' part of the attention, merged into
 * the result of a decode over the cached prefix.  Sources: all drafts of a
 * sequence verified in one decode pass (PaddlePaddle 3.0 inference page,
 * speculative decoding section); EAGLE-style top-k drafting, whose drafts
 * form a tree (Dewu DeepSeek deployment slides, MTP); the merge is the
 * log-sum-exp combination of split-K (FlashAttention-3 in DeepSeek-R1 page,
 * chapter 2).
 *
 * With EAGLE-style speculative decoding (top-k candidates per step) the
 * q_b draft tokens of sequence b form a tree and are verified in one pass:
 * token t sees the L_b - q_b cached prefix keys and the drafts on its branch.
 * tree_mask [B, max_q_len] uint32 (device): bit k of word t set means token t
 * sees draft k (cache position L_b - q_b + k); bits k >= q_b are ignored.
 * A lower-triangular mask is the ordinary causal decode.
 *
 * Calling sequence for one step (all on one stream):
 *   1. plan and run mla_decode_fwd + mla_combine over the prefix only: the
 *      same shape with causal = 0, kv_lens_prefix[b] = kv_lens[b] - q_lens[b],
 *      and lse not NULL;
 *   2. mla_tree_attend with the full kv_lens: for every row (b, t < q_b, h)
 *      it computes the scores of the visible drafts, and replaces O and LSE
 *      (read from step 1) by the log-sum-exp merge of both parts:
 *        LSE = ln(e^LSE_prefix + sum_k e^(s_k)),
 *        O   = e^(LSE_prefix - LSE) O_prefix + sum_k e^(s_k - LSE) latent_k.
 *      Rows t >= q_b are untouched; a row whose mask names no draft keeps the
 *      prefix result.  Draft positions or pages outside the pool are skipped.
 * The merge reads the prefix O as bf16, so the result carries one extra bf16
 * rounding of the prefix part.
 *
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, HIP.
 */
mla_status mla_tree_attend(const mla_shape* shape, const void* q, const void* kv_cache,
                           const float* kv_scale, const int32_t* block_table,
                           const int32_t* kv_lens, const int32_t* q_lens,
                           const uint32_t* tree_mask, float softmax_scale, void* o, float* lse,
                           mla_stream_t stream);

/*
 * Cache append: writes this step's new tokens into the paged cache, the
 * write that precedes the decode of every step.
 *
 * Token t (t < n_b) of sequence b goes to position p = kv_lens[b] - n_b + t
 * (kv_lens counts the new tokens, as for the decode), i.e. slot p % page_size
 * of page block_table[b][p / page_size] (the page/block-table layout of the
 * FlashAttention-3 in DeepSeek-R1 page, section 4.1).
 *
 *   shape          the decode's shape: batch, page_size, num_pages,
 *                  max_pages_per_seq and kv_dtype are used (num_heads,
 *                  max_q_len and causal are validated but not used).
 *   max_new_tokens padded new tokens per sequence (>= 1; may exceed
 *                  MLA_MAX_Q_LEN, e.g. for a prompt's tokens).
 *   new_rows       [B, max_new_tokens, d_latent + d_rope] bf16, row-major: the
 *                  latent + rope row of each new token.  Rows t >= n_b are not
 *                  read.
 *   new_lens       [B] int32 device n_b, or NULL (every n_b = max_new_tokens).
 *   block_table, kv_lens  as for mla_decode_fwd (device).
 *   kv_cache       [num_pages, page_size, d_latent + d_rope] bf16 or e4m3 bytes;
 *                  only the slots of new tokens are written.
 *   kv_scale       [num_pages, page_size] fp32 (e4m3 only, else ignored).
 *                  For e4m3 each row is stored as code = RNE(x / s), the
 *                  magnitude clamped to 448, with s = max|x| / 448 in fp32
 *                  (1 for an all-zero row) written to kv_scale: one symmetric
 *                  scale per token, the per-token absmax calibration of the
 *                  FlashAttention-3 page (section 3.1) over the e4m3 range.
 *                  Values must be finite.
 *   skipped        optional int32 device counter (may be NULL): incremented
 *                  once for each new token whose position falls outside
 *                  [0, max_pages_per_seq * page_size) or whose page id falls
 *                  outside [0, num_pages), and for every row of a sequence
 *                  with n_b > max_new_tokens; such rows are not written.  The
 *                  caller zeroes it.
 *
 * Rows of different tokens must not share a slot (a block table never maps
 * two positions to one slot); nothing else in the cache changes.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED (new_rows, kv_cache
 * not 16-byte aligned), HIP (launch failure).  B = 0 is a no-op.
 */
mla_status mla_kv_append(const mla_shape* shape, int32_t max_new_tokens, const void* new_rows,
                         const int32_t* new_lens, const int32_t* block_table,
                         const int32_t* kv_lens, void* kv_cache, float* kv_scale,
                         int32_t* skipped, mla_stream_t stream);

/*
 * Quantized causal prefill, SageAttention style (PaddlePaddle 3.0 inference
 * page, long-sequence inference: Q and K quantized to INT8 and V to FP8 on the
 * fly, the INT32 products converted to FP32 and dequantized, an online softmax,
 * P quantized to FP8 and multiplied with the FP8 V, V's scale taken off
 * afterwards; head dim 192 for Q and K, 128 for V, as in DeepSeek's prefill).
 *
 * Sequences are packed along the token axis: sequence s owns tokens
 * cu_seqlens[s] .. cu_seqlens[s + 1] - 1 (N_s of them), and token i of a
 * sequence sees keys 0..i of the same sequence.  For each (token, head):
 *
 *   s_j = (qc . kc_j) * q_scale * k_scale(block of j) * softmax_scale  (INT32 exact)
 *   keys taken in blocks of 128 from the sequence start; per block
 *     m' = max(m, max s_j),  a = e^(m - m'),  P_j = e^(s_j - m'),
 *     l = a l + sum_j P_j,   acc = a acc + sum_j e4m3(448 P_j) * vc_j * v_scale(block)
 *   O = acc / (448 l)  (bf16, round to nearest even),  LSE = m + ln l (fp32)
 *
 * Calling sequence: mla_prefill_quantize, then mla_prefill_attn, on one
 * stream.  Blocks: a sequence has ceil(N_s / 128) 128-token blocks; they are
 * numbered over all sequences in order (num_blocks in total, see
 * mla_prefill_num_blocks).
 */
typedef struct mla_prefill_shape {
  int32_t num_seqs;    /* S >= 0 */
  int32_t num_tokens;  /* T = cu_seqlens[S] */
  int32_t num_heads;   /* H >= 1 */
  int32_t d_qk;        /* 192 */
  int32_t d_v;         /* 128 */
  int32_t num_blocks;  /* sum_s ceil(N_s / 128) */
} mla_prefill_shape;

/* Number of 128-token blocks of S sequences with host lengths seqlens[S]
 * (>= 0); -1 if a length is negative or the sum overflows int32. */
int32_t mla_prefill_num_blocks(const int32_t* seqlens, int32_t num_seqs);

/*
 * Quantizes packed bf16 Q, K, V (all device pointers, 16-byte aligned).
 *
 *   cu_seqlens  [S + 1] int32, device: 0 = cu[0] <= cu[1] <= ... <= cu[S] = T.
 *   q, k        [T, H, 192] bf16;  v  [T, H, 128] bf16.  Values must be finite.
 *   q_codes, k_codes  [T, H, 192] int8: code = RNE(x / s) clamped to +-127,
 *               s = max|x| / 127 in fp32 (1 if the maximum is 0), taken over
 *               each (token, head) row for Q (q_scale [T, H] fp32) and over
 *               each (128-token block, head) for K (k_scale [num_blocks, H]).
 *   v_codes     [num_blocks, H, 128 channels, 128 keys] e4m3 bytes: for block
 *               b of a sequence and channel c, code = the e4m3 value nearest
 *               (ties to even) to v / s, s the smallest power of two 2^e
 *               (e >= -127) with max|v| / s <= 448 over the block's tokens in
 *               channel c (2^0 if zero), written to v_scale [num_blocks, H, 128]
 *               fp32 (powers of two: the fp8 matrix instruction applies them
 *               as e8m0 scales).  Within a (block, head,
 *               channel) row of 128 bytes, key k = 16 a + 4 g + r
 *               (a < 8, g < 4, r < 4) sits at byte 32 g + 4 a + r: the order
 *               in which the PV matrix instruction takes them.  Keys past
 *               the sequence's end hold code 0.
 *
 * Q and K quotients are correctly rounded fp32 divisions; V's are exact.
 * Errors: NULL_ARG,
 * BAD_SHAPE (negative sizes, d_qk != 192 or d_v != 128 is UNSUPPORTED),
 * MISALIGNED, HIP.  Blocks of a sequence whose cu_seqlens entries are out of
 * order or past T, or past num_blocks, are not written.  T = 0 is a no-op.
 */
mla_status mla_prefill_quantize(const mla_prefill_shape* shape, const int32_t* cu_seqlens,
                                const void* q, const void* k, const void* v, int8_t* q_codes,
                                float* q_scale, int8_t* k_codes, float* k_scale,
                                uint8_t* v_codes, float* v_scale, mla_stream_t stream);

/*
 * The attention of the formula above, from mla_prefill_quantize's outputs.
 *
 *   o    [T, H, 128] bf16 (device, 16-byte aligned); lse [T, H] fp32 (device).
 *   softmax_scale  finite and > 0 (BAD_SHAPE otherwise).
 *
 * Two workgroups per (128-token query block, head), 64 queries each; the P V
 * product runs on e4m3 matrix instructions and the Q K product on INT8 ones.
 * Errors as for
 * mla_prefill_quantize; rows of sequences with inconsistent cu_seqlens are
 * not written.
 */
mla_status mla_prefill_attn(const mla_prefill_shape* shape, const int32_t* cu_seqlens,
                            const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                            const float* k_scale, const uint8_t* v_codes, const float* v_scale,
                            float softmax_scale, void* o, float* lse, mla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
