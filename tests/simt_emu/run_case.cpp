// Runs one decode case through the library's C ABI with the kernels executed
// by the lane-thread emulator.  Every buffer is allocated at its exact size,
// so AddressSanitizer reports any access of the kernels outside the inputs,
// outputs, plan or workspace.
//
// usage: run_case <in.bin> <out.bin>
//   in.bin : int32 header[12] = {magic, B, H, qmax, page_size, num_pages,
//            max_pages, kv_dtype, causal, num_workgroups, has_q_lens,
//            fixed_shape (1: plan with mla_decode_plan_fixed)},
//            float scale, then q (B*qmax*H*576 bf16), kv cache (pages*P*576
//            elements), kv scales (pages*P fp32, e4m3 only), block table
//            (B*max_pages int32), kv_lens (B int32), q_lens (B int32, if any)
//   out.bin: int32 {num_items, num_partials, num_combine, phases}, then O
//            (B*qmax*H*512 bf16) and LSE (B*qmax*H fp32)
//
// A tree-draft case has its own magic and the decode layout, followed by the
// tree mask words (B*qmax uint32): the prefix (kv_len - q_len keys) goes
// through plan + mla_decode_fwd + mla_combine, non-causal, and
// mla_tree_attend merges the drafts; the output is as for a decode case.
//
// A device-planner case (mla_decode_plan_device) has its own magic:
//   in.bin : int32 header[12] = {magic, B, H, qmax, page_size, num_pages,
//            max_pages, causal, num_workgroups, has_q_lens, 0, 0}, then
//            kv_lens, q_lens (if any)
//   out.bin: int32 call status, plan status, image words, then the image
//
// A cache-append case (mla_kv_append) has its own magic:
//   in.bin : int32 header[12] = {magic, B, max_new, page_size, num_pages,
//            max_pages, kv_dtype, has_new_lens, has_skipped, 0, 0, 0}, then
//            the new rows (B*max_new*576 bf16), kv cache, kv scales (e4m3
//            only), block table, kv_lens, new_lens (if any)
//   out.bin: int32 skipped count (-1 without a counter), then the kv cache
//            and, for e4m3, the kv scales
//
// A debug-check case (mla_decode_plan, then mla_decode_check) has its own
// magic; the plan is built from its own lengths, so a stale plan can be
// checked against new device lengths, and words of the image can be poked:
//   in.bin : int32 header[12] = {magic, B, H, qmax, page_size, num_pages,
//            max_pages, kv_dtype, causal, num_workgroups, has_q_lens,
//            n_pokes}, then the planner's kv_lens and q_lens (if any), the
//            device kv_lens and q_lens (if any), the block table, and n_pokes
//            (word index, value) pairs applied to the plan image
//   out.bin: int32 {call status, err[0], err[1]}
//
// A quantized-prefill case (mla_prefill_quantize + mla_prefill_attn) has its
// own magic:
//   in.bin : int32 header[12] = {magic, S, T, H, num_blocks, 0, ...}, float
//            softmax scale, cu_seqlens (S+1 int32), q, k (T*H*192 bf16),
//            v (T*H*128 bf16)
//   out.bin: q codes, q scales (T*H), k codes, k scales (blocks*H), v codes,
//            v scales, O
//            (T*H*128 bf16), LSE (T*H fp32), each at its exact size
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla_decode.h"

namespace {

[[noreturn]] void die(const char* m) {
  std::fprintf(stderr, "run_case: %s\n", m);
  std::exit(2);
}

void* exact_alloc(size_t n, size_t align = 16) {
  if (n == 0) return nullptr;
  const size_t rounded = (n + align - 1) / align * align;
  if (rounded != n) die("buffer size is not a multiple of its alignment");
  void* p = std::aligned_alloc(align, n);
  if (!p) die("out of memory");
  return p;
}

void read_into(FILE* f, void* dst, size_t n) {
  if (n && std::fread(dst, 1, n, f) != n) die("short input file");
}

int run_append(FILE* f, const int32_t* hd, const char* out_path) {
  mla_shape s{};
  s.batch = hd[1];
  s.num_heads = 1;
  s.max_q_len = 1;
  s.d_latent = 512;
  s.d_rope = 64;
  s.page_size = hd[3];
  s.num_pages = hd[4];
  s.max_pages_per_seq = hd[5];
  s.kv_dtype = hd[6];
  s.causal = 1;
  const int max_new = hd[2];
  const bool has_nl = hd[7] != 0, has_sk = hd[8] != 0;
  const bool fp8 = s.kv_dtype == MLA_KV_FP8_E4M3;
  const size_t src_bytes = size_t(s.batch) * max_new * 576 * 2;
  const size_t kv_bytes = size_t(s.num_pages) * s.page_size * 576 * (fp8 ? 1 : 2);
  const size_t sc_bytes = fp8 ? size_t(s.num_pages) * s.page_size * 4 : 0;
  void* src = exact_alloc(src_bytes);
  void* kv = exact_alloc(kv_bytes);
  float* ksc = fp8 ? static_cast<float*>(exact_alloc(sc_bytes, 4)) : nullptr;
  int32_t* bt = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * s.max_pages_per_seq * 4, 4));
  int32_t* kvl = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4));
  int32_t* nl = has_nl ? static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4)) : nullptr;
  int32_t* sk = has_sk ? static_cast<int32_t*>(exact_alloc(4, 4)) : nullptr;
  read_into(f, src, src_bytes);
  read_into(f, kv, kv_bytes);
  if (ksc) read_into(f, ksc, sc_bytes);
  read_into(f, bt, size_t(s.batch) * s.max_pages_per_seq * 4);
  read_into(f, kvl, size_t(s.batch) * 4);
  if (nl) read_into(f, nl, size_t(s.batch) * 4);
  std::fclose(f);
  if (sk) *sk = 0;
  const mla_status st = mla_kv_append(&s, max_new, src, nl, bt, kvl, kv, ksc, sk, nullptr);
  if (st != MLA_OK) die("mla_kv_append failed");
  FILE* g = std::fopen(out_path, "wb");
  if (!g) die("cannot open output");
  const int32_t skipped = sk ? *sk : -1;
  std::fwrite(&skipped, 1, sizeof skipped, g);
  std::fwrite(kv, 1, kv_bytes, g);
  if (ksc) std::fwrite(ksc, 1, sc_bytes, g);
  std::fclose(g);
  std::free(src);
  std::free(kv);
  std::free(ksc);
  std::free(bt);
  std::free(kvl);
  std::free(nl);
  std::free(sk);
  return 0;
}

int run_prefill(FILE* f, const int32_t* hd, const char* out_path) {
  mla_prefill_shape s{};
  s.num_seqs = hd[1];
  s.num_tokens = hd[2];
  s.num_heads = hd[3];
  s.d_qk = 192;
  s.d_v = 128;
  s.num_blocks = hd[4];
  float scale = 0.f;
  read_into(f, &scale, sizeof scale);
  const size_t TH = size_t(s.num_tokens) * s.num_heads;
  const size_t BH = size_t(s.num_blocks) * s.num_heads;
  int32_t* cu = static_cast<int32_t*>(exact_alloc(size_t(s.num_seqs + 1) * 4, 4));
  void* q = exact_alloc(TH * 192 * 2);
  void* k = exact_alloc(TH * 192 * 2);
  void* v = exact_alloc(TH * 128 * 2);
  int8_t* qc = static_cast<int8_t*>(exact_alloc(TH * 192));
  int8_t* kc = static_cast<int8_t*>(exact_alloc(TH * 192));
  float* qs = static_cast<float*>(exact_alloc(TH * 4, 4));
  float* ks = static_cast<float*>(exact_alloc(BH * 4, 4));
  uint8_t* vc = static_cast<uint8_t*>(exact_alloc(BH * 128 * 128));
  float* vs = static_cast<float*>(exact_alloc(BH * 128 * 4));
  void* o = exact_alloc(TH * 128 * 2);
  float* lse = static_cast<float*>(exact_alloc(TH * 4, 4));
  read_into(f, cu, size_t(s.num_seqs + 1) * 4);
  read_into(f, q, TH * 192 * 2);
  read_into(f, k, TH * 192 * 2);
  read_into(f, v, TH * 128 * 2);
  std::fclose(f);
  // sentinels: rows the kernels do not write keep them
  if (TH) {
    std::memset(o, 0xC1, TH * 128 * 2);
    for (size_t i = 0; i < TH; ++i) lse[i] = 12345.f;
  }
  mla_status st = mla_prefill_quantize(&s, cu, q, k, v, qc, qs, kc, ks, vc, vs, nullptr);
  if (st != MLA_OK) die("mla_prefill_quantize failed");
  st = mla_prefill_attn(&s, cu, qc, qs, kc, ks, vc, vs, scale, o, lse, nullptr);
  if (st != MLA_OK) die("mla_prefill_attn failed");
  FILE* g = std::fopen(out_path, "wb");
  if (!g) die("cannot open output");
  std::fwrite(qc, 1, TH * 192, g);
  std::fwrite(qs, 1, TH * 4, g);
  std::fwrite(kc, 1, TH * 192, g);
  std::fwrite(ks, 1, BH * 4, g);
  std::fwrite(vc, 1, BH * 128 * 128, g);
  std::fwrite(vs, 1, BH * 128 * 4, g);
  std::fwrite(o, 1, TH * 128 * 2, g);
  std::fwrite(lse, 1, TH * 4, g);
  std::fclose(g);
  for (void* p : {static_cast<void*>(cu), q, k, v, static_cast<void*>(qc),
                  static_cast<void*>(kc), static_cast<void*>(qs), static_cast<void*>(ks),
                  static_cast<void*>(vc), static_cast<void*>(vs), o, static_cast<void*>(lse)})
    std::free(p);
  return 0;
}

int run_plan(FILE* f, const int32_t* hd, const char* out_path) {
  mla_shape s{};
  s.batch = hd[1];
  s.num_heads = hd[2];
  s.max_q_len = hd[3];
  s.d_latent = 512;
  s.d_rope = 64;
  s.page_size = hd[4];
  s.num_pages = hd[5];
  s.max_pages_per_seq = hd[6];
  s.kv_dtype = MLA_KV_BF16;
  s.causal = hd[7];
  const int nwg = hd[8];
  const bool has_ql = hd[9] != 0;
  int32_t* kvl = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4));
  int32_t* ql = has_ql ? static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4)) : nullptr;
  read_into(f, kvl, size_t(s.batch) * 4);
  if (ql) read_into(f, ql, size_t(s.batch) * 4);
  std::fclose(f);
  const uint64_t bound = mla_plan_bytes_bound(&s, nwg);
  if (bound == 0) die("shape rejected by mla_plan_bytes_bound");
  // the "device" plan buffer, exactly the bound, filled with a pattern
  int32_t* plan = static_cast<int32_t*>(exact_alloc((bound + 15) / 16 * 16, 16));
  for (uint64_t w = 0; w < (bound + 15) / 16 * 4; ++w) plan[w] = 0x5A5A5A5A;
  int32_t* status = static_cast<int32_t*>(exact_alloc(4, 4));
  *status = -1;
  mla_plan_info info{};
  const mla_status st = mla_decode_plan_device(&s, nwg, kvl, ql, plan, (bound + 15) / 16 * 16,
                                               status, &info, nullptr);
  FILE* g = std::fopen(out_path, "wb");
  if (!g) die("cannot open output");
  const int32_t words = int32_t(bound / 4);
  const int32_t meta[3] = {int32_t(st), *status, words};
  std::fwrite(meta, 1, sizeof meta, g);
  std::fwrite(plan, 1, size_t(words) * 4, g);
  std::fclose(g);
  std::free(kvl);
  std::free(ql);
  std::free(plan);
  std::free(status);
  return 0;
}

int run_check(FILE* f, const int32_t* hd, const char* out_path) {
  mla_shape s{};
  s.batch = hd[1];
  s.num_heads = hd[2];
  s.max_q_len = hd[3];
  s.d_latent = 512;
  s.d_rope = 64;
  s.page_size = hd[4];
  s.num_pages = hd[5];
  s.max_pages_per_seq = hd[6];
  s.kv_dtype = hd[7];
  s.causal = hd[8];
  const int nwg = hd[9];
  const bool has_ql = hd[10] != 0;
  const int n_pokes = hd[11];
  const size_t B4 = size_t(s.batch) * 4;
  std::vector<int32_t> plan_kvl(s.batch), plan_ql(has_ql ? s.batch : 0);
  read_into(f, plan_kvl.data(), B4);
  if (has_ql) read_into(f, plan_ql.data(), B4);
  int32_t* kvl = static_cast<int32_t*>(exact_alloc(B4, 4));
  int32_t* ql = has_ql ? static_cast<int32_t*>(exact_alloc(B4, 4)) : nullptr;
  int32_t* bt = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * s.max_pages_per_seq * 4, 4));
  read_into(f, kvl, B4);
  if (ql) read_into(f, ql, B4);
  read_into(f, bt, size_t(s.batch) * s.max_pages_per_seq * 4);
  std::vector<int32_t> pokes(size_t(2) * n_pokes);
  read_into(f, pokes.data(), pokes.size() * 4);
  std::fclose(f);
  const uint64_t bound = mla_plan_bytes_bound(&s, nwg);
  if (bound == 0) die("shape rejected by mla_plan_bytes_bound");
  std::vector<int32_t> host_plan(bound / 4 + 1);
  mla_plan_info info{};
  if (mla_decode_plan(&s, plan_kvl.data(), has_ql ? plan_ql.data() : nullptr, nwg,
                      host_plan.data(), host_plan.size() * 4, &info) != MLA_OK)
    die("mla_decode_plan failed");
  int32_t* plan = static_cast<int32_t*>(exact_alloc(info.plan_bytes));
  std::memcpy(plan, host_plan.data(), info.plan_bytes);
  if (const char* dump = std::getenv("EMU_PLAN_OUT")) {   // the image before the pokes
    FILE* pf = std::fopen(dump, "wb");
    if (!pf) die("cannot open the plan dump file");
    std::fwrite(plan, 1, info.plan_bytes, pf);
    std::fclose(pf);
  }
  for (int k = 0; k < n_pokes; ++k) {
    if (pokes[2 * k] < 0 || uint64_t(pokes[2 * k]) >= info.plan_bytes / 4) die("poke out of range");
    plan[pokes[2 * k]] = pokes[2 * k + 1];
  }
  int32_t* err = static_cast<int32_t*>(exact_alloc(8, 8));
  err[0] = err[1] = -7;
  const mla_status st = mla_decode_check(&s, &info, plan, bt, kvl, ql, err, nullptr);
  FILE* g = std::fopen(out_path, "wb");
  if (!g) die("cannot open output");
  const int32_t out[3] = {int32_t(st), err[0], err[1]};
  std::fwrite(out, 1, sizeof out, g);
  std::fclose(g);
  std::free(kvl);
  std::free(ql);
  std::free(bt);
  std::free(plan);
  std::free(err);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) die("usage: run_case <in.bin> <out.bin>");
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) die("cannot open input");
  int32_t hd[12];
  float scale;
  read_into(f, hd, sizeof hd);
  if (hd[0] == 0x4d4c4141) return run_append(f, hd, argv[2]);
  if (hd[0] == 0x4d4c4150) return run_plan(f, hd, argv[2]);
  if (hd[0] == 0x4d4c5046) return run_prefill(f, hd, argv[2]);
  if (hd[0] == 0x4d4c4143) return run_check(f, hd, argv[2]);
  read_into(f, &scale, sizeof scale);
  const bool tree = hd[0] == 0x4d4c4154;
  if (hd[0] != 0x4d4c4145 && !tree) die("bad magic");
  mla_shape s{};
  s.batch = hd[1];
  s.num_heads = hd[2];
  s.d_latent = 512;
  s.d_rope = 64;
  s.max_q_len = hd[3];
  s.page_size = hd[4];
  s.num_pages = hd[5];
  s.max_pages_per_seq = hd[6];
  s.kv_dtype = hd[7];
  s.causal = hd[8];
  const int nwg = hd[9];
  const bool has_ql = hd[10] != 0;
  const size_t rows = size_t(s.batch) * s.max_q_len * s.num_heads;
  const size_t kv_elems = size_t(s.num_pages) * s.page_size * 576;
  const size_t kv_bytes = kv_elems * (s.kv_dtype == MLA_KV_FP8_E4M3 ? 1 : 2);

  void* q = exact_alloc(rows * 576 * 2);
  void* kv = exact_alloc(kv_bytes);
  float* ksc = s.kv_dtype == MLA_KV_FP8_E4M3
                   ? static_cast<float*>(exact_alloc(size_t(s.num_pages) * s.page_size * 4, 4))
                   : nullptr;
  int32_t* bt = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * s.max_pages_per_seq * 4, 4));
  int32_t* kvl = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4));
  int32_t* ql = has_ql ? static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4)) : nullptr;
  read_into(f, q, rows * 576 * 2);
  read_into(f, kv, kv_bytes);
  if (ksc) read_into(f, ksc, size_t(s.num_pages) * s.page_size * 4);
  read_into(f, bt, size_t(s.batch) * s.max_pages_per_seq * 4);
  read_into(f, kvl, size_t(s.batch) * 4);
  if (ql) read_into(f, ql, size_t(s.batch) * 4);
  uint32_t* mask = nullptr;
  int32_t* full_kvl = nullptr;
  if (tree) {
    if (!ql) die("a tree case needs q_lens");
    mask = static_cast<uint32_t*>(exact_alloc(size_t(s.batch) * s.max_q_len * 4, 4));
    read_into(f, mask, size_t(s.batch) * s.max_q_len * 4);
    // the decode runs over the prefix: kv_len - q_len keys, non-causal
    full_kvl = kvl;
    kvl = static_cast<int32_t*>(exact_alloc(size_t(s.batch) * 4, 4));
    for (int b = 0; b < s.batch; ++b) kvl[b] = full_kvl[b] - ql[b];
    s.causal = 0;
  }
  std::fclose(f);

  const uint64_t bound = mla_plan_bytes_bound(&s, nwg);
  if (bound == 0) die("shape rejected by mla_plan_bytes_bound");
  std::vector<int32_t> host_plan(bound / 4 + 1);
  mla_plan_info info{};
  // EMU_PLAN_KV_LENS="l0,l1,...": plan for these lengths instead of the
  // device ones (a stale plan)
  std::vector<int32_t> plan_kvl(kvl, kvl + s.batch);
  if (const char* pk = std::getenv("EMU_PLAN_KV_LENS")) {
    const char* c = pk;
    for (int b = 0; b < s.batch; ++b) {
      char* end = nullptr;
      plan_kvl[b] = int32_t(std::strtol(c, &end, 10));
      if (end == c) die("EMU_PLAN_KV_LENS: too few lengths");
      c = *end == ',' ? end + 1 : end;
    }
  }
  mla_status st = hd[11] ? mla_decode_plan_fixed(&s, plan_kvl.data(), ql, nwg, host_plan.data(),
                                                  host_plan.size() * 4, &info)
                         : mla_decode_plan(&s, plan_kvl.data(), ql, nwg, host_plan.data(),
                                           host_plan.size() * 4, &info);
  if (st != MLA_OK) die("mla_decode_plan failed");
  // the "device" plan image: exactly plan_bytes long
  void* plan = exact_alloc(info.plan_bytes);
  std::memcpy(plan, host_plan.data(), info.plan_bytes);
  if (const char* dump = std::getenv("EMU_PLAN_OUT")) {   // the image, for the caller to inspect
    FILE* pf = std::fopen(dump, "wb");
    if (!pf) die("cannot open the plan dump file");
    std::fwrite(plan, 1, info.plan_bytes, pf);
    std::fclose(pf);
  }
  void* ws = info.workspace_bytes ? exact_alloc(info.workspace_bytes, 256) : nullptr;

  void* o = exact_alloc(rows * 512 * 2);
  float* lse = static_cast<float*>(exact_alloc(rows * 4, 4));
  // sentinels: rows the kernels must not write keep them
  std::memset(o, 0xC1, rows * 512 * 2);
  for (size_t i = 0; i < rows; ++i) lse[i] = 12345.0f;

  st = mla_decode_fwd(&s, &info, plan, q, kv, ksc, bt, kvl, ql, scale, o, lse, ws,
                      info.workspace_bytes, nullptr);
  if (st != MLA_OK) die("mla_decode_fwd failed");
  st = mla_combine(&s, &info, plan, ws, info.workspace_bytes, ql, o, lse, nullptr);
  if (st != MLA_OK) die("mla_combine failed");
  if (tree) {
    st = mla_tree_attend(&s, q, kv, ksc, bt, full_kvl, ql, mask, scale, o, lse, nullptr);
    if (st != MLA_OK) die("mla_tree_attend failed");
  }

  FILE* g = std::fopen(argv[2], "wb");
  if (!g) die("cannot open output");
  const int32_t meta[4] = {info.num_items, info.num_partials, info.num_combine, info.phases};
  std::fwrite(meta, 1, sizeof meta, g);
  std::fwrite(o, 1, rows * 512 * 2, g);
  std::fwrite(lse, 1, rows * 4, g);
  std::fclose(g);
  std::free(q);
  std::free(kv);
  std::free(ksc);
  std::free(bt);
  std::free(kvl);
  std::free(full_kvl);
  std::free(mask);
  std::free(ql);
  std::free(plan);
  std::free(ws);
  std::free(o);
  std::free(lse);
  return 0;
}
