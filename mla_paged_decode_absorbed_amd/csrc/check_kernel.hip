// Debug validation of the device-resident inputs the decode kernels take on
// trust: the plan image against the launch info and the device lengths, the
// lengths against the shape, and every block-table entry a planned key reads.
//
// The decode kernels index pages through the block table (the page / block
// table layout of the FlashAttention-3 in DeepSeek-R1 page, section 4.1) and
// key ranges through the split-K plan (same page, chapter 2) without checking
// either, since both live in device memory.  A stale plan (lengths changed
// but the image was not rebuilt) or a block-table entry outside the pool then
// makes them read outside the cache.  This kernel finds such inputs first: it
// only reads, and every read is bounded by sizes it has checked before.
//
// One workgroup of 256 threads strides over the header, the lengths, the
// block-table entries in use, the items and the combine entries, and counts
// the (key, query row) pairs the items cover against those the lengths ask
// for; the first violation (lowest check code, then lowest index) is written
// to err[0..1].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check.h"
#include "mla_decode.h"
#include "plan_layout.h"

namespace mla {
namespace {

constexpr int kCheckThreads = 256;
constexpr int kNone = 0x7FFFFFFF;

// code in the top 7 bits, index (saturated) in the low 24: the minimum over
// all reports is the lowest code, then the lowest index
__device__ __forceinline__ void report(int* first, int code, int64_t index) {
  const int64_t i = index < 0 ? 0 : (index > 0xFFFFFF ? 0xFFFFFF : index);
  atomicMin(first, (code << 24) | int(i));
}

__device__ __forceinline__ bool lengths_ok(const CheckArgs& a, int b, int* L_out, int* q_out) {
  const int L = a.kv_lens[b];
  const int q = a.q_lens ? a.q_lens[b] : a.max_q_len;
  *L_out = L;
  *q_out = q;
  if (L < 0 || int64_t(L) > int64_t(a.max_pages) * a.page_size) return false;
  if (q < 0 || q > a.max_q_len) return false;
  if (a.causal && q > 0 && L < q) return false;
  return true;
}

__global__ __launch_bounds__(kCheckThreads) void mla_check_kernel(const CheckArgs a) {
  __shared__ int first;
  // (key, row) pairs the items cover, and the pairs the lengths ask for
  __shared__ unsigned long long covered, wanted;
  const int tid = threadIdx.x;
  if (tid == 0) {
    first = kNone;
    covered = 0;
    wanted = 0;
  }
  __syncthreads();

  const int32_t* p = a.plan;
  const int64_t W = a.plan_words;
  // ---- header (every thread evaluates it: the bounds below depend on it)
  bool ok = W >= kHeaderWords;
  int G = 0, N = 0, C = 0, NP = 0, off_wg = 0, off_items = 0, off_comb = 0;
  if (ok) {
    G = p[kWNumWg];
    N = p[kWNumItems];
    C = p[kWNumCombine];
    NP = p[kWNumPartials];
    off_wg = p[kWOffWgStart];
    off_items = p[kWOffItems];
    off_comb = p[kWOffCombine];
    ok = p[kWMagic] == kPlanMagic && p[kWVersion] == kPlanVersion && G == a.num_wg &&
         p[kWPhases] == a.phases && p[kWTile] == kTileTokens &&
         p[kWRowsPerBlock] == kRowsPerBlock && N >= 0 && C >= 0 && NP >= 0 &&
         NP <= a.num_partials && off_wg >= kHeaderWords && off_items >= kHeaderWords &&
         off_comb >= kHeaderWords && int64_t(off_wg) + G + 1 <= W &&
         int64_t(off_items) + int64_t(N) * kItemWords <= W &&
         int64_t(off_comb) + int64_t(C) * kCombineWords <= W;
  }
  if (!ok) {
    if (tid == 0) report(&first, MLA_CHECK_PLAN, 0);
  } else {
    // workgroup item ranges: 0 = wg_start[0] <= ... <= wg_start[G] = N
    const int32_t* ws = p + off_wg;
    for (int g = tid; g <= G; g += kCheckThreads) {
      const int v = ws[g];
      const bool bad = v < 0 || v > N || (g == 0 && v != 0) || (g == G && v != N) ||
                       (g > 0 && ws[g - 1] > v);
      if (bad) report(&first, MLA_CHECK_PLAN, g);
    }
  }

  // ---- lengths
  unsigned long long want = 0;
  for (int b = tid; b < a.batch; b += kCheckThreads) {
    int L, q;
    if (!lengths_ok(a, b, &L, &q)) {
      report(&first, MLA_CHECK_LENGTHS, b);
    } else {
      want += (unsigned long long)L * (unsigned long long)q * (unsigned long long)a.num_heads;
    }
  }
  if (want) atomicAdd(&wanted, want);

  // ---- block-table entries of the pages each sequence uses
  const int64_t bt_entries = int64_t(a.batch) * a.max_pages;
  for (int64_t i = tid; i < bt_entries; i += kCheckThreads) {
    const int b = int(i / a.max_pages), j = int(i % a.max_pages);
    int L, q;
    if (!lengths_ok(a, b, &L, &q)) continue;   // reported above
    const int64_t used = (int64_t(L) + a.page_size - 1) / a.page_size;
    if (j >= used) continue;
    const int page = a.block_table[i];
    if (page < 0 || page >= a.num_pages) report(&first, MLA_CHECK_BLOCK_TABLE, b);
  }

  if (ok) {
    // ---- items: sequence, key range, rows and partial slot
    const int rows_per_item = kRowsPerBlock / a.phases;
    unsigned long long cover = 0;
    for (int n = tid; n < N; n += kCheckThreads) {
      const int32_t* it = p + off_items + int64_t(n) * kItemWords;
      const int b = it[0], row0 = it[1], k0 = it[2], k1 = it[3], slot = it[4], slot_row = it[5];
      bool good = b >= 0 && b < a.batch;
      int L = 0, q = 0;
      if (good) good = lengths_ok(a, b, &L, &q);
      if (good) {
        good = k0 >= 0 && k0 <= k1 && k1 <= L && k0 % kRoundTokens == 0 && row0 >= 0 &&
               row0 < q * a.num_heads && slot >= -1 && slot < NP && slot_row >= 0 &&
               slot_row % rows_per_item == 0 && slot_row + rows_per_item <= kRowsPerBlock;
      }
      if (!good) {
        report(&first, MLA_CHECK_ITEM, n);
      } else {
        const int rows = min(rows_per_item, q * a.num_heads - row0);
        cover += (unsigned long long)(k1 - k0) * (unsigned long long)rows;
      }
    }
    if (cover) atomicAdd(&covered, cover);
    // ---- combine entries: rows that exist, partial slots the plan has
    for (int e = tid; e < C; e += kCheckThreads) {
      const int32_t* c = p + off_comb + int64_t(e) * kCombineWords;
      const int b = c[0], row0 = c[1], s0 = c[2], ns = c[3];
      bool good = b >= 0 && b < a.batch;
      int L = 0, q = 0;
      if (good) good = lengths_ok(a, b, &L, &q);
      if (good)
        good = row0 >= 0 && row0 < q * a.num_heads && s0 >= 0 && ns >= 1 &&
               int64_t(s0) + ns <= NP;
      if (!good) report(&first, MLA_CHECK_COMBINE, e);
    }
  }

  __syncthreads();
  // every key of every valid query row is covered exactly once by the items
  // of a plan built for these lengths (the pieces of a unit partition its
  // keys); a plan for other lengths that still passes the item checks
  // covers a different count.  Reported as item N (one past the last).
  if (tid == 0) {
    if (ok && covered != wanted) report(&first, MLA_CHECK_ITEM, N);
    const int f = first;
    a.err[0] = f == kNone ? 0 : (f >> 24);
    a.err[1] = f == kNone ? 0 : (f & 0xFFFFFF);
  }
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_check_kernel, dim3(1), dim3(kCheckThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
