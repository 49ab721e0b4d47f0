// Weight-absorbed MLA decode over a paged latent cache, for gfx950 (MI355X).
//
// What is computed (per query row = (sequence b, token t, head h)):
//   s_j = scale * <q, c_j> over the visible cached latent rows c_j (576 wide),
//   O = softmax(s) . latent (the first 512 columns of the same rows), LSE.
// Sources: decode-only weight-absorbed MLA (KsanaLLM 0.6.0 page, prefill/decode
// disaggregation section); several draft tokens verified in one decode pass
// (PaddlePaddle 3.0 inference page, speculative decoding section); LSE output
// and split-K (FlashAttention-3 in DeepSeek-R1 page, chapter 2); per-token fp8
// cache scales (same page, section 3.1).
//
// Mapping onto CDNA4:
//   * One 256-thread workgroup (4 wave64s, one per SIMD) per CU, persistent
//     over the work items the planner gave it.  A work item is 128 query rows
//     of one sequence and a key range; wave w owns rows 32w..32w+31.
//   * The 128 rows share one key stream, so every key tile is fetched from HBM
//     once per item with global_load_lds_dwordx4 (HBM -> LDS, no VGPR
//     staging) into a 4-stage ring; each wave reads the whole tile from LDS.
//     The copies are issued from inline assembly so that the compiler's
//     conservative LDS-DMA waits do not drain the ring before every LDS read;
//     the ring is ordered by explicit vmcnt waits and workgroup barriers.
//   * QK^T runs as S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 with Q resident
//     in VGPRs (32 rows x 576 = 144 VGPRs per wave).  In that layout every lane
//     owns one query row, so the online softmax needs one cross-lane max.
//   * PV runs as O^T = V^T . P^T: the S^T accumulator already is the B operand
//     of the next MFMA, so P never leaves registers.  V^T comes from the same
//     LDS tile through the transposing ds_read_b64_tr_b16 (bf16) or
//     ds_read_b64_tr_b8 (fp8).
//   * The O accumulator is 32 rows x 512 fp32 per wave (256 AGPRs) and is only
//     rescaled when a row's running max grows by more than 2^8 (softmax does
//     not depend on the reference max; this keeps p <= 256).
//   * fp8 e4m3 keys are widened exactly to bf16 in registers; the per-token
//     scale multiplies the score column (QK) and the probability (PV), so Q
//     keeps bf16 precision.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "plan_layout.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T) T __attribute__((address_space(3)))*

constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kStageBytes = 36864;            // 2304 16-byte chunks per key tile
constexpr int kLoadsPerWave = 9;              // dwordx4 copies per wave per tile
constexpr int kScaleStageBytes = 4 * 64 * 4;  // fp8: one 64-scale copy per wave
constexpr float kRescaleThreshold = 8.0f;     // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

// Tile geometry.  Each wave copies RPW consecutive tile rows (576 chunks of
// 16 bytes = 9 KiB, contiguous in LDS), so all waves issue the same number of
// copies and one vmcnt value serves every wave.
template <int KVD> struct Tile;
template <> struct Tile<0> {   // bf16 rows: 32 tokens x 72 chunks
  static constexpr int T = 32, ROW_BYTES = 1152, ROW_CHUNKS = 72, RPW = 8;
  static constexpr int LOADS = kLoadsPerWave;
};
template <> struct Tile<1> {   // e4m3 rows: 64 tokens x 36 chunks, plus scales
  static constexpr int T = 64, ROW_BYTES = 576, ROW_CHUNKS = 36, RPW = 16;
  static constexpr int LOADS = kLoadsPerWave + 1;
};

// LDS swizzle of the 16-byte chunks of one key row so that the 32 rows read by
// one MFMA operand load spread over the banks.  XOR keeps a chunk inside its
// aligned group (8 chunks for bf16 rows, 4 for e4m3 rows); it is an involution.
__device__ __forceinline__ int swz_bf16(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz_fp8(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

// HBM -> LDS copy of 16 bytes per lane: LDS destination = lds_base + 16 * lane,
// source = sbase + voff.  M0 is saved and restored around the copy.
__device__ __forceinline__ void lds_dma_x4(uint32_t lds_base, int voff, const void* sbase) {
  int tmp;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(tmp)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}
__device__ __forceinline__ void lds_dma_x1(uint32_t lds_base, int voff, const void* sbase) {
  int tmp;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3 offset:0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(tmp)
      : "s"(lds_base), "v"(voff), "s"(sbase)
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight,
// then meet the other waves.  The "memory" clobber keeps LDS reads after it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N < 64, "vmcnt is 6 bits");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 20) asm volatile("s_waitcnt vmcnt(20)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0, "add the literal above");
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Widen 8 e4m3 bytes to 8 bf16 values (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(i32x2 v) {
  bf16x8 r;
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, true);
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)b.x; r[3] = (__bf16)b.y;
  r[4] = (__bf16)c.x; r[5] = (__bf16)c.y; r[6] = (__bf16)d.x; r[7] = (__bf16)d.y;
  return r;
}

// Multiply one accumulator tile held in AGPRs by a per-lane factor without
// moving the whole tile into VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = acc[r];
    float tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(tmp)
        : "v"(alpha));
    acc[r] = x;
  }
}

// Issue the HBM -> LDS copy of the key tile that starts at token j0 of
// sequence b (the tile lies inside one page).  Rows at or past the sequence
// length are redirected to row 0 of the tile (always a valid token): their
// probabilities are zero, and a finite value keeps 0 * v = 0 inside the MFMA
// whatever the page tail holds.
template <int KVD>
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ kv,
                                           const float* __restrict__ kv_scale, int page,
                                           int page_shift, int j0, int L, uint32_t stage_lds,
                                           uint32_t scale_lds, int wave, int lane_o) {
  using TL = Tile<KVD>;
  const int row0 = (page << page_shift) + (j0 & ((1 << page_shift) - 1));
  const uint8_t* base = kv + (int64_t)row0 * TL::ROW_BYTES;
  const int nvalid = min(TL::T, L - j0);
  const uint32_t wave_lds = stage_lds + wave * (kLoadsPerWave * 1024);
#pragma unroll
  for (int ins = 0; ins < kLoadsPerWave; ++ins) {
    const int q = ins * 64 + lane_o;                // chunk inside this wave's 9 KiB
    const int lr = q / TL::ROW_CHUNKS;
    const int pc = q - lr * TL::ROW_CHUNKS;
    const int r = wave * TL::RPW + lr;              // tile row
    const int c = KVD == 0 ? swz_bf16(lr, pc) : swz_fp8(lr, pc);
    const int voff = (r < nvalid ? r * TL::ROW_BYTES : 0) + c * 16;
    lds_dma_x4(wave_lds + ins * 1024, voff, base);
  }
  if constexpr (KVD == 1) {
    // 64 per-token scales, one private copy per wave
    lds_dma_x1(scale_lds + wave * 256, (lane_o < nvalid ? lane_o : 0) * 4, kv_scale + row0);
  }
}

template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(
    const int32_t* __restrict__ plan, const uint8_t* __restrict__ q,
    const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, float scale_log2, int H,
    int max_q_len, int page_shift, int max_pages, int causal, int num_wg) {
  using TL = Tile<KVD>;
  __shared__ __attribute__((aligned(1024)))
  char smem[kStages * kStageBytes + (KVD == 1 ? kStages * kScaleStageBytes : 0)];
  const uint32_t smem_base = (uint32_t)(uintptr_t)(LDS_PTR(char))smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hl = lane >> 5;            // which half of the wave
  const int lrow = lane & 31;          // query row in the wave / key row in an MFMA tile

  // Consecutive logical workgroups land on one XCD (dispatch is round-robin
  // over the 8 XCDs), so the pieces of one sequence share an L2.
  const int bid = blockIdx.x;
  const int g = (num_wg % 8 == 0) ? (bid & 7) * (num_wg >> 3) + (bid >> 3) : bid;

  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  const int it_begin = wg_start[g], it_end = wg_start[g + 1];

  // Per-lane LDS read offsets (stage-relative), constant over the run.
  int kaddr[4];   // K operand: key row lrow, dims 16c + 8hl .. +7 of MFMA step c
  int vaddr[2];   // V^T operand, see the transposing-read contract below
  if constexpr (KVD == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) kaddr[j] = lrow * 1152 + (((2 * j + hl) ^ (lrow & 7)) * 16);
    // ds_read_b64_tr_b16 on a 16-lane group: lane i gives the address of row
    // i/4, elements 4(i%4)..+3 of a 4 x 16 block; it returns column i.
    const int G16 = lane >> 4, i = lane & 15;
    const int rowl = 4 * (G16 >> 1) + (i >> 2);      // key row inside an 8-row band
    const int u = 2 * (G16 & 1) + ((i & 3) >> 1);     // chunk inside a 32-column block
#pragma unroll
    for (int e = 0; e < 2; ++e)
      vaddr[e] = rowl * 1152 + (((4 * e + u) ^ (rowl & 7)) * 16) + 8 * (i & 1);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) kaddr[j] = lrow * 576 + ((j ^ ((lrow >> 1) & 3)) * 16) + 8 * hl;
    // ds_read_b64_tr_b8 on a 16-lane group: lane i gives the address of row
    // i/2, bytes 8(i%2)..+7 of an 8 x 16 byte block; it returns column i.
    const int G16 = lane >> 4, i = lane & 15;
    const int s = i >> 1;                                      // k slot = block row
    const int rowl = 8 * (s >> 2) + 4 * (G16 >> 1) + (s & 3);  // key row in a 16-row band
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int chunk = 2 * e + (G16 & 1);
      vaddr[e] = rowl * 576 + ((chunk ^ ((rowl >> 1) & 3)) * 16) + 8 * (i & 1);
    }
  }

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* item = items + it * kItemWords;
    const int b = item[0], row_base = item[1], k0 = item[2], k1 = item[3], slot = item[4];
    const int L = kv_lens[b];
    const int qb = q_lens ? q_lens[b] : max_q_len;
    const int R = qb * H;

    const int my_row = row_base + wave * 32 + lrow;    // row inside the sequence
    const bool row_valid = my_row < R;
    const int t = row_valid ? my_row / H : 0;
    const int h = row_valid ? my_row - t * H : 0;
    // keys j < lim are visible to this row inside this item
    const int vis = causal ? L - qb + t + 1 : L;
    const int lim = min(vis, k1);

    const int ntiles = k1 > k0 ? (k1 - k0 + TL::T - 1) / TL::T : 0;
    const int32_t* bt_row = block_table + (int64_t)b * max_pages;

    // ---- prologue: tiles 0 .. kStages-2, then Q.  Q is waited for here, so
    // no wait on it is left inside the key loop (where it would also drain
    // the copies in flight).
    int lane_o;
    asm volatile("" : "=v"(lane_o) : "0"(lane));
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      if (s < ntiles) {
        const int j0 = k0 + s * TL::T;
        issue_tile<KVD>(kv, kv_scale, bt_row[j0 >> page_shift], page_shift, j0, L,
                        smem_base + s * kStageBytes,
                        smem_base + kStages * kStageBytes + s * kScaleStageBytes, wave, lane_o);
      }
    }
    bf16x8 qf[36];
    {
      // invalid rows read row (b, 0, 0), which exists; their results are dropped
      const uint8_t* qp =
          q + ((int64_t)((b * max_q_len + t) * H + h)) * (kDQK * 2) + hl * 16;
#pragma unroll
      for (int c = 0; c < 36; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 32);
#pragma unroll
      for (int c = 0; c < 36; ++c) asm volatile("" ::"v"(qf[c]));
    }

    f32x16 acc[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    for (int i = 0; i < ntiles; ++i) {
      // tiles issued after tile i so far: min(ntiles, i + kStages - 1) - i - 1
      const int ahead = min(ntiles, i + kStages - 1) - i - 1;
      if (ahead >= 2) wait_and_barrier<2 * TL::LOADS>();
      else if (ahead == 1) wait_and_barrier<TL::LOADS>();
      else wait_and_barrier<0>();

      if (i + kStages - 1 < ntiles) {
        const int s = (i + kStages - 1) % kStages;
        const int j0 = k0 + (i + kStages - 1) * TL::T;
        asm volatile("" : "=v"(lane_o) : "0"(lane));
        issue_tile<KVD>(kv, kv_scale, bt_row[j0 >> page_shift], page_shift, j0, L,
                        smem_base + s * kStageBytes,
                        smem_base + kStages * kStageBytes + s * kScaleStageBytes, wave, lane_o);
      }

      const int stage = i % kStages;
      const char* st = smem + stage * kStageBytes;
      const int j0 = k0 + i * TL::T;
      const float* scl = nullptr;
      if constexpr (KVD == 1)
        scl = reinterpret_cast<const float*>(smem + kStages * kStageBytes +
                                             stage * kScaleStageBytes + wave * 256);

#pragma unroll
      for (int half = 0; half < TL::T / 32; ++half) {
        // ---- S^T[32 keys x 32 rows] = K . Q^T, K fragments two steps ahead
        f32x16 S = f32x16{};
        if constexpr (KVD == 0) {
          bf16x8 kb[3];
          auto kload = [&](int c) {
            return *(const LDS_PTR(bf16x8))(st + kaddr[c & 3] + 128 * (c >> 2));
          };
          kb[0] = kload(0);
          kb[1] = kload(1);
#pragma unroll
          for (int c = 0; c < 36; ++c) {
            if (c + 2 < 36) kb[(c + 2) % 3] = kload(c + 2);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c % 3], qf[c], S, 0, 0, 0);
          }
        } else {
          const char* sth = st + half * 32 * 576;
          i32x2 kb[3];
          auto kload = [&](int c) {
            return *(const LDS_PTR(i32x2))(sth + kaddr[c & 3] + 64 * (c >> 2));
          };
          kb[0] = kload(0);
          kb[1] = kload(1);
#pragma unroll
          for (int c = 0; c < 36; ++c) {
            if (c + 2 < 36) kb[(c + 2) % 3] = kload(c + 2);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(kb[c % 3]), qf[c], S, 0,
                                                        0, 0);
          }
        }

        // ---- online softmax: lane owns row lrow, keys 8(r/4) + 4hl + r%4
        const int jt = j0 + half * 32;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
          float v = S[r] * scale_log2;
          if constexpr (KVD == 1) v *= scl[half * 32 + key];
          v = (jt + key < lim) ? v : -INFINITY;
          S[r] = v;
          mx = fmaxf(mx, v);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));   // lanes l and l^32 hold the same row
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run + kRescaleThreshold)) {
          const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) scale_acc(acc[cb], alpha);
          l_run *= alpha;
          m_run = m_new;
        }
        const bool dead = (m_run == -INFINITY);
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = dead ? 0.f : __builtin_amdgcn_exp2f(S[r] - m_run);
          l_run += p;
          if constexpr (KVD == 1) p *= scl[half * 32 + 8 * (r >> 2) + 4 * hl + (r & 3)];
          pb[r >> 3][r & 7] = (__bf16)p;
        }

        // ---- O^T[512 x 32 rows] += V^T . P^T: two 16-key steps x 16 column blocks
        if constexpr (KVD == 0) {
          auto vload = [&](int n) {   // n = step * 16 + cb
            const int step = n >> 4, cb = n & 15;
            const char* vp = st + vaddr[cb & 1] + 128 * (cb >> 1) + step * 16 * 1152;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))vp);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(vp + 8 * 1152));
            return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          };
          bf16x8 vb[3];
          vb[0] = vload(0);
          vb[1] = vload(1);
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            if (n + 2 < 32) vb[(n + 2) % 3] = vload(n + 2);
            acc[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[n % 3], pb[n >> 4],
                                                                  acc[n & 15], 0, 0, 0);
          }
        } else {
          auto vload = [&](int n) {
            const int step = n >> 4, cb = n & 15;
            const char* vp = st + half * 32 * 576 + vaddr[cb & 1] + 64 * (cb >> 1) +
                             step * 16 * 576;
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))vp);
          };
          i32x2 vb[3];
          vb[0] = vload(0);
          vb[1] = vload(1);
#pragma unroll
          for (int n = 0; n < 32; ++n) {
            if (n + 2 < 32) vb[(n + 2) % 3] = vload(n + 2);
            acc[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                e4m3x8_to_bf16(vb[n % 3]), pb[n >> 4], acc[n & 15], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue: lane owns row lrow, columns 32cb + 8(r/4) + 4hl + r%4
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_v = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
    if (row_valid) {
      if (slot < 0) {
        uint8_t* op = o + ((int64_t)((b * max_q_len + t) * H + h)) * (kDLatent * 2);
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * inv);
            const int col = 32 * cb + 8 * q4 + 4 * hl;
            *reinterpret_cast<bf16x4*>(op + col * 2) = v;
          }
        }
        if (lse && hl == 0) lse[(b * max_q_len + t) * H + h] = lse_v;
      } else {
        const int rb = wave * 32 + lrow;
        float* pp = part_o + ((int64_t)slot * kRowsPerBlock + rb) * kDLatent;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * inv;
            const int col = 32 * cb + 8 * q4 + 4 * hl;
            *reinterpret_cast<f32x4*>(pp + col) = v;
          }
        }
        if (hl == 0) part_lse[(int64_t)slot * kRowsPerBlock + rb] = lse_v;
      }
    }
    // every wave leaves the ring before the next item's prologue refills it
    barrier();
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  const dim3 grid(a.num_wg), block(kThreads);
  auto k = kv_dtype == 0 ? mla_decode_kernel<0> : mla_decode_kernel<1>;
  hipLaunchKernelGGL(k, grid, block, 0, stream, a.plan, a.q, a.kv, a.kv_scale, a.block_table,
                     a.kv_lens, a.q_lens, a.o, a.lse, a.part_o, a.part_lse, a.scale_log2,
                     a.num_heads, a.max_q_len, a.page_shift, a.max_pages, a.causal, a.num_wg);
  return hipGetLastError();
}

}  // namespace mla
