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
// Two kernels share the copy ring, waits, barriers, restart and epilogue
// described below; they differ in the per-tile compute.
//   * mla_decode_kernel_pairs (bf16 cache, one workgroup per 128-row block:
//     the default plan) steps keys in pairs of 16-key ring stages.
//     QK^T: S^T[32 keys x 32 rows] = K . Q^T on v_mfma_f32_32x32x16_bf16; a
//     lane holds 16 keys of one score row and its partner lane l^32 the other
//     16, so the row max is one v_permlane32_swap.  The PV contraction takes
//     the keys in the order the score layout holds them (lane half hl: keys
//     0-3, 8-11 / 4-7, 12-15 of each stage), so the probabilities are the B
//     operand with no permute; V^T is read by ds_read_b64_tr_b16 in the same
//     key order.  Per 32 keys the compiler moves 48 accumulator registers
//     between AGPRs and VGPRs (208 for two tiles of the 16-key kernel), and
//     issues about half the VALU work.
//   * mla_decode_kernel (e4m3 cache, and plans whose phases share a row
//     group) steps one 16-key tile at a time, as described next.
//
// Mapping onto CDNA4:
//   * One 256-thread workgroup (4 wave64s, one per SIMD) per CU, persistent
//     over the work items the planner gave it.  Every wave owns 32 query rows
//     (Q resident in VGPRs, the 32 x 512 fp32 output accumulator in AGPRs).
//   * A work item is 128/PH query rows of one sequence and a key range.  PH
//     (phases) waves share each row group and split its key tiles: tile i goes
//     to phase i % PH.  PH = 1 lets four row groups share every tile; PH = 4
//     gives all four waves the same 32 rows, so four CUs on one XCD can each
//     take 32 heads of a sequence and read its cache once from HBM (the other
//     three reads hit that XCD's L2).  Phases merge through LDS at item end.
//   * Key tiles of 16 tokens stream HBM -> LDS with global_load_lds_dwordx4
//     (no VGPR staging) through an 8-stage ring (16 for e4m3).  Tiles are
//     issued in rounds of four (one per wave); the copies are inline assembly
//     ordered by explicit vmcnt waits, so the compiler's conservative waits do
//     not drain the ring before every LDS read.
//   * QK^T: S^T[16 keys x 16 rows] = K . Q^T on v_mfma_f32_16x16x32_bf16, two
//     row blocks per key fragment.  Each score row is spread over 4 lanes
//     (4 keys each); its max takes two lane-swap steps.
//   * PV: O^T[512 x 32 rows] += V^T . P^T on v_mfma_f32_32x32x16_bf16.  Two
//     v_permlane16_swap turn the probabilities of the two 16-row score blocks
//     into the 32-row B operand with keys in natural order; V^T comes from the
//     same LDS tile through ds_read_b64_tr_b16 (bf16) or ds_read_b64_tr_b8
//     (e4m3, widened exactly in registers).
//   * No rescaling of the accumulator: each row's reference max is fixed by
//     its first visible tile (softmax does not depend on it, and bf16/fp32
//     keep full relative precision up to p = 2^32).  A later score above the
//     reference by more than 32 (log2 units) restarts the item with the
//     raised reference; the accumulator is only ever written by MFMAs, so it
//     stays in AGPRs.
//   * e4m3 keys are widened exactly to bf16 in registers; the per-token scale
//     multiplies the score (QK) and the probability (PV), so Q keeps bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_asm.h"
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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTileTok = 16;                  // keys per tile
constexpr int kRoundTiles = 4;                // tiles per round (one issued per wave)
constexpr int kRoundTok = kTileTok * kRoundTiles;
constexpr int kRingBytes = 147456;
constexpr int kScaleSlotBytes = 256;          // 64 fp32 scales of one round
constexpr float kRestartMargin = 32.0f;       // log2 units above the reference max
constexpr float kLn2 = 0.69314718055994530942f;

template <int KVD> struct Cfg;
template <> struct Cfg<0> {      // bf16 rows
  static constexpr int ROW = 1152, CHUNKS = 72, TILE = 18432, STAGES = 8, DMA = 18;
};
template <> struct Cfg<1> {      // e4m3 rows (+ one fp32 scale per token)
  static constexpr int ROW = 576, CHUNKS = 36, TILE = 9216, STAGES = 16, DMA = 9;
};
template <int KVD> constexpr int kRounds = Cfg<KVD>::STAGES / kRoundTiles;   // rounds in the ring
template <int KVD> constexpr int kOps = Cfg<KVD>::DMA + (KVD == 1 ? 1 : 0);   // vm ops per wave per round

constexpr int kScaleOff = kRingBytes;                                 // e4m3 scales
constexpr int kMlOff = kRingBytes + 4 * 4 * kScaleSlotBytes;          // merge (m, l)
constexpr int kFlagOff = kMlOff + 4 * 32 * 2 * 4;                    // restart flag
constexpr int kSmemBytes = kFlagOff + 16;

// LDS layout of one key tile (16 cached rows).  Each 1 KB block of the tile
// is written by one copy instruction (64 lanes x 16 bytes, in lane order), so
// the layout is the lane order of the copies:
//   bf16: block 2*cg + rh holds rows 8rh..8rh+7 x 16-byte chunks 8cg..8cg+7
//         (128 contiguous bytes of each row); chunk (r8, c8) sits in slot
//         16*(c8>>1) + 8*((c8&1)^rh) + (r8 ^ 4*((c8>>1)&1)).
//   e4m3: block ins holds rows 0..15 x chunks 4ins..4ins+3; chunk (r, cc) sits
//         in slot 16*cc + (r ^ 8*(cc&1)).
// Both place the 16 rows of one chunk (a K-fragment read) and the 4 or 8 rows
// x 2-4 adjacent chunks of a transposing V read on distinct LDS banks, and
// make every per-lane LDS address a base plus a compile-time offset.
__device__ __forceinline__ int slot_bf16(int r8, int c8, int rh) {
  return 16 * (c8 >> 1) + 8 * ((c8 & 1) ^ rh) + (r8 ^ (4 * ((c8 >> 1) & 1)));
}
__device__ __forceinline__ int slot_fp8(int r, int cc) { return 16 * cc + (r ^ (8 * (cc & 1))); }

// A wave-uniform pointer, kept in SGPRs (the copies take a scalar base).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

// Wait for round j of this wave given `ahead` later rounds already issued
// (bf16 rings hold 2 rounds, so nothing is ever issued beyond round j when
// it is waited for; e4m3 rings hold 4 rounds of 10 operations).
template <int KVD>
__device__ __forceinline__ void vm_wait_rounds(int ahead) {
  if constexpr (KVD == 0) {
    MLA_VM_WAIT(0);
  } else {
    static_assert(kOps<1> == 10 && kRounds<1> == 4, "wait literals below");
    if (ahead >= 2) MLA_VM_WAIT(20);
    else if (ahead == 1) MLA_VM_WAIT(10);
    else MLA_VM_WAIT(0);
  }
}

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

// max / sum over the 4 lanes {l, l^16, l^32, l^48} that share a score row.
__device__ __forceinline__ float quad_max(float x) {
  const unsigned u = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const unsigned v = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  const unsigned u = __float_as_uint(x);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const unsigned v = __float_as_uint(x);
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

template <int KVD>
struct DmaCtx {
  const uint8_t* kv;
  const float* kv_scale;
  const int32_t* bt_row;
  uint32_t ring;       // LDS address of the ring
  uint32_t scales;     // LDS address of this wave's scale slots
  int page_shift, k0, L, ntiles, wave, lane;
};

// Issue this wave's share of round j: tile 4j + wave into its ring stage (a
// harmless dummy copy when that tile lies past the item), and for e4m3 the 64
// scales of the round into this wave's private slot.  Every wave issues
// exactly kOps operations per round, so vmcnt arithmetic is uniform.
template <int KVD>
__device__ __forceinline__ void issue_round(const DmaCtx<KVD>& c, int j) {
  using C = Cfg<KVD>;
  const int tile = kRoundTiles * j + c.wave;
  const int stage = tile % C::STAGES;
  const int kr = c.k0 + kRoundTok * j;          // first key of the round (< L)
  const bool real = tile < c.ntiles;
  const int kt = real ? c.k0 + kTileTok * tile : kr;
  const int pmask = (1 << c.page_shift) - 1;
  const int row0 = (c.bt_row[kt >> c.page_shift] << c.page_shift) + (kt & pmask);
  const uint8_t* base = uniform_ptr(c.kv + (int64_t)row0 * C::ROW);
  const int nvalid = real ? min(kTileTok, c.L - kt) : 0;
  const uint32_t lds = c.ring + stage * C::TILE;
  // an opaque copy of the lane id keeps these offsets from being hoisted out
  // of the key loop (they would pin VGPRs for its whole duration)
  const int lane = opaque(c.lane);
  if constexpr (KVD == 0) {
    // copy 2*cg + rh: rows 8rh.., chunks 8cg.. (row bytes 128cg .. 128cg+127)
    const int c8a = 2 * (lane >> 4), lo = (lane >> 3) & 1;
    const int r8 = (lane & 7) ^ (4 * ((lane >> 4) & 1));
    int vo[2];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int row = 8 * rh + r8;
      const int c8 = c8a + (lo ^ rh);
      vo[rh] = (row < nvalid ? row * C::ROW : 0) + c8 * 16;
    }
#pragma unroll
    for (int ins = 0; ins < C::DMA; ++ins)
      lds_dma_x4(lds + ins * 1024, vo[ins & 1], base + 128 * (ins >> 1));
  } else {
    // copy ins: rows 0..15, chunks 4ins.. (row bytes 64ins .. 64ins+63)
    const int cc = lane >> 4;
    const int r = (lane & 15) ^ (8 * (cc & 1));
    const int vo = (r < nvalid ? r * C::ROW : 0) + cc * 16;
#pragma unroll
    for (int ins = 0; ins < C::DMA; ++ins) lds_dma_x4(lds + ins * 1024, vo, base + 64 * ins);
    const int rrow0 = (c.bt_row[kr >> c.page_shift] << c.page_shift) + (kr & pmask);
    const int tok = lane < c.L - kr ? lane : 0;
    lds_dma_x1(c.scales + (j % kRounds<KVD>) * kScaleSlotBytes, tok * 4,
               uniform_ptr(c.kv_scale + rrow0));
  }
}

template <int KVD, int PH>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  // Every pointer is a separate restrict-qualified argument: the stores to the
  // outputs then provably leave the plan, lengths and block table untouched,
  // so their uniform loads become scalar loads (a vector load would need a
  // vmcnt wait that also drains the copies in flight).
  using C = Cfg<KVD>;
  constexpr int RG = 4 / PH;          // row groups of 32 per item
  constexpr int NR = kRounds<KVD>;
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const uint32_t smem_base = lds_address(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int rg = wave % RG;           // row group of this wave
  const int ph = wave / RG;           // phase of this wave
  const int l16 = lane & 15, g4 = lane >> 4;

  // Consecutive logical workgroups land on one XCD (dispatch is round-robin
  // over the 8 XCDs), so the CUs that share a sequence share an L2.
  const int bid = blockIdx.x;
  const int nwg = a.num_wg;
  const int g = (nwg % 8 == 0) ? (bid & 7) * (nwg >> 3) + (bid >> 3) : bid;

  if (tid == 0) *(volatile LDS_PTR(int))(smem + kFlagOff) = 0;
  barrier();

  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  const int it_begin = wg_start[g], it_end = wg_start[g + 1];
  const int H = a.num_heads;

  // ---- per-lane LDS read offsets (stage relative), constant over the run.
  // K fragment of QK step c (16 keys x 32 dims): key row l16, dims 32c + 8g4.
  // V^T fragment of PV column block cb: column 32cb + lane%32, keys 8(lane/32)
  // + 0..3 (first read) and + 4..7 (second read).  Per-step offsets are
  // compile-time: kstep(c) and vstep(cb) below.
  int kbase, vbase1, vbase2;
  if constexpr (KVD == 0) {
    const int h = g4 >> 1, rh = l16 >> 3, r8 = l16 & 7;
    kbase = rh * 1024 + (16 * h + 8 * ((g4 & 1) ^ rh) + (r8 ^ (4 * h))) * 16;
    const int eta = lane >> 5, j = l16, G = g4 & 1, u1 = (j >> 1) & 1;
    const int ra = j >> 2, rb = ra + 4;
    vbase1 = eta * 1024 + (16 * G + 8 * (u1 ^ eta) + (ra ^ (4 * G))) * 16 + 8 * (j & 1);
    vbase2 = eta * 1024 + (16 * G + 8 * (u1 ^ eta) + (rb ^ (4 * G))) * 16 + 8 * (j & 1);
  } else {
    const int h = g4 >> 1;
    kbase = (16 * h + (l16 ^ (8 * h))) * 16 + 8 * (g4 & 1);
    const int eta = lane >> 5, j = l16, G = g4 & 1;
    const int r1 = 8 * eta + (j >> 1);
    vbase1 = (16 * G + (r1 ^ (8 * G))) * 16 + 8 * (j & 1);
    vbase2 = 0;
  }

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* item = items + it * kItemWords;
    const int b = item[0], row_base = item[1], k0 = item[2], k1 = item[3], slot = item[4];
    const int slot_row = item[5];
    const int L = kv_lens[b];
    const int qb = q_lens ? q_lens[b] : a.max_q_len;
    const int R = qb * H;
    const int ntiles = k1 > k0 ? (k1 - k0 + kTileTok - 1) / kTileTok : 0;
    const int nrounds = (ntiles + kRoundTiles - 1) / kRoundTiles;

    // rows of this wave: block A = rows 0..15, block B = rows 16..31
    const int rowA = row_base + 32 * rg + l16, rowB = rowA + 16;
    const bool vA = rowA < R, vB = rowB < R;
    const int tA = vA ? rowA / H : 0, hA = vA ? rowA - tA * H : 0;
    const int tB = vB ? rowB / H : 0, hB = vB ? rowB - tB * H : 0;
    const int visA = a.causal ? L - qb + tA + 1 : L, visB = a.causal ? L - qb + tB + 1 : L;
    const int limA = vA ? min(visA, k1) : k0, limB = vB ? min(visB, k1) : k0;
    // keys below lim_all are visible to every row of the wave
    int lim_all = min(limA, limB);
    lim_all = min(lim_all, __shfl_xor(lim_all, 1));
    lim_all = min(lim_all, __shfl_xor(lim_all, 2));
    lim_all = min(lim_all, __shfl_xor(lim_all, 4));
    lim_all = min(lim_all, __shfl_xor(lim_all, 8));
    lim_all = __builtin_amdgcn_readfirstlane(lim_all);

    // ---- Q (issued first, so waiting for round 0 also covers it)
    bf16x8 qA[18], qB[18];
    {
      const uint8_t* pa = qg + ((int64_t)((b * a.max_q_len + tA) * H + hA)) * (kDQK * 2) + g4 * 16;
      const uint8_t* pb = qg + ((int64_t)((b * a.max_q_len + tB) * H + hB)) * (kDQK * 2) + g4 * 16;
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        qA[c] = *reinterpret_cast<const bf16x8*>(pa + c * 64);
        qB[c] = *reinterpret_cast<const bf16x8*>(pb + c * 64);
      }
#ifdef MLA_DECODE_Q_RESIDENT
      // Q resident before any copy is issued: otherwise the compiler, which
      // does not see the copies, waits for the Q loads inside the key loop
      // with vmcnt literals that at run time also count the rounds issued
      // ahead (decode_kernel_qres.hip)
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        require_vgpr(qA[c]);
        require_vgpr(qB[c]);
      }
#endif
    }

    DmaCtx<KVD> dc;
    dc.kv = kvg;
    dc.kv_scale = kv_scale;
    dc.bt_row = block_table + (int64_t)b * a.max_pages;
    dc.ring = smem_base;
    dc.scales = smem_base + kScaleOff + wave * (kRounds<1> * kScaleSlotBytes);
    dc.page_shift = a.page_shift;
    dc.k0 = k0;
    dc.L = L;
    dc.ntiles = ntiles;
    dc.wave = wave;
    dc.lane = lane;
    volatile LDS_PTR(int) restart_flag = (volatile LDS_PTR(int))(smem + kFlagOff);

    f32x16 acc[16];
    float mA = -INFINITY, mB = -INFINITY, lA = 0.f, lB = 0.f;
    for (;;) {   // runs once unless a score overshoots the reference max
#pragma unroll
      for (int j = 0; j < NR - 1; ++j)
        if (j < nrounds) issue_round<KVD>(dc, j);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
      lA = 0.f;
      lB = 0.f;
      bool overshoot = false;   // wave-uniform

      for (int j = 0; j < nrounds; ++j) {
        const int ahead = min(nrounds, j + NR - 1) - j - 1;
        vm_wait_rounds<KVD>(ahead);
        if constexpr (PH != 4) {
          barrier();   // tiles of round j come from all waves
          if (*restart_flag) {
            overshoot = true;
            break;
          }
        } else {
          if (overshoot) break;
        }
        if (j + NR - 1 < nrounds) issue_round<KVD>(dc, j + NR - 1);
        if (overshoot) continue;   // keep the round protocol until all waves see the flag

#pragma unroll
        for (int tt = 0; tt < kRoundTiles / PH; ++tt) {
          const int t_in_round = ph + PH * tt;
          const int tile = kRoundTiles * j + t_in_round;
          if (tile >= ntiles) break;
          const int kt = k0 + kTileTok * tile;
          const char* st = smem + (tile % C::STAGES) * C::TILE;

          // ---- S^T = K . Q^T, two 16-row blocks per K fragment
          f32x4 SA = f32x4{}, SB = f32x4{};
          if constexpr (KVD == 0) {
            bf16x8 kb[4];
            auto kload = [&](int c) {   // chunk group c>>1, half c&1
              return *(const LDS_PTR(bf16x8))(st + kbase + 2048 * (c >> 1) + 512 * (c & 1));
            };
#pragma unroll
            for (int c = 0; c < 3; ++c) kb[c] = kload(c);
#pragma unroll
            for (int c = 0; c < 18; ++c) {
              if (c + 3 < 18) kb[(c + 3) & 3] = kload(c + 3);
              SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[c & 3], qA[c], SA, 0, 0, 0);
              SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[c & 3], qB[c], SB, 0, 0, 0);
            }
          } else {
            i32x2 kb[4];
            auto kload = [&](int c) { return *(const LDS_PTR(i32x2))(st + kbase + 512 * c); };
#pragma unroll
            for (int c = 0; c < 3; ++c) kb[c] = kload(c);
#pragma unroll
            for (int c = 0; c < 18; ++c) {
              if (c + 3 < 18) kb[(c + 3) & 3] = kload(c + 3);
              const bf16x8 kf = e4m3x8_to_bf16(kb[c & 3]);
              SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qA[c], SA, 0, 0, 0);
              SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qB[c], SB, 0, 0, 0);
            }
          }

          // ---- online softmax.  Lane holds keys kt + 4*g4 + r (r = 0..3) of
          // row l16 (block A) and row 16 + l16 (block B).
          f32x4 ksc = f32x4{1.f, 1.f, 1.f, 1.f};
          if constexpr (KVD == 1) {
            const char* sp = smem + kScaleOff + wave * (kRounds<1> * kScaleSlotBytes) +
                             (j % NR) * kScaleSlotBytes + (t_in_round * kTileTok + 4 * g4) * 4;
            ksc = *(const LDS_PTR(f32x4))sp;
          }
          float sA[4], sB[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sA[r] = SA[r] * a.scale_log2;
            sB[r] = SB[r] * a.scale_log2;
            if constexpr (KVD == 1) {
              sA[r] *= ksc[r];
              sB[r] *= ksc[r];
            }
          }
          if (kt + kTileTok > lim_all) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = kt + 4 * g4 + r;
              sA[r] = key < limA ? sA[r] : -INFINITY;
              sB[r] = key < limB ? sB[r] : -INFINITY;
            }
          }
          float mxA = fmaxf(fmaxf(sA[0], sA[1]), fmaxf(sA[2], sA[3]));
          float mxB = fmaxf(fmaxf(sB[0], sB[1]), fmaxf(sB[2], sB[3]));
          mxA = quad_max(mxA);
          mxB = quad_max(mxB);
          // a row's first visible tile fixes its reference max
          mA = (mA == -INFINITY) ? mxA : mA;
          mB = (mB == -INFINITY) ? mxB : mB;
          if (__any((mxA > mA + kRestartMargin) || (mxB > mB + kRestartMargin))) {
            mA = fmaxf(mA, mxA);
            mB = fmaxf(mB, mxB);
            overshoot = true;
            if constexpr (PH != 4) *restart_flag = 1;
            break;
          }
          float pA[4], pB[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pA[r] = (mA == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sA[r] - mA);
            pB[r] = (mB == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sB[r] - mB);
            lA += pA[r];
            lB += pB[r];
            if constexpr (KVD == 1) {
              pA[r] *= ksc[r];
              pB[r] *= ksc[r];
            }
          }
          // probabilities -> B operand of the 32x32x16 PV step (keys in order)
          bf16x8 pf;
          {
            bf16x4 xa, xb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              xa[r] = (__bf16)pA[r];
              xb[r] = (__bf16)pB[r];
            }
            const u32x2 ua = __builtin_bit_cast(u32x2, xa), ub = __builtin_bit_cast(u32x2, xb);
            auto s0 = __builtin_amdgcn_permlane16_swap(ua.x, ub.x, false, false);
            auto s1 = __builtin_amdgcn_permlane16_swap(ua.y, ub.y, false, false);
            const u32x2 lo = {s0[0], s1[0]}, hi = {s0[1], s1[1]};
            const bf16x4 blo = __builtin_bit_cast(bf16x4, lo), bhi = __builtin_bit_cast(bf16x4, hi);
            pf = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
          }

          // ---- O^T[512 x 32] += V^T . P^T: 16 column blocks, V fragments 2 ahead
          if constexpr (KVD == 0) {
            auto vload = [&](int cb) {
              const int o = 2048 * (cb >> 1) + 512 * (cb & 1);
              const char* p1 = st + vbase1 + o;
              const char* p2 = st + vbase2 + o;
              const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))p1);
              const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))p2);
              return (bf16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            bf16x8 vb[3];
            vb[0] = vload(0);
            vb[1] = vload(1);
#pragma unroll
            for (int cb = 0; cb < 16; ++cb) {
              if (cb + 2 < 16) vb[(cb + 2) % 3] = vload(cb + 2);
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[cb % 3], pf, acc[cb], 0, 0, 0);
            }
          } else {
            auto vload = [&](int cb) {
              return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(st + vbase1 + 512 * cb));
            };
            i32x2 vb[3];
            vb[0] = vload(0);
            vb[1] = vload(1);
#pragma unroll
            for (int cb = 0; cb < 16; ++cb) {
              if (cb + 2 < 16) vb[(cb + 2) % 3] = vload(cb + 2);
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(vb[cb % 3]), pf,
                                                                acc[cb], 0, 0, 0);
            }
          }
        }
      }
      // every wave must agree before the ring is reused: drain the copies
      MLA_VM_WAIT(0);
      if constexpr (PH != 4) {
        barrier();
        const bool again = *restart_flag != 0;
        barrier();
        if (!again) break;
        if (wave == 0 && lane == 0) *restart_flag = 0;
        barrier();
      } else {
        if (!overshoot) break;
      }
    }

    // ---- per-wave totals.  Accumulator lane owns row lane%32: block A for
    // (lane>>4)&1 == 0, block B otherwise.
    const float lAt = quad_sum(lA), lBt = quad_sum(lB);
    const bool inB = (g4 & 1) != 0;
    float m_own = inB ? mB : mA;
    float l_own = inB ? lBt : lAt;

    // ---- merge of the PH phases of each row group.  Phase p owns column
    // blocks [p*16/PH, (p+1)*16/PH); the other phases pass their (scaled)
    // blocks through LDS (the ring is free once every wave is done).  The
    // accumulator is only read, never written, so it stays in AGPRs.
    constexpr int NB = 16 / PH;        // blocks owned per phase
    f32x16 own[NB];                    // owned blocks, scaled and summed
    float M = m_own, Lt = l_own;
    if constexpr (PH > 1) {
      barrier();
      LDS_PTR(float) ml = (LDS_PTR(float))(smem + kMlOff);
      if (lane < 32) {
        ml[(wave * 32 + lane) * 2] = m_own;
        ml[(wave * 32 + lane) * 2 + 1] = l_own;
      }
      barrier();
      const int rl = lane & 31;
      M = -INFINITY;
#pragma unroll
      for (int p = 0; p < PH; ++p) M = fmaxf(M, ml[((p * RG + rg) * 32 + rl) * 2]);
      Lt = 0.f;
#pragma unroll
      for (int p = 0; p < PH; ++p) {
        const float mp = ml[((p * RG + rg) * 32 + rl) * 2];
        const float lp = ml[((p * RG + rg) * 32 + rl) * 2 + 1];
        Lt += (mp == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mp - M) * lp;
      }
      const float f_own = (m_own == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_own - M);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
        if (cb / NB == ph) own[cb % NB] = acc[cb] * f_own;
      // exchange in steps of at most 2 destination phases (32 KB per wave)
      constexpr int STEP = PH == 2 ? 1 : 2;
      auto slot_addr = [&](int srg, int sph, int d, int cbl, int q4) -> LDS_PTR(f32x4) {
        // [row group][writer phase][destination index][block][q4][lane] x 16 B
        return (LDS_PTR(f32x4))(smem + (((((srg * PH + sph) * STEP + d) * NB + cbl) * 4 + q4) *
                                             64 + lane) * 16);
      };
#pragma unroll
      for (int s0 = 1; s0 < PH; s0 += STEP) {
#pragma unroll
        for (int d = 0; d < STEP; ++d) {
          const int s = s0 + d;
          if (s >= PH) break;
          const int owner = (ph + s) % PH;
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            if (cb / NB != owner) continue;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * f_own;
              *slot_addr(rg, ph, d, cb % NB, q4) = v;
            }
          }
        }
        barrier();
#pragma unroll
        for (int d = 0; d < STEP; ++d) {
          const int s = s0 + d;
          if (s >= PH) break;
          const int src = (ph - s + PH) % PH;   // wave that wrote this phase's blocks
#pragma unroll
          for (int cbl = 0; cbl < NB; ++cbl) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 v = *slot_addr(rg, src, d, cbl, q4);
#pragma unroll
              for (int e = 0; e < 4; ++e) own[cbl][4 * q4 + e] += v[e];
            }
          }
        }
        barrier();
      }
    }

    // ---- epilogue: lane owns row lane%32, columns 32cb + 8(r/4) + 4(lane/32) + r%4
    {
      const bool empty = !(Lt > 0.f);
      const float inv = empty ? 0.f : 1.f / Lt;
      const float lse_v = empty ? -INFINITY : (M + __log2f(Lt)) * kLn2;
      const int rl = lane & 31;
      const int row = row_base + 32 * rg + rl;
      const bool valid = row < R;
      const int t = valid ? row / H : 0, h = valid ? row - t * H : 0;
      const int hl = lane >> 5;
      auto block = [&](int cb) -> f32x16 {
        if constexpr (PH == 1) return acc[cb];
        else return own[cb % NB];
      };
      if (valid) {
        if (slot < 0) {
          uint8_t* op = o + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDLatent * 2);
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            if (PH > 1 && cb / NB != ph) continue;
            const f32x16 blk = block(cb);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              bf16x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (__bf16)(blk[4 * q4 + e] * inv);
              *reinterpret_cast<bf16x4*>(op + (32 * cb + 8 * q4 + 4 * hl) * 2) = v;
            }
          }
          if (lse && hl == 0 && ph == 0) lse[(b * a.max_q_len + t) * H + h] = lse_v;
        } else {
          const int rb = slot_row + 32 * rg + rl;
          float* pp = part_o + ((int64_t)slot * kRowsPerBlock + rb) * kDLatent;
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
            if (PH > 1 && cb / NB != ph) continue;
            const f32x16 blk = block(cb);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = blk[4 * q4 + e] * inv;
              *reinterpret_cast<f32x4*>(pp + 32 * cb + 8 * q4 + 4 * hl) = v;
            }
          }
          if (hl == 0 && ph == 0) part_lse[(int64_t)slot * kRowsPerBlock + rb] = lse_v;
        }
      }
    }
    // every wave leaves the ring (and the merge buffers) before the next
    // item's prologue refills them
    barrier();
  }
}

// max / sum over the two lanes {l, l^32} that share a score row
__device__ __forceinline__ float pair_max(float x) {
  const unsigned v = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned v = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}


// One workgroup = four waves, each owning 32 query rows of a 128-row block;
// all four read every key tile.  Keys are processed in pairs of 16-key ring
// stages (32 keys): S^T[32 keys x 32 rows] = K . Q^T on 32x32x16 MFMA puts
// a whole score row in the lane pair {l, l^32} (16 keys each), so the row
// max is one lane swap and the probabilities are the B operand of the PV
// step with no permute (the PV contraction takes the keys in the order the
// score layout holds them; V^T is read in the same order).  bf16 caches only:
// with e4m3 widening in the loop this schedule no longer fits the registers.
template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel_pairs(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  static_assert(KVD == 0, "the 32-key kernel takes bf16 caches");
  using C = Cfg<KVD>;
  constexpr int NR = kRounds<KVD>;
  constexpr int KW = 4;   // K fragments in flight in the QK step
  constexpr int VW = 4;   // V fragments in flight in the PV step
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  const uint32_t smem_base = lds_address(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int bid = blockIdx.x;
  const int nwg = a.num_wg;
  const int g = (nwg % 8 == 0) ? (bid & 7) * (nwg >> 3) + (bid >> 3) : bid;

  if (tid == 0) *(volatile LDS_PTR(int))(smem + kFlagOff) = 0;
  barrier();

  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  const int it_begin = wg_start[g], it_end = wg_start[g + 1];
  const int H = a.num_heads;

  // ---- per-lane LDS read offsets, relative to the first stage of a pair.
  // K fragment of QK step c (32 keys x 16 dims, A operand): key l32 of the
  // pair (stage l32/16, row l32%16), dims 16c + 8hl ..; its offset is
  // kb[c&1] + (c>>2)*KSTEP + (c&3)*256.  V^T fragment of PV step s (keys of
  // stage s), column block cb: column 32cb + l32 and, for hl = 0, keys
  // 0..3 and 8..11 of the stage, for hl = 1 keys 4..7 and 12..15.
  int kb_e, kb_o, vb1, vb2;
  {
    const int rl = l32 & 15, rh = rl >> 3, r8 = rl & 7, sp = l32 >> 4;
    kb_e = sp * C::TILE + rh * 1024 + (8 * (hl ^ rh) + r8) * 16;
    kb_o = sp * C::TILE + rh * 1024 + (8 * (hl ^ rh) + (r8 ^ 4)) * 16;
    const int i = l16, G = g4 & 1, u = (i >> 1) & 1, rr = 4 * hl + (i >> 2);
    vb1 = (16 * G + 8 * u + (rr ^ (4 * G))) * 16 + 8 * (i & 1);
    vb2 = 1024 + (16 * G + 8 * (u ^ 1) + (rr ^ (4 * G))) * 16 + 8 * (i & 1);
  }
  constexpr int KSTEP = 2048;   // 4 QK steps (64 dims) of a key row
  volatile LDS_PTR(int) restart_flag = (volatile LDS_PTR(int))(smem + kFlagOff);

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* item = items + it * kItemWords;
    const int b = item[0], row_base = item[1], k0 = item[2], k1 = item[3], slot = item[4];
    const int slot_row = item[5];
    const int L = kv_lens[b];
    const int qb = q_lens ? q_lens[b] : a.max_q_len;
    const int R = qb * H;
    const int ntiles = k1 > k0 ? (k1 - k0 + kTileTok - 1) / kTileTok : 0;
    const int nrounds = (ntiles + kRoundTiles - 1) / kRoundTiles;

    // this lane's query row: l32 of the wave's 32 (lanes l and l^32 share it)
    const int row = row_base + 32 * wave + l32;
    const bool valid = row < R;
    const int t = valid ? row / H : 0, h = valid ? row - t * H : 0;
    const int vis = a.causal ? L - qb + t + 1 : L;
    // rows past the sequence's last query row run over all keys (never
    // written), so that they never force the masked path
    const int lim = valid ? min(vis, k1) : k1;
    int lim_all = lim;
    lim_all = min(lim_all, __shfl_xor(lim_all, 1));
    lim_all = min(lim_all, __shfl_xor(lim_all, 2));
    lim_all = min(lim_all, __shfl_xor(lim_all, 4));
    lim_all = min(lim_all, __shfl_xor(lim_all, 8));
    lim_all = min(lim_all, __shfl_xor(lim_all, 16));
    lim_all = __builtin_amdgcn_readfirstlane(lim_all);

    // ---- Q^T fragments (B operand): row l32, dims 16c + 8hl .. +7
    bf16x8 qf[36];
    {
      const uint8_t* qp = qg + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDQK * 2) + hl * 16;
#pragma unroll
      for (int c = 0; c < 36; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 32);
    }

    DmaCtx<KVD> dc;
    dc.kv = kvg;
    dc.kv_scale = kv_scale;
    dc.bt_row = block_table + (int64_t)b * a.max_pages;
    dc.ring = smem_base;
    dc.scales = smem_base + kScaleOff + wave * (kRounds<1> * kScaleSlotBytes);
    dc.page_shift = a.page_shift;
    dc.k0 = k0;
    dc.L = L;
    dc.ntiles = ntiles;
    dc.wave = wave;
    dc.lane = lane;

    f32x16 acc[16];
    float m = -INFINITY, l = 0.f;
    for (;;) {   // runs once unless a score overshoots the reference max
#pragma unroll
      for (int j = 0; j < NR - 1; ++j)
        if (j < nrounds) issue_round<KVD>(dc, j);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
      l = 0.f;
      bool overshoot = false;   // wave-uniform

      for (int j = 0; j < nrounds; ++j) {
        const int ahead = min(nrounds, j + NR - 1) - j - 1;
        vm_wait_rounds<KVD>(ahead);
        barrier();   // tiles of round j come from all waves
        if (*restart_flag) {
          overshoot = true;
          break;
        }
        if (j + NR - 1 < nrounds) issue_round<KVD>(dc, j + NR - 1);

#pragma unroll
        for (int pp = 0; pp < kRoundTiles / 2; ++pp) {
          const int tile = kRoundTiles * j + 2 * pp;   // first tile of the pair
          if (tile >= ntiles) break;
          const int kp = k0 + kTileTok * tile;          // first key of the pair
          const char* st = smem + (tile % C::STAGES) * C::TILE;

          // ---- S^T = K . Q^T over 36 steps of 16 dims
          f32x16 S = f32x16{};
          {
            auto kload = [&](int c) -> bf16x8 {
              const int o = ((c & 1) ? kb_o : kb_e) + (c >> 2) * KSTEP + (c & 3) * 256;
              return *(const LDS_PTR(bf16x8))(st + o);
            };
            bf16x8 kb[KW];
#pragma unroll
            for (int c = 0; c < KW - 1; ++c) kb[c] = kload(c);
#pragma unroll
            for (int c = 0; c < 36; ++c) {
              if (c + KW - 1 < 36) kb[(c + KW - 1) % KW] = kload(c + KW - 1);
              S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c % KW], qf[c], S, 0, 0, 0);
            }
          }

          // ---- online softmax over keys kp + 8(r/4) + 4hl + r%4 (r = 0..15)
          float s[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = S[r] * a.scale_log2;
          if (kp + 2 * kTileTok > lim_all) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kp + 8 * (r >> 2) + 4 * hl + (r & 3);
              s[r] = key < lim ? s[r] : -INFINITY;
            }
          }
          float mx = s[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
          mx = pair_max(mx);
          // a row's first visible pair fixes its reference max
          m = (m == -INFINITY) ? mx : m;
          if (__any(mx > m + kRestartMargin)) {
            m = fmaxf(m, mx);
            overshoot = true;
            *restart_flag = 1;
            break;
          }
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[r] - m);
            l += p[r];
          }
          bf16x8 pf[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)p[r];

          // ---- O^T[512 x 32] += V^T . P^T: 2 key steps x 16 column blocks
          {
            auto vload = [&](int n) -> bf16x8 {   // n = 16 * step + cb
              const int sidx = n >> 4, cb = n & 15;
              const char* sb = st + sidx * C::TILE;
              const int o = 2048 * (cb >> 1) + 512 * (cb & 1);
              const bf16x4 lo =
                  __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + vb1 + o));
              const bf16x4 hi =
                  __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + vb2 + o));
              return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            bf16x8 vf[VW];
#pragma unroll
            for (int n = 0; n < VW - 1; ++n) vf[n] = vload(n);
#pragma unroll
            for (int n = 0; n < 32; ++n) {
              if (n + VW - 1 < 32) vf[(n + VW - 1) % VW] = vload(n + VW - 1);
              const int cb = n & 15;
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n % VW], pf[n >> 4], acc[cb],
                                                                0, 0, 0);
            }
          }
        }
      }
      // every wave must agree before the ring is reused: drain the copies
      MLA_VM_WAIT(0);
      barrier();
      const bool again = *restart_flag != 0;
      barrier();
      if (!again) break;
      if (wave == 0 && lane == 0) *restart_flag = 0;
      barrier();
    }

    // ---- epilogue: lane owns row l32, columns 32cb + 8(r/4) + 4hl + r%4
    {
      const float lt = pair_sum(l);
      const bool empty = !(lt > 0.f);
      const float inv = empty ? 0.f : 1.f / lt;
      const float lse_v = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
      if (valid) {
        if (slot < 0) {
          uint8_t* op = o + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDLatent * 2);
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              bf16x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * inv);
              *reinterpret_cast<bf16x4*>(op + (32 * cb + 8 * q4 + 4 * hl) * 2) = v;
            }
          }
          if (lse && hl == 0) lse[(b * a.max_q_len + t) * H + h] = lse_v;
        } else {
          const int rb = slot_row + 32 * wave + l32;
          float* pp = part_o + ((int64_t)slot * kRowsPerBlock + rb) * kDLatent;
#pragma unroll
          for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * inv;
              *reinterpret_cast<f32x4*>(pp + 32 * cb + 8 * q4 + 4 * hl) = v;
            }
          }
          if (hl == 0) part_lse[(int64_t)slot * kRowsPerBlock + rb] = lse_v;
        }
      }
    }
    // every wave leaves the ring before the next item's prologue refills it
    barrier();
  }
}


template <int KVD>
hipError_t launch_kvd(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_wg), block(kThreads);
  switch (a.phases) {
    case 1:
      if constexpr (KVD == 0)   // bf16, one workgroup per block: 32-key score steps
        hipLaunchKernelGGL((mla_decode_kernel_pairs<KVD>), grid, block, 0, stream, a, a.plan, a.q,
                           a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse,
                           a.part_o, a.part_lse);
      else
        hipLaunchKernelGGL((mla_decode_kernel<KVD, 1>), grid, block, 0, stream, a, a.plan, a.q,
                           a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse,
                           a.part_o, a.part_lse);
      break;
    case 2: hipLaunchKernelGGL((mla_decode_kernel<KVD, 2>), grid, block, 0, stream, a, a.plan, a.q,
                                  a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse,
                                  a.part_o, a.part_lse); break;
    case 4: hipLaunchKernelGGL((mla_decode_kernel<KVD, 4>), grid, block, 0, stream, a, a.plan, a.q,
                                  a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse,
                                  a.part_o, a.part_lse); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

#ifdef MLA_DECODE_Q_RESIDENT
hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  return kv_dtype == 1 ? launch_kvd<1>(a, stream) : hipErrorInvalidValue;
}
#else
hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  return kv_dtype == 0 ? launch_kvd<0>(a, stream) : launch_kvd<1>(a, stream);
}
#endif

}  // namespace mla
