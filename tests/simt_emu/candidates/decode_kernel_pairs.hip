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
// CANDIDATE REVISION of csrc/decode_kernel.hip, kept with the CPU emulator:
// it has passed the emulated parity cases (tests/test_kernel_emulated.py) but
// has not run on a GPU, and the library does not build it.  Everything but
// the per-tile compute is the library kernel's (copy ring, waits, barriers,
// restart, epilogue); only one workgroup per 128-row block (PH = 1).
//
// Change: keys are processed in pairs of 16-key ring stages (32 keys).
//   * QK^T: S^T[32 keys x 32 rows] = K . Q^T on v_mfma_f32_32x32x16_bf16; a
//     lane holds 16 keys of one score row, its partner lane l^32 the other
//     16, so the row max is one v_permlane32_swap.
//   * The PV contraction takes the keys in the order the score layout holds
//     them (lane half hl: keys 0-3, 8-11 / 4-7, 12-15 of each stage), so the
//     probabilities are the B operand with no permute; V^T is read by
//     ds_read_b64_tr_b16 (tr_b8 for e4m3) in the same key order.
//   * Per 32 keys the compiler moves 48 accumulator registers between AGPRs
//     and VGPRs (the library kernel: 208), and issues about half the VALU
//     work of two 16-key tiles.
// Open: the e4m3 instantiation spills inside the key loop.
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

#ifndef MLA_KW5
#define MLA_KW5 4
#endif
#ifndef MLA_VW5
#define MLA_VW5 4
#endif

// One workgroup = four waves, each owning 32 query rows of a 128-row block;
// all four read every key tile.  Keys are processed in pairs of 16-key ring
// stages (32 keys): S^T[32 keys x 32 rows] = K . Q^T on 32x32x16 MFMA puts
// a whole score row in the lane pair {l, l^32} (16 keys each), so the row
// max is one lane swap and the probabilities are the B operand of the PV
// step with no permute (the PV contraction takes the keys in the order the
// score layout holds them; V^T is read in the same order).
template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = Cfg<KVD>;
  constexpr int NR = kRounds<KVD>;
  constexpr int KW = MLA_KW5;
  constexpr int VW = MLA_VW5;
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
  if constexpr (KVD == 0) {
    const int rl = l32 & 15, rh = rl >> 3, r8 = rl & 7, sp = l32 >> 4;
    kb_e = sp * C::TILE + rh * 1024 + (8 * (hl ^ rh) + r8) * 16;
    kb_o = sp * C::TILE + rh * 1024 + (8 * (hl ^ rh) + (r8 ^ 4)) * 16;
    const int i = l16, G = g4 & 1, u = (i >> 1) & 1, rr = 4 * hl + (i >> 2);
    vb1 = (16 * G + 8 * u + (rr ^ (4 * G))) * 16 + 8 * (i & 1);
    vb2 = 1024 + (16 * G + 8 * (u ^ 1) + (rr ^ (4 * G))) * 16 + 8 * (i & 1);
  } else {
    const int rl = l32 & 15, sp = l32 >> 4;
    kb_e = sp * C::TILE + rl * 16 + 8 * hl;
    kb_o = sp * C::TILE + (rl ^ 8) * 16 + 8 * hl;
    const int i = l16, G = g4 & 1, k = i >> 1;
    const int key = (k & 3) + 4 * hl + 8 * (k >> 2);
    vb1 = (16 * G + (key ^ (8 * G))) * 16 + 8 * (i & 1);
    vb2 = 0;
  }
  constexpr int KSTEP = KVD == 0 ? 2048 : 1024;   // 4 QK steps (64 dims) of a key row
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
            typedef typename std::conditional<KVD == 0, bf16x8, i32x2>::type KFrag;
            auto kload = [&](int c) -> KFrag {
              const int o = ((c & 1) ? kb_o : kb_e) + (c >> 2) * KSTEP + (c & 3) * 256;
              return *(const LDS_PTR(KFrag))(st + o);
            };
            KFrag kb[KW];
#pragma unroll
            for (int c = 0; c < KW - 1; ++c) kb[c] = kload(c);
#pragma unroll
            for (int c = 0; c < 36; ++c) {
              if (c + KW - 1 < 36) kb[(c + KW - 1) % KW] = kload(c + KW - 1);
              if constexpr (KVD == 0)
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c % KW], qf[c], S, 0, 0, 0);
              else
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(kb[c % KW]), qf[c],
                                                            S, 0, 0, 0);
            }
          }

          // ---- online softmax over keys kp + 8(r/4) + 4hl + r%4 (r = 0..15)
          float s[16];
          if constexpr (KVD == 1) {
            const char* sp = smem + kScaleOff + wave * (kRounds<1> * kScaleSlotBytes) +
                             (j % NR) * kScaleSlotBytes + (32 * pp + 4 * hl) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 ks = *(const LDS_PTR(f32x4))(sp + 32 * q);
#pragma unroll
              for (int e = 0; e < 4; ++e) s[4 * q + e] = S[4 * q + e] * (a.scale_log2 * ks[e]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = S[r] * a.scale_log2;
          }
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
          if constexpr (KVD == 1) {
            const char* sp = smem + kScaleOff + wave * (kRounds<1> * kScaleSlotBytes) +
                             (j % NR) * kScaleSlotBytes + (32 * pp + 4 * hl) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 ks = *(const LDS_PTR(f32x4))(sp + 32 * q);
#pragma unroll
              for (int e = 0; e < 4; ++e) p[4 * q + e] *= ks[e];
            }
          }
          bf16x8 pf[2];
#pragma unroll
          for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)p[r];

          // ---- O^T[512 x 32] += V^T . P^T: 2 key steps x 16 column blocks
          {
            typedef typename std::conditional<KVD == 0, bf16x8, i32x2>::type VFrag;
            auto vload = [&](int n) -> VFrag {   // n = 16 * step + cb
              const int sidx = n >> 4, cb = n & 15;
              const char* sb = st + sidx * C::TILE;
              if constexpr (KVD == 0) {
                const int o = 2048 * (cb >> 1) + 512 * (cb & 1);
                const bf16x4 lo =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + vb1 + o));
                const bf16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + vb2 + o));
                return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
              } else {
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2))(sb + vb1 + 512 * cb));
              }
            };
            VFrag vf[VW];
#pragma unroll
            for (int n = 0; n < VW - 1; ++n) vf[n] = vload(n);
#pragma unroll
            for (int n = 0; n < 32; ++n) {
              if (n + VW - 1 < 32) vf[(n + VW - 1) % VW] = vload(n + VW - 1);
              const int cb = n & 15;
              if constexpr (KVD == 0)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n % VW], pf[n >> 4], acc[cb],
                                                                  0, 0, 0);
              else
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(vf[n % VW]),
                                                                  pf[n >> 4], acc[cb], 0, 0, 0);
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
  if (a.phases != 1) return hipErrorInvalidValue;
  const dim3 grid(a.num_wg), block(kThreads);
  hipLaunchKernelGGL((mla_decode_kernel<KVD>), grid, block, 0, stream, a, a.plan, a.q, a.kv,
                     a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse, a.part_o,
                     a.part_lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  return kv_dtype == 0 ? launch_kvd<0>(a, stream) : launch_kvd<1>(a, stream);
}

}  // namespace mla
