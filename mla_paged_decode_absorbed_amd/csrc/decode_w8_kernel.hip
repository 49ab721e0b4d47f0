// Weight-absorbed MLA decode over a paged latent cache, two waves per SIMD:
// a candidate successor of the library's decode kernels for one-phase plans,
// bf16 or e4m3 cache.  It computes what they compute (same plan, same work
// items, same outputs and partials):
//   s_j = scale * <q, c_j> over the visible cached rows, O = softmax(s) .
//   latent, LSE (KsanaLLM 0.6.0 page, weight-absorbed MLA for decode;
//   PaddlePaddle 3.0 inference page, draft tokens verified in one pass;
//   FlashAttention-3 in DeepSeek-R1 page, chapter 2: LSE and split-K; same
//   page, section 3.1: per-token fp8 cache scales).
//
// Why: with one wave per SIMD, the library kernels serialise each wave's
// chain QK^T -> softmax -> PV, and the matrix unit sits idle during the
// softmax and the LDS waits.  Here the 128 rows of a work item are spread
// over eight waves of 16 rows, two per SIMD, so one wave's softmax and waits
// can run under the other wave's MFMAs.  A wave then has 256 registers:
// Q (16 rows x 576) takes 72, the output accumulator (16 rows x 512 fp32)
// 128.  Every wave reads every key tile from LDS (twice the LDS reads per key
// of the four-wave kernels; the layout keeps them free of bank conflicts).
//
// Mapping onto CDNA4:
//   * 512 threads (eight wave64s), one workgroup per CU, persistent over its
//     plan items; wave w owns rows 16w .. 16w + 15 of an item.
//   * bf16: key tiles of 16 tokens stream HBM -> LDS through the library's
//     8-stage ring and tile layout, in rounds of four tiles: tile t of a
//     round is copied by waves t and t + 4, nine 1 KB copies each.
//   * e4m3: a round of 64 keys (36 KB, contiguous in its page) is copied as
//     it lies into a two-round ring, then widened once per CU, a 32-key pair
//     at a time, into one of two pair buffers in the bf16 tile layout (exact:
//     every e4m3 value is a bf16 value); the per-key scale multiplies the
//     score and the probability, so Q keeps bf16 and the MFMA steps are the
//     bf16 ones.  Widening in LDS costs each CU one conversion per cached
//     value, where widening K and V fragments in registers would cost every
//     wave one.
//   * Keys are processed 32 at a time (two 16-key stages).  QK^T: S^T[16 keys
//     x 16 rows] = K . Q^T on v_mfma_f32_16x16x32_bf16 for each stage, 18
//     steps of 32 dimensions sharing the Q fragment; a lane holds keys
//     4(lane/16) + r of its row in each stage.
//   * PV: O^T[16 columns x 16 rows] += V^T . P^T on v_mfma_f32_16x16x32_bf16
//     for 32 column blocks.  The contraction takes a lane's own 8 keys (four
//     of each stage) in the order it holds them, so the probabilities are the
//     B operand with no lane exchange; V^T is read by ds_read_b64_tr_b16, four
//     keys of one stage per read.
//   * The softmax keeps the library kernels' fixed reference max: a row's
//     reference is its first visible pair's max, and probabilities are taken
//     against it with no rescaling while scores stay within 32 (log2 units)
//     of it (fp32 and bf16 keep full relative precision below 2^32).  When a
//     row's score overshoots by more, the library kernels restart the item;
//     here the accumulator is in VGPRs, so the wave raises the reference of
//     its overshooting rows and rescales their sums in place (128
//     multiplications per lane), with no exchange between waves: each wave's
//     rows are its own.  An item's cost is then linear in its length for any
//     scores.
//   * An item's key range is clamped to the sequence's device length, so a
//     plan made for longer lengths reads no row past the sequence's pages.
//   * Split row blocks leave bf16 partials (normalised O) and fp32 LSE, which
//     mla_combine_kernel_bf16 merges: half the partial bytes of the library
//     kernels' fp32 partials, written once and read once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_asm.h"
#include "kernels.h"
#include "plan_layout.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kTileTok = 16;                  // keys per ring stage
constexpr int kRoundTiles = 4;                // stages per round
constexpr int kRoundTok = kTileTok * kRoundTiles;
constexpr int kRowBytes = 1152;               // one bf16 cache row
constexpr int kTileBytes = kTileTok * kRowBytes;
constexpr int kF8RowBytes = 576;              // one e4m3 cache row
constexpr int kF8RoundBytes = kRoundTok * kF8RowBytes;   // one round of e4m3 rows, 36 KB
constexpr int kF8Copies = kF8RoundBytes / 1024;          // its 1 KB copies
constexpr int kScaleRoundBytes = kRoundTok * 4;          // one round's fp32 scales

// LDS map.  bf16: an 8-stage ring of key tiles (two rounds).  e4m3: two pair
// buffers of two bf16 tiles each (the keys being computed, widened), a ring
// of two e4m3 rounds in cache row order, the rounds' scales and the pair
// buffers' scales.
template <int KVD> struct Lds;
template <> struct Lds<0> {
  static constexpr int kStages = 8;
  static constexpr int kBytes = kStages * kTileBytes;
};
template <> struct Lds<1> {
  static constexpr int kStages = 4;
  static constexpr int kRing = kStages * kTileBytes;
  static constexpr int kRingScale = kRing + 2 * kF8RoundBytes;
  static constexpr int kPairScale = kRingScale + 2 * kScaleRoundBytes;
  static constexpr int kBytes = kPairScale + 2 * 2 * kTileTok * 4;
};
static_assert(Lds<1>::kBytes <= 160 * 1024, "e4m3 LDS map exceeds a workgroup's LDS");
constexpr float kRescaleMargin = 32.0f;       // log2 units above the reference max
constexpr float kLn2 = 0.69314718055994530942f;

// A wave-uniform pointer, kept in SGPRs (the copies take a scalar base).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

// max / sum over the 4 lanes {l, l^16, l^32, l^48} that share a score row
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

struct Ring {
  const uint8_t* kv;
  const int32_t* bt_row;
  uint32_t lds;        // LDS address of the ring
  int page_shift, k0, L, ntiles, lane;
};

// First key of tile t of round j: a tile past the item stands for the
// round's first key (a harmless dummy copy of real cache rows).
__device__ __forceinline__ int tile_key(const Ring& r, int t, int j) {
  const int tile = kRoundTiles * j + t;
  return tile < r.ntiles ? r.k0 + kTileTok * tile : r.k0 + kRoundTok * j;
}

// The cache page holding tile t of round j (a block-table read, issued a
// round ahead of the copies that use it).
__device__ __forceinline__ int tile_page(const Ring& r, int t, int j) {
  return r.bt_row[tile_key(r, t, j) >> r.page_shift];
}

// This wave's share of round j: half HALF (copies 9*HALF .. 9*HALF + 8) of
// tile `t` of the round, which lies in page pg, into its ring stage (every
// wave issues exactly nine copies per round, so each wave's vmcnt count is
// the same).  Copy ins fills the stage's 1 KB block ins: rows 8(ins&1) .. +7,
// bytes 128(ins>>1) .. +127 of each row, in the library's tile layout.
template <int HALF>
__device__ __forceinline__ void issue_half(const Ring& r, int t, int j, int pg) {
  const int tile = kRoundTiles * j + t;
  const int stage = tile % Lds<0>::kStages;
  const bool real = tile < r.ntiles;
  const int kt = tile_key(r, t, j);
  const int pmask = (1 << r.page_shift) - 1;
  const int row0 = (pg << r.page_shift) + (kt & pmask);
  const uint8_t* base = uniform_ptr(r.kv + (int64_t)row0 * kRowBytes);
  const int nvalid = real ? min(kTileTok, r.L - kt) : 0;
  const uint32_t lds = r.lds + stage * kTileBytes;
  const int lane = opaque(r.lane);
  const int c8a = 2 * (lane >> 4), lo = (lane >> 3) & 1;
  const int r8 = (lane & 7) ^ (4 * ((lane >> 4) & 1));
  int vo[2];
#pragma unroll
  for (int rh = 0; rh < 2; ++rh) {
    const int row = 8 * rh + r8;
    const int c8 = c8a + (lo ^ rh);
    vo[rh] = (row < nvalid ? row * kRowBytes : 0) + c8 * 16;
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    constexpr int first = 9 * HALF;
    const int ins = first + k;
    lds_dma_x4(lds + ins * 1024, vo[ins & 1], base + 128 * (ins >> 1));
  }
}

__device__ __forceinline__ void issue_round(const Ring& r, int t, int half, int j, int pg) {
  if (half) issue_half<1>(r, t, j, pg);
  else issue_half<0>(r, t, j, pg);
}

// ---- e4m3 caches.  A round of 64 keys is one run of one page (pages hold a
// multiple of 64 rows and items start on a multiple of 64 keys), i.e. 36 KB
// contiguous in the cache, copied as it lies; the 64 scales of the round are
// contiguous too.
struct RingF8 {
  const uint8_t* kv;
  const float* kv_scale;
  const int32_t* bt_row;
  uint32_t ring, ring_scale;   // LDS addresses
  int page_shift, k0, L, wave, lane;
};

__device__ __forceinline__ int round_page_f8(const RingF8& r, int j) {
  return r.bt_row[(r.k0 + kRoundTok * j) >> r.page_shift];
}

// This wave's share of round j, which lies in page pg, into ring slot j & 1: copies wave, wave + 8,
// ... (< 36) of the round's 36 KB (copy ins = bytes 1024 ins .. + 1023, lane
// l taking 16 bytes at 16 l; a row is 36 such pieces, so a piece lies in one
// row), and for wave 7 the round's 64 scales.  Lanes whose piece lies in a
// row past the sequence's end are masked off, so no cache slot past the
// sequence is read (the widening zeroes those rows; a scale lane past the end
// copies the round's first scale).
__device__ __forceinline__ void issue_round_f8(const RingF8& r, int j, int pg) {
  const int kr = r.k0 + kRoundTok * j;          // first key of the round (< L)
  const int pmask = (1 << r.page_shift) - 1;
  const int row0 = (pg << r.page_shift) + (kr & pmask);
  const uint8_t* base = uniform_ptr(r.kv + (int64_t)row0 * kF8RowBytes);
  const uint32_t lds = r.ring + (j & 1) * kF8RoundBytes;
  const int lane = opaque(r.lane);
  const int vo = 16 * lane;
  // bytes of the round inside the sequence (rows < L - kr)
  const int valid_bytes = min(r.L - kr, kRoundTok) * kF8RowBytes;
  const int wave = opaque_s(r.wave);
#pragma unroll
  for (int k = 0; k < (kF8Copies + 7) / 8; ++k) {
    const int ins = wave + 8 * k;
    if (ins < kF8Copies && vo + 1024 * ins < valid_bytes)
      lds_dma_x4(lds + ins * 1024, vo, base + 1024 * ins);
  }
  if (wave == 7) {
    const int tok = lane < r.L - kr ? lane : 0;
    lds_dma_x1(r.ring_scale + (j & 1) * kScaleRoundBytes, tok * 4,
               uniform_ptr(r.kv_scale + row0));
  }
}

// Widen 8 e4m3 bytes to 8 bf16 values (exact: e4m3's values are bf16 values).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  bf16x8 v;
  v[0] = (__bf16)a.x; v[1] = (__bf16)a.y; v[2] = (__bf16)b.x; v[3] = (__bf16)b.y;
  v[4] = (__bf16)c.x; v[5] = (__bf16)c.y; v[6] = (__bf16)d.x; v[7] = (__bf16)d.y;
  return v;
}

// Widen pair p of the item (keys kp .. kp + 31, the half p & 1 of round p >> 1
// in ring slot (p >> 1) & 1) into pair buffer p & 1, in the bf16 tile layout
// the MFMA steps read, and its 32 scales into the buffer's scale slot.  The
// pair's 36 output blocks of 1 KB (stage bi / 18, block bi % 18 = 2 cg + rh:
// rows 8 rh .. + 7, chunks 8 cg .. + 7) go to the waves by bi % 8.  Lane l
// takes chunk c8 = l % 8 of row r8 = c8 ^ (l / 8): each 16 lanes then read
// one 8-byte piece per bank pair (rows 576 bytes apart fall on alternate
// halves of the banks, and the two rows of a chunk have opposite parity), and
// each 8 lanes write distinct 16-byte bank groups of the tile layout.  Rows at
// or past the sequence's end become zeros.
__device__ __forceinline__ void widen_pair_f8(char* smem, int p, int kp, int L, int wave_id,
                                              int lane_id) {
  // opaque copies of the lane and wave ids keep the per-lane offsets and the
  // per-wave conditions below inside the key loop rather than hoisted out of
  // it (they would pin registers there)
  const int lane = opaque(lane_id);
  const int wave = opaque_s(wave_id);
  const int rh = wave & 1;
  const int c8 = lane & 7;
  const int r8 = c8 ^ (lane >> 3);
  const int row = 8 * rh + r8;   // within a stage
  const int slot = 16 * (c8 >> 1) + 8 * ((c8 & 1) ^ rh) + (r8 ^ (4 * ((c8 >> 1) & 1)));
  const uint32_t src = Lds<1>::kRing + ((p >> 1) & 1) * kF8RoundBytes +
                       (p & 1) * (2 * kTileTok * kF8RowBytes) + row * kF8RowBytes + 8 * c8;
  const uint32_t dst = (p & 1) * 2 * kTileBytes + 16 * slot;
#pragma unroll
  for (int k = 0; k < (2 * 18 + 7) / 8; ++k) {
    const int bi = wave + 8 * k;
    if (bi < 2 * 18) {
      const int st = bi >= 18 ? 1 : 0;
      const int blk = bi - 18 * st, cg = blk >> 1;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 raw =
          *(const LDS_PTR(u32x2))(smem + src + st * kTileTok * kF8RowBytes + 64 * cg);
      bf16x8 v = e4m3x8_to_bf16(raw.x, raw.y);
      if (kp + kTileTok * st + row >= L) v = bf16x8{};
      *(LDS_PTR(bf16x8))(smem + dst + st * kTileBytes + blk * 1024) = v;
    }
  }
  if (wave == 5 && lane < 2 * kTileTok) {
    const float sc = *(const LDS_PTR(float))(smem + Lds<1>::kRingScale +
                                             ((p >> 1) & 1) * kScaleRoundBytes +
                                             ((p & 1) * 2 * kTileTok + lane) * 4);
    *(LDS_PTR(float))(smem + Lds<1>::kPairScale + ((p & 1) * 2 * kTileTok + lane) * 4) = sc;
  }
}

// Per-lane LDS read offsets of the MFMA operands (stage relative).
struct Frag {
  int kbase, vb_e, vb_o;
};

// QK^T, softmax and PV of one pair of 16-key stages (keys kp .. kp + 31) whose
// bf16 tiles sit at LDS offset so and so + one tile.  For e4m3 the 32 per-key
// scales at ksc_off multiply the scores and the probabilities.
template <int KVD>
__device__ __forceinline__ void pair_step(char* smem, const Frag& fr, int so, int ksc_off, int kp,
                                          int lim, int lim_all, float scale_log2, int g4,
                                          const bf16x8 (&qf)[18], f32x4 (&acc)[32], float& m,
                                          float& l) {
  constexpr int KW = 2;   // QK steps whose K fragments are in flight
  constexpr int VW = 3;   // PV column blocks whose V fragments are in flight
  // this pair's per-lane LDS bases: one add each per pair, through opaque
  // copies so that the compiler keeps three registers here rather than
  // precomputing a base per ring stage for the whole loop
  const int kb_s = opaque(fr.kbase + so);
  const int ve_s = opaque(fr.vb_e + so), vo_s = opaque(fr.vb_o + so);

  // ---- S^T = K . Q^T for both stages, 18 steps of 32 dims
  f32x4 SA = f32x4{}, SB = f32x4{};
  {
    auto kload = [&](int s, int c) -> bf16x8 {
      return *(const LDS_PTR(bf16x8))(smem + kb_s + s * kTileBytes + 2048 * (c >> 1) +
                                      512 * (c & 1));
    };
    bf16x8 ka[KW], kb[KW];
#pragma unroll
    for (int c = 0; c < KW - 1; ++c) {
      ka[c] = kload(0, c);
      kb[c] = kload(1, c);
    }
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      if (c + KW - 1 < 18) {
        ka[(c + KW - 1) % KW] = kload(0, c + KW - 1);
        kb[(c + KW - 1) % KW] = kload(1, c + KW - 1);
      }
      SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c % KW], qf[c], SA, 0, 0, 0);
      SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[c % KW], qf[c], SB, 0, 0, 0);
    }
  }

  // ---- online softmax: keys kp + 4g4 + r (stage 0), kp + 16 + 4g4 + r
  float s[8];
  f32x4 ka4, kb4;   // e4m3: the per-key scales of those keys
  if constexpr (KVD == 1) {
    ka4 = *(const LDS_PTR(f32x4))(smem + ksc_off + 16 * g4);
    kb4 = *(const LDS_PTR(f32x4))(smem + ksc_off + 64 + 16 * g4);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (KVD == 1) {
      s[r] = SA[r] * (scale_log2 * ka4[r]);
      s[4 + r] = SB[r] * (scale_log2 * kb4[r]);
    } else {
      s[r] = SA[r] * scale_log2;
      s[4 + r] = SB[r] * scale_log2;
    }
  }
  if (kp + 2 * kTileTok > lim_all) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = kp + 16 * (r >> 2) + 4 * g4 + (r & 3);
      s[r] = key < lim ? s[r] : -INFINITY;
    }
  }
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 8; ++r) mx = fmaxf(mx, s[r]);
  mx = quad_max(mx);
  // a row's first visible pair fixes its reference max
  m = (m == -INFINITY) ? mx : m;
  if (__any(mx > m + kRescaleMargin)) {
    // raise the overshooting rows' reference to this pair's max and rescale
    // their sums (a factor of at most 2^-32; 1 for the other rows)
    const float alpha = mx > m + kRescaleMargin ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
    m = mx > m + kRescaleMargin ? mx : m;
    l *= alpha;
#pragma unroll
    for (int cm = 0; cm < 32; ++cm) acc[cm] *= alpha;
  }
  bf16x8 pf;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float p = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[r] - m);
    l += p;
    if constexpr (KVD == 1)
      pf[r] = (__bf16)(p * (r < 4 ? ka4[r] : kb4[r - 4]));
    else
      pf[r] = (__bf16)p;
  }

  // ---- O^T[512 x 16] += V^T . P^T: 32 column blocks of 16
  {
    auto vload = [&](int cm) -> bf16x8 {
      const int off = ((cm & 1) ? vo_s : ve_s) + 2048 * (cm >> 2) + 256 * (cm & 3);
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(smem + off));
      const bf16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(smem + kTileBytes + off));
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vf[VW];
#pragma unroll
    for (int n = 0; n < VW - 1; ++n) vf[n] = vload(n);
#pragma unroll
    for (int cm = 0; cm < 32; ++cm) {
      if (cm + VW - 1 < 32) vf[(cm + VW - 1) % VW] = vload(cm + VW - 1);
      acc[cm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[cm % VW], pf, acc[cm], 0, 0, 0);
    }
  }
}

template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel_w8(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) char smem[Lds<KVD>::kBytes];
  const uint32_t smem_base = lds_address(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int tq = wave & 3, half = wave >> 2;   // the round tile this wave copies, and its half

  // Consecutive logical workgroups land on one XCD (dispatch is round-robin
  // over the 8 XCDs), so the CUs that share a sequence share an L2.
  const int bid = blockIdx.x;
  const int nwg = a.num_wg;
  const int g = (nwg % 8 == 0) ? (bid & 7) * (nwg >> 3) + (bid >> 3) : bid;

  barrier();

  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  const int it_begin = wg_start[g], it_end = wg_start[g + 1];
  const int H = a.num_heads;

  // ---- per-lane LDS read offsets (stage relative), constant over the run.
  // K fragment of QK step c (A operand, 16 keys x 32 dims): key l16 of the
  // stage, dims 32c + 8g4 .. +7, at kbase + 2048(c>>1) + 512(c&1).
  Frag fr;
  {
    const int kh = g4 >> 1, krh = l16 >> 3, kr8 = l16 & 7;
    fr.kbase = krh * 1024 + (16 * kh + 8 * ((g4 & 1) ^ krh) + (kr8 ^ (4 * kh))) * 16;
    // V^T fragment of PV column block m (A operand, 16 columns x 4 keys of a
    // stage): the lane names row 4g4 + l16/4, columns 16m + 4(l16%4) .. +3
    // and receives column 16m + l16, rows 4g4 .. 4g4 + 3; at vb[m&1] +
    // 2048(m>>2) + 256(m&3).
    const int vr = 4 * g4 + (l16 >> 2), vrh = vr >> 3, vr8 = vr & 7, vx = (l16 & 3) >> 1;
    fr.vb_e = vrh * 1024 + 16 * (8 * (vx ^ vrh) + vr8) + 8 * (l16 & 1);
    fr.vb_o = vrh * 1024 + 16 * (8 * (vx ^ vrh) + (vr8 ^ 4)) + 8 * (l16 & 1);
  }

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* item = items + it * kItemWords;
    const int b = item[0], row_base = item[1], slot = item[4];
    const int slot_row = item[5];
    const int L = kv_lens[b];
    // a plan made for other lengths never reads past the sequence
    const int k1 = min(item[3], L), k0 = min(item[2], k1);
    const int qb = q_lens ? q_lens[b] : a.max_q_len;
    const int R = qb * H;
    const int ntiles = k1 > k0 ? (k1 - k0 + kTileTok - 1) / kTileTok : 0;
    const int nrounds = (ntiles + kRoundTiles - 1) / kRoundTiles;

    // this lane's query row: l16 of the wave's 16 (lanes l16 + 16k share it)
    const int row = row_base + 16 * wave + l16;
    const bool valid = row < R;
    const int t = valid ? row / H : 0, h = valid ? row - t * H : 0;
    const int vis = a.causal ? L - qb + t + 1 : L;
    // rows past the sequence's last query row run over all keys (never
    // written), so that they never force the masked path
    const int lim = valid ? min(vis, k1) : k1;
    // the smallest lim of the wave's rows: visibility grows with the token,
    // so it is the wave's first row's (all rows are past the end if it is)
    const int first = row_base + 16 * wave;
    const int lim_all =
        first < R ? min(a.causal ? L - qb + first / H + 1 : L, k1) : k1;

    // ---- Q^T fragments (B operand): row, dims 32c + 8g4 .. +7
    bf16x8 qf[18];
    {
      // (through an opaque lane id: a per-lane base hoisted out of the item
      // loop would hold two registers through the key loop)
      const uint8_t* qp = qg + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDQK * 2) +
                          (opaque(lane) >> 4) * 16;
#pragma unroll
      for (int c = 0; c < 18; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 64);
    }

    f32x4 acc[32];
    float m = -INFINITY, l = 0.f;
    if constexpr (KVD == 0) {
      Ring ring;
      ring.kv = kvg;
      ring.bt_row = block_table + (int64_t)b * a.max_pages;
      ring.lds = smem_base;
      ring.page_shift = a.page_shift;
      ring.k0 = k0;
      ring.L = L;
      ring.ntiles = ntiles;
      ring.lane = lane;

#pragma unroll
      for (int cb = 0; cb < 32; ++cb) acc[cb] = f32x4{};
      if (nrounds > 0) issue_round(ring, tq, half, 0, tile_page(ring, tq, 0));
      // Q must be resident before the key loop: otherwise the compiler,
      // which does not see the copies, keeps its loads pending into the loop
      // and waits for them there with vmcnt literals that, at run time, also
      // count the next round's copies in flight.  Here the wave waits for
      // round 0 anyway (the loop's first wait).
#pragma unroll
      for (int c = 0; c < 18; ++c) require_vgpr(qf[c]);
      int pg = nrounds > 1 ? tile_page(ring, tq, 1) : 0;   // page of the next round's tile
      // Round j opens by waiting for this wave's copies and the barrier (the
      // round's tiles come from all waves, and every wave is done with the
      // stages round j + 1 refills); round j + 1, whose page was read in the
      // previous round, is then issued.
      for (int j = 0; j < nrounds; ++j) {
        MLA_VM_WAIT(0);
        barrier();   // tiles of round j come from all waves
        if (j + 1 < nrounds) issue_round(ring, tq, half, j + 1, pg);
#pragma unroll
        for (int pp = 0; pp < kRoundTiles / 2; ++pp) {
          const int tile = kRoundTiles * j + 2 * pp;   // first stage of the pair
          if (tile >= ntiles) break;
          const int kp = k0 + kTileTok * tile;          // first key of the pair
          const int so = (tile % Lds<0>::kStages) * kTileBytes;
          pair_step<0>(smem, fr, so, 0, kp, lim, lim_all, a.scale_log2, g4, qf, acc, m, l);
        }
        // the page of round j + 2's tile, read under the round's last MFMAs
        // and the barrier rather than between the barrier and the next pair
        if (j + 2 < nrounds) pg = tile_page(ring, tq, j + 2);
      }
    } else {
      RingF8 ring;
      ring.kv = kvg;
      ring.kv_scale = kv_scale;
      ring.bt_row = block_table + (int64_t)b * a.max_pages;
      ring.ring = smem_base + Lds<1>::kRing;
      ring.ring_scale = smem_base + Lds<1>::kRingScale;
      ring.page_shift = a.page_shift;
      ring.k0 = k0;
      ring.L = L;
      ring.wave = wave;
      ring.lane = lane;
      const int npairs = (ntiles + 1) >> 1;

      // Three stages per pair of 32 keys: copy (a round of two pairs at a
      // time), widen into a pair buffer, compute.  Iteration p widens pair
      // p + 1 and computes pair p between two barriers; round r + 1 is issued
      // in iteration 2r - 1, into the ring slot whose round was widened by
      // then, and waited for in iteration 2r + 1, the first to widen it.  Only
      // that round is in flight at the wait.
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) acc[cb] = f32x4{};
      int pg = 0;   // page of the next round to issue
      if (npairs > 0) {
        issue_round_f8(ring, 0, round_page_f8(ring, 0));
        MLA_VM_WAIT(0);
      }
      // Q resident before the key loop (see the bf16 path), on every path
      // into it
#pragma unroll
      for (int c = 0; c < 18; ++c) require_vgpr(qf[c]);
      if (npairs > 0) {
        barrier();   // round 0 comes from all waves
        widen_pair_f8(smem, 0, k0, L, wave, lane);
        if (nrounds > 1) issue_round_f8(ring, 1, round_page_f8(ring, 1));
        if (nrounds > 2) pg = round_page_f8(ring, 2);
      }
      // Pair p opens with the barrier after which pair p is widened by all
      // waves (and, for odd p, round (p + 1) / 2 has landed).  The two pairs
      // of a round are written out, so that a pair's parity (its buffer,
      // whether it waits and issues) is known at compile time.
      for (int j = 0; j < nrounds; ++j) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int p = 2 * j + pp;
          if (p >= npairs) break;
          if (pp == 1) MLA_VM_WAIT(0);
          barrier();   // pair p widened by all waves; for odd p, round j + 1 copied
          if (pp == 1 && j + 2 < nrounds) issue_round_f8(ring, j + 2, pg);
          if (p + 1 < npairs)
            widen_pair_f8(smem, p + 1, k0 + 2 * kTileTok * (p + 1), L, wave, lane);
          pair_step<1>(smem, fr, pp * 2 * kTileBytes, Lds<1>::kPairScale + pp * 2 * kTileTok * 4,
                       k0 + 2 * kTileTok * p, lim, lim_all, a.scale_log2, g4, qf, acc, m, l);
          // the page of round j + 3, read a round ahead of its copies
          if (pp == 1 && j + 3 < nrounds) pg = round_page_f8(ring, j + 3);
        }
      }
    }

    // ---- epilogue: lane owns row l16, columns 16cm + 4g4 + r.  The lane's
    // column offset goes through an opaque copy of the lane id, so that the
    // compiler does not hoist the output addresses out of the item loop (they
    // would pin registers through the key loop).
    {
      const int ge = opaque(lane) >> 4;
      const float lt = quad_sum(l);
      const bool empty = !(lt > 0.f);
      const float inv = empty ? 0.f : 1.f / lt;
      const float lse_v = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
      if (valid) {
        if (slot < 0) {
          uint8_t* op = o + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDLatent * 2);
#pragma unroll
          for (int cm = 0; cm < 32; ++cm) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cm][e] * inv);
            *reinterpret_cast<bf16x4*>(op + (16 * cm + 4 * ge) * 2) = v;
          }
          if (lse && ge == 0) lse[(b * a.max_q_len + t) * H + h] = lse_v;
        } else {
          // bf16 partials: half the bytes of fp32 ones, written here and
          // read back by the combine (mla_combine_kernel_bf16)
          const int rb = slot_row + 16 * wave + l16;
          uint8_t* pp = reinterpret_cast<uint8_t*>(part_o) +
                        ((int64_t)slot * kRowsPerBlock + rb) * (kDLatent * 2);
#pragma unroll
          for (int cm = 0; cm < 32; ++cm) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cm][e] * inv);
            *reinterpret_cast<bf16x4*>(pp + (16 * cm + 4 * ge) * 2) = v;
          }
          if (ge == 0) part_lse[(int64_t)slot * kRowsPerBlock + rb] = lse_v;
        }
      }
    }
    // every wave leaves the ring before the next item's prologue refills it
    barrier();
  }
}

}  // namespace

hipError_t launch_decode_w8(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (a.phases != 1) return hipErrorInvalidValue;
  if (kv_dtype == 0) {
    hipLaunchKernelGGL((mla_decode_kernel_w8<0>), dim3(a.num_wg), dim3(kThreads), 0, stream, a,
                       a.plan, a.q, a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o,
                       a.lse, a.part_o, a.part_lse);
  } else {
    hipLaunchKernelGGL((mla_decode_kernel_w8<1>), dim3(a.num_wg), dim3(kThreads), 0, stream, a,
                       a.plan, a.q, a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o,
                       a.lse, a.part_o, a.part_lse);
  }
  return hipGetLastError();
}

}  // namespace mla
