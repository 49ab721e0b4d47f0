// Weight-absorbed MLA decode over a paged latent cache, two waves per SIMD
// with the work of a 32-row group split between a pair of waves: a second
// candidate successor of the library's decode kernels for one-phase plans,
// bf16 or e4m3 cache.  It computes what they compute (same plan, same work
// items, same outputs; bf16 partials as the other two-waves-per-SIMD
// candidate writes them):
//   s_j = scale * <q, c_j> over the visible cached rows, O = softmax(s) .
//   latent, LSE (KsanaLLM 0.6.0 page, weight-absorbed MLA for decode;
//   PaddlePaddle 3.0 inference page, draft tokens verified in one pass, and
//   its MLA operator section: PV split across warp groups for registers;
//   FlashAttention-3 in DeepSeek-R1 page, chapter 2: LSE and split-K; same
//   page, section 3.1: per-token fp8 cache scales).
//
// Why: the 16-row candidate (decode_w8_kernel.hip) gives every wave all 576
// dimensions of K and all 512 columns of V, so a CU reads 544 KB from LDS per
// 32 keys, twice what the four-wave kernels read.  Here the two waves of a
// pair share 32 rows: wave half hf scores them over half of the 576
// dimensions and accumulates half of the 512 output columns.  The partial
// scores (32 x 32 fp32 per wave) are exchanged through LDS and added, so
// both waves of a pair hold the same scores and take the same softmax
// decisions, each for its own columns.  Per 32 keys and CU that is 144 KB of
// K reads, 128 KB of V reads and 64 KB of exchange: 336 KB.  A wave keeps
// the 256-register budget of two waves per SIMD: Q (32 rows x 288 dims) 72
// registers, the accumulator (32 rows x 256 columns fp32) 128.
//
// Mapping onto CDNA4:
//   * 512 threads (eight wave64s), one workgroup per CU, persistent over its
//     plan items.  Wave w takes row group w / 2 (rows 32 (w / 2) .. + 31 of
//     an item) and half w % 2; its partner is wave w ^ 1.  Waves w and w + 4
//     share a SIMD (waves are dealt to the four SIMDs in turn), so a SIMD
//     holds two different pairs, and while one pair exchanges and runs its
//     softmax the SIMD's other wave can keep the matrix unit busy.
//   * Keys go 32 at a time (a round: two 16-key stages in the library's bf16
//     tile layout).  bf16: rounds stream HBM -> LDS through a ring of three
//     rounds and are computed in place.  e4m3: a round (18 KB, contiguous in
//     its page) is copied as it lies into a ring of three e4m3 rounds, then
//     widened once per CU into one of two pair buffers in the bf16 tile
//     layout (exact: every e4m3 value is a bf16 value), whose 32 per-key
//     scales multiply the scores and the probabilities; the MFMA steps are
//     then the bf16 ones.  Either way round j + 2 (e4m3: j + 3) is issued
//     after the barrier that opens round j, into the slot of a round every
//     wave has finished, and every wave waits for a round with one vmcnt
//     literal while the next round is in flight (the literal is the smallest
//     number of copies any wave issues per round).
//   * QK^T: S^T[32 keys x 32 rows] on v_mfma_f32_32x32x16_bf16 (the library's
//     32-key step), 18 steps of 16 dimensions per wave: half hf takes the
//     steps c with (c / 2) % 2 == hf, which puts its K reads at a fixed
//     offset of 512 bytes from the other half's in the tile layout.  A lane
//     holds 16 keys of row l % 32, its partner lane l ^ 32 the other 16.
//   * Exchange: each wave writes its partial scores to its own LDS slot and
//     raises its round counter (an LDS word, after its writes complete); it
//     then waits for its partner's counter, reads the partner's partial and
//     adds it (the same sum in both waves: fp32 addition commutes).  A slot
//     is written again only after the next round's barrier, which the
//     partner reaches after reading it.  The wait always ends: the partner
//     raises its counter after its QK step, which waits for nothing of this
//     wave; a bound on the polls keeps even a broken invariant from hanging.
//   * Softmax: the library kernels' fixed reference max; a score above it by
//     more than 32 (log2 units) raises the reference of that row and rescales
//     its sums in place (both waves of a pair decide alike on the same
//     scores), so there is no restart and an item's cost is linear in its
//     length.
//   * PV: O^T[256 x 32 rows] += V^T . P^T on v_mfma_f32_32x32x16_bf16, 8
//     column blocks x 2 key steps per wave, half hf taking columns 256 hf ..
//     + 255 (a fixed offset of 8 KB in the tile layout); the probabilities
//     are the B operand in the order the score layout holds them, V^T comes
//     from ds_read_b64_tr_b16.
//   * An item's key range is clamped to the sequence's device length, so a
//     plan made for longer lengths reads no row past the sequence's pages.
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

constexpr int kThreads = 512;
constexpr int kTileTok = 16;                  // keys per stage
constexpr int kRoundTok = 2 * kTileTok;       // keys per round
constexpr int kRowBytes = 1152;               // one bf16 cache row
constexpr int kTileBytes = kTileTok * kRowBytes;
constexpr int kRoundBytes = 2 * kTileBytes;   // one round in the bf16 tile layout
constexpr int kF8RowBytes = 576;              // one e4m3 cache row
constexpr int kF8RoundBytes = kRoundTok * kF8RowBytes;   // one e4m3 round, 18 KB
constexpr int kSlots = 3;                     // rounds in the ring
constexpr int kExchWaveBytes = 64 * 16 * 4;   // a wave's 32 x 32 fp32 partial scores
constexpr float kRescaleMargin = 32.0f;       // log2 units above the reference max
constexpr float kLn2 = 0.69314718055994530942f;

// LDS map.  bf16: a ring of three rounds, computed in place.  e4m3: two pair
// buffers of one widened round each, a ring of three e4m3 rounds, the ring's
// per-key scales (256 bytes per round: the copy writes 64 lanes) and the pair
// buffers' scales.  Then the eight waves' exchange slots and round counters.
template <int KVD> struct Lds;
template <> struct Lds<0> {
  static constexpr int kExch = kSlots * kRoundBytes;
};
template <> struct Lds<1> {
  static constexpr int kPair = 0;
  static constexpr int kRing = 2 * kRoundBytes;
  static constexpr int kRingScale = kRing + kSlots * kF8RoundBytes;
  static constexpr int kPairScale = kRingScale + kSlots * 256;
  static constexpr int kExch = kPairScale + 2 * kRoundTok * 4;
};
template <int KVD> constexpr int kFlagOff = Lds<KVD>::kExch + 8 * kExchWaveBytes;
template <int KVD> constexpr int kSmemBytes = kFlagOff<KVD> + 8 * 4;
static_assert(kSmemBytes<0> <= 160 * 1024 && kSmemBytes<1> <= 160 * 1024,
              "LDS map exceeds a workgroup's LDS");

// A wave-uniform pointer, kept in SGPRs (the copies take a scalar base).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
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

// ---- bf16 caches
struct Ring {
  const uint8_t* kv;
  const int32_t* bt_row;
  uint32_t lds;        // LDS address of the ring
  int page_shift, k0, L, ntiles, wave, lane;
};

// One copy of a round: copy number ins (0..35) fills 1 KB block ins % 18 of
// the round's stage ins / 18: rows 8 (blk & 1) .. + 7, bytes 128 (blk >> 1)
// .. + 127 of each row, in the library's tile layout.
__device__ __forceinline__ void copy_block(int lane_id, int ins, const uint8_t* const (&base)[2],
                                           const int (&nvalid)[2], uint32_t lds) {
  const int lane = opaque(lane_id);
  const int c8a = 2 * (lane >> 4), lo = (lane >> 3) & 1;
  const int r8 = (lane & 7) ^ (4 * ((lane >> 4) & 1));
  const int t = ins >= 18 ? 1 : 0;
  const int blk = ins - 18 * t, rh = blk & 1, cg = blk >> 1;
  const int row = 8 * rh + r8;
  const int vo = (row < nvalid[t] ? row * kRowBytes : 0) + (c8a + (lo ^ rh)) * 16;
  lds_dma_x4(lds + t * kTileBytes + blk * 1024, vo, (t ? base[1] : base[0]) + 128 * cg);
}

// First key of stage t (0, 1) of round j: a stage past the item stands for
// the round's first key (a dummy copy of real cache rows).
__device__ __forceinline__ int stage_key(const Ring& r, int j, int t) {
  const int tile = 2 * j + t;
  return tile < r.ntiles ? r.k0 + kTileTok * tile : r.k0 + kRoundTok * j;
}

// The cache pages holding the two stages of round j (block-table reads,
// issued a round ahead of the copies that use them).
__device__ __forceinline__ void round_pages(const Ring& r, int j, int& pg0, int& pg1) {
  pg0 = r.bt_row[stage_key(r, j, 0) >> r.page_shift];
  pg1 = r.bt_row[stage_key(r, j, 1) >> r.page_shift];
}

// This wave's copies of round j, whose stages lie in pages pg0 and pg1, into
// ring slot j % 3: copy numbers wave, wave + 8, wave + 16, wave + 24 and, for
// waves 0..3, wave + 32.  Rows past the sequence read row 0 of their stage,
// so every byte that lands is a cached value and no cache slot past the
// sequence is read.
__device__ __forceinline__ void issue_round(const Ring& r, int j, int pg0, int pg1) {
  const int pmask = (1 << r.page_shift) - 1;
  const uint8_t* base[2];
  int nvalid[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kt = stage_key(r, j, t);
    const int row0 = ((t ? pg1 : pg0) << r.page_shift) + (kt & pmask);
    base[t] = uniform_ptr(r.kv + (int64_t)row0 * kRowBytes);
    nvalid[t] = 2 * j + t < r.ntiles ? min(kTileTok, r.L - kt) : 0;
  }
  const uint32_t lds = r.lds + (j % kSlots) * kRoundBytes;
  const int wave = opaque_s(r.wave);
#pragma unroll
  for (int k = 0; k < 4; ++k) copy_block(r.lane, wave + 8 * k, base, nvalid, lds);
  if (wave < 4) copy_block(r.lane, wave + 32, base, nvalid, lds);
}

// ---- e4m3 caches.  A round of 32 keys is one run of one page (pages hold a
// multiple of 64 rows and items start on a multiple of 64 keys), 18 KB
// contiguous in the cache; its 32 scales are contiguous too.
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

// This wave's copies of round j, which lies in page pg, into ring slot j % 3:
// copies wave, wave + 8 and, for waves 0 and 1, wave + 16 of the round's 18
// KB (copy ins = bytes 1024 ins .. + 1023, lane l taking 16 bytes at 16 l),
// and for wave 7 the round's scales (64 lanes of 4 bytes; lanes past the
// round's keys in the sequence copy its first scale).  A lane whose 16 bytes
// lie in a row past the sequence's end copies the round's first 16 bytes
// instead: every copy is issued, so the waits can count them, and no cache
// slot past the sequence is read.
__device__ __forceinline__ void issue_round_f8(const RingF8& r, int j, int pg) {
  const int kr = r.k0 + kRoundTok * j;          // first key of the round (< L)
  const int pmask = (1 << r.page_shift) - 1;
  const int row0 = (pg << r.page_shift) + (kr & pmask);
  const uint8_t* base = uniform_ptr(r.kv + (int64_t)row0 * kF8RowBytes);
  const uint32_t lds = r.ring + (j % kSlots) * kF8RoundBytes;
  const int nkeys = min(r.L - kr, kRoundTok);   // keys of the round in the sequence
  const int lane = opaque(r.lane);
  const int wave = opaque_s(r.wave);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int vo = 1024 * (wave + 8 * k) + 16 * lane;
    lds_dma_x4(lds + (wave + 8 * k) * 1024, vo < nkeys * kF8RowBytes ? vo : 0, base);
  }
  if (wave < 2) {
    const int vo = 1024 * (wave + 16) + 16 * lane;
    lds_dma_x4(lds + (wave + 16) * 1024, vo < nkeys * kF8RowBytes ? vo : 0, base);
  }
  if (wave == 7)
    lds_dma_x1(r.ring_scale + (j % kSlots) * 256, (lane < nkeys ? lane : 0) * 4,
               uniform_ptr(r.kv_scale + row0));
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

// Widen round p (keys kp .. kp + 31, ring slot p % 3) into pair buffer p % 2,
// in the bf16 tile layout the MFMA steps read, and its 32 scales into the
// buffer's scale slot.  The round's 36 output blocks of 1 KB (stage bi / 18,
// block bi % 18 = 2 cg + rh: rows 8 rh .. + 7, chunks 8 cg .. + 7) go to the
// waves by bi % 8.  Lane l takes chunk c8 = l % 8 of row r8 = c8 ^ (l / 8):
// each 16 lanes then read one 8-byte piece per bank pair (rows 576 bytes
// apart fall on alternate halves of the banks, and the two rows of a chunk
// have opposite parity), and each 8 lanes write distinct 16-byte bank groups
// of the tile layout.  Rows at or past the sequence's end become zeros.
__device__ __forceinline__ void widen_round_f8(char* smem, int p, int kp, int L, int wave_id,
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
  const uint32_t src = Lds<1>::kRing + (p % kSlots) * kF8RoundBytes + row * kF8RowBytes + 8 * c8;
  const uint32_t dst = Lds<1>::kPair + (p & 1) * kRoundBytes + 16 * slot;
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
  if (wave == 5 && lane < kRoundTok) {
    const float sc = *(const LDS_PTR(float))(smem + Lds<1>::kRingScale + (p % kSlots) * 256 +
                                             lane * 4);
    *(LDS_PTR(float))(smem + Lds<1>::kPairScale + ((p & 1) * kRoundTok + lane) * 4) = sc;
  }
}

// ---- one round: partial QK^T, exchange, softmax, PV
//
// Per-lane LDS read offsets, relative to the first stage of a round in the
// bf16 tile layout.  K fragment of QK step c of the full 576 dims (A operand,
// 32 keys x 16 dims): key l32 of the round (stage l32/16, row l32%16), dims
// 16c + 8hl .. + 7, at kb[c&1] + 2048 (c>>2) + 256 (c&3).  This half's i-th
// step is c = 4 (i>>1) + 2 hf + (i&1): kb[i&1] + 512 hf + 2048 (i>>1) + 256
// (i&1).  V^T fragment of PV step s (keys of stage s), column block cb:
// column 32 cb + l32 and, for hl = 0, keys 0..3 and 8..11 of the stage, for
// hl = 1 keys 4..7 and 12..15, at vb1 / vb2 + 2048 (cb>>1) + 512 (cb&1); this
// half's blocks are cb = 8 hf + 0..7 (8 KB further for hf = 1).  Exchange
// slots: [q4][lane] x 16 bytes.
struct Frag {
  int kb_e, kb_o, vb1, vb2, xown, xpar;
};

// Round of keys kp .. kp + 31, whose bf16 tiles start at LDS offset `so`
// (for e4m3, with the 32 per-key scales at sc_off).
template <int KVD>
__device__ __forceinline__ void round_step(char* smem, const Frag& fr, int so, int sc_off, int kp,
                                           int lim, int lim_all, float scale_log2, int lane,
                                           LDS_PTR(int) flag_own, const LDS_PTR(int) flag_par,
                                           int& seq, const bf16x8 (&qf)[18], f32x16 (&acc)[8],
                                           float& m, float& l) {
  constexpr int KW = 4;   // K fragments in flight in the QK step
  constexpr int VW = 4;   // V fragments in flight in the PV step
  const int hl = lane >> 5;
  const char* st = smem + so;

  // ---- partial S^T = K . Q^T over this half's 18 steps of 16 dims
  f32x16 S = f32x16{};
  {
    const int kbe = opaque(fr.kb_e), kbo = opaque(fr.kb_o);
    auto kload = [&](int i) -> bf16x8 {
      const int off = ((i & 1) ? kbo : kbe) + 2048 * (i >> 1) + 256 * (i & 1);
      return *(const LDS_PTR(bf16x8))(st + off);
    };
    bf16x8 kb[KW];
#pragma unroll
    for (int i = 0; i < KW - 1; ++i) kb[i] = kload(i);
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      if (i + KW - 1 < 18) kb[(i + KW - 1) % KW] = kload(i + KW - 1);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % KW], qf[i], S, 0, 0, 0);
    }
  }

  // ---- exchange the partial scores with the partner wave
  {
    const int xo = opaque(fr.xown + lane * 16);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = S[4 * q4 + e];
      *(LDS_PTR(f32x4))(smem + xo + q4 * 1024) = v;
    }
  }
  lds_publish(flag_own, ++seq);
  lds_wait_at_least(flag_par, seq);
  {
    const int xp = opaque(fr.xpar + lane * 16);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = *(const LDS_PTR(f32x4))(smem + xp + q4 * 1024);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[4 * q4 + e] += v[e];
    }
  }

  // ---- online softmax over keys kp + 8(r/4) + 4hl + r%4 (r = 0..15); for
  // e4m3 the keys' scales multiply the scores and the probabilities
  f32x4 sc[4];
  if constexpr (KVD == 1) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      sc[q4] = *(const LDS_PTR(f32x4))(smem + sc_off + (8 * q4 + 4 * hl) * 4);
  }
  float s[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if constexpr (KVD == 1) s[r] = S[r] * (scale_log2 * sc[r >> 2][r & 3]);
    else s[r] = S[r] * scale_log2;
  }
  if (kp + kRoundTok > lim_all) {
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
  // a row's first visible round fixes its reference max
  m = (m == -INFINITY) ? mx : m;
  if (__any(mx > m + kRescaleMargin)) {
    // raise the overshooting rows' reference to this round's max and rescale
    // their sums (a factor of at most 2^-32; 1 for other rows)
    const float alpha = mx > m + kRescaleMargin ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
    m = mx > m + kRescaleMargin ? mx : m;
    l *= alpha;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] *= alpha;
  }
  bf16x8 pf[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[r] - m);
    l += p;
    if constexpr (KVD == 1) pf[r >> 3][r & 7] = (__bf16)(p * sc[r >> 2][r & 3]);
    else pf[r >> 3][r & 7] = (__bf16)p;
  }

  // ---- O^T[256 x 32] += V^T . P^T: 2 key steps x this half's 8 column blocks
  {
    const int v1 = opaque(fr.vb1), v2 = opaque(fr.vb2);
    auto vload = [&](int n) -> bf16x8 {   // n = 8 * step + block of this half
      const char* sb = st + (n >> 3) * kTileBytes;
      const int off = 2048 * ((n & 7) >> 1) + 512 * (n & 1);
      const bf16x4 lo4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + v1 + off));
      const bf16x4 hi4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(sb + v2 + off));
      return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vf[VW];
#pragma unroll
    for (int n = 0; n < VW - 1; ++n) vf[n] = vload(n);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if (n + VW - 1 < 16) vf[(n + VW - 1) % VW] = vload(n + VW - 1);
      acc[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[n % VW], pf[n >> 3], acc[n & 7],
                                                           0, 0, 0);
    }
  }
}

template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel_split(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ q_lens, uint8_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes<KVD>];
  const uint32_t smem_base = lds_address(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int rg = wave >> 1, hf = wave & 1;   // row group of the pair, and this wave's half

  // Consecutive logical workgroups land on one XCD (dispatch is round-robin
  // over the 8 XCDs), so the CUs that share a sequence share an L2.
  const int bid = blockIdx.x;
  const int nwg = a.num_wg;
  const int g = (nwg % 8 == 0) ? (bid & 7) * (nwg >> 3) + (bid >> 3) : bid;

  if (tid < 8) *(volatile LDS_PTR(int))(smem + kFlagOff<KVD> + 4 * tid) = 0;
  barrier();

  const int32_t* wg_start = plan + plan[kWOffWgStart];
  const int32_t* items = plan + plan[kWOffItems];
  const int it_begin = wg_start[g], it_end = wg_start[g + 1];
  const int H = a.num_heads;

  Frag fr;
  {
    const int rl = l32 & 15, rh = rl >> 3, r8 = rl & 7, sp = l32 >> 4;
    fr.kb_e = sp * kTileBytes + rh * 1024 + (8 * (hl ^ rh) + r8) * 16 + 512 * hf;
    fr.kb_o = sp * kTileBytes + rh * 1024 + (8 * (hl ^ rh) + (r8 ^ 4)) * 16 + 512 * hf;
    const int i = lane & 15, G = (lane >> 4) & 1, u = (i >> 1) & 1, rr = 4 * hl + (i >> 2);
    fr.vb1 = (16 * G + 8 * u + (rr ^ (4 * G))) * 16 + 8 * (i & 1) + 8192 * hf;
    fr.vb2 = 1024 + (16 * G + 8 * (u ^ 1) + (rr ^ (4 * G))) * 16 + 8 * (i & 1) + 8192 * hf;
    fr.xown = Lds<KVD>::kExch + wave * kExchWaveBytes;
    fr.xpar = Lds<KVD>::kExch + (wave ^ 1) * kExchWaveBytes;
  }
  LDS_PTR(int) flag_own = (LDS_PTR(int))(smem + kFlagOff<KVD> + 4 * wave);
  const LDS_PTR(int) flag_par = (const LDS_PTR(int))(smem + kFlagOff<KVD> + 4 * (wave ^ 1));
  int seq = 0;   // rounds whose partial scores this wave has published

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
    const int nrounds = (ntiles + 1) >> 1;

    // This lane's query row: l32 of the pair's 32 (lanes l and l^32 share
    // it).  Its token and head are taken from an opaque copy of the lane id
    // here and again after the key loop, so that no per-lane value of them
    // holds a register through the loop.
    int lim;
    bf16x8 qf[18];
    {
      const int ln = opaque(lane);
      const int row = row_base + 32 * rg + (ln & 31);
      const bool valid = row < R;
      const int t = valid ? row / H : 0, h = valid ? row - t * H : 0;
      const int vis = a.causal ? L - qb + t + 1 : L;
      // rows past the sequence's last query row run over all keys (never
      // written), so that they never force the masked path
      lim = valid ? min(vis, k1) : k1;
      // ---- Q^T fragments (B operand) of this half's 18 steps: row l32,
      // dims 16c + 8hl .. + 7 of step c = 4 (i>>1) + 2 hf + (i&1)
      // (query row t H + h of sequence b, i.e. its row `row`; a wave-uniform
      // base for the sequence keeps the kernel argument in SGPRs)
      const uint8_t* qs = uniform_ptr(qg + (int64_t)b * a.max_q_len * H * (kDQK * 2));
      const int64_t qo = (int64_t)(valid ? row : 0) * (kDQK * 2) + (ln >> 5) * 16 + 64 * hf;
#pragma unroll
      for (int i = 0; i < 18; ++i)
        qf[i] = *reinterpret_cast<const bf16x8*>(qs + qo + 128 * (i >> 1) + 32 * (i & 1));
    }
    // the smallest lim of the pair's rows: visibility grows with the token,
    // so it is the first row's (all rows are past the end if it is)
    const int first = row_base + 32 * rg;
    const int lim_all = first < R ? min(a.causal ? L - qb + first / H + 1 : L, k1) : k1;

    f32x16 acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x16{};
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
      ring.wave = wave;
      ring.lane = lane;

      int pg0 = 0, pg1 = 0;   // pages of the next round to issue
      if (nrounds > 0) {
        round_pages(ring, 0, pg0, pg1);
        issue_round(ring, 0, pg0, pg1);
      }
      // Q must be resident before the key loop: otherwise the compiler, which
      // does not see the copies, keeps its loads pending into the loop and
      // waits for them there with vmcnt literals that, at run time, also
      // count the copies in flight.  (This waits for round 0 too, as the
      // loop's first wait would.)
#pragma unroll
      for (int i = 0; i < 18; ++i) require_vgpr(qf[i]);
      if (nrounds > 1) {
        round_pages(ring, 1, pg0, pg1);
        issue_round(ring, 1, pg0, pg1);
      }
      if (nrounds > 2) round_pages(ring, 2, pg0, pg1);

      // Round j opens by waiting for this wave's copies of round j (with
      // round j + 1 in flight: at least four copies per wave and round) and
      // the barrier; round j + 2, whose pages were read in the previous
      // round, is then issued into the slot of round j - 1.
      for (int j = 0; j < nrounds; ++j) {
        if (j + 1 < nrounds) MLA_VM_WAIT(4);
        else MLA_VM_WAIT(0);
        barrier();   // round j from all waves; round j - 1 and its exchange done
        if (j + 2 < nrounds) issue_round(ring, j + 2, pg0, pg1);
        round_step<0>(smem, fr, (j % kSlots) * kRoundBytes, 0, k0 + kRoundTok * j, lim, lim_all,
                      a.scale_log2, lane, flag_own, flag_par, seq, qf, acc, m, l);
        // the pages of round j + 3, read under the round's last MFMAs and
        // the barrier rather than between the barrier and the next QK step
        if (j + 3 < nrounds) round_pages(ring, j + 3, pg0, pg1);
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

      // Three stages per round: copy (three rounds ahead), widen into a pair
      // buffer, compute.  Iteration p widens round p + 1 and computes round
      // p between two barriers; round p + 3 is issued in iteration p into the
      // ring slot of round p, widened in iteration p - 1.  The wait that opens
      // iteration p is for round p + 1, with round p + 2 in flight: every
      // wave issues at least two copies per round, so vmcnt(2) suffices.
      int pg = 0;   // page of the next round to issue
      if (nrounds > 0) {
        issue_round_f8(ring, 0, round_page_f8(ring, 0));
        MLA_VM_WAIT(0);   // this wave's copies of round 0 (and its Q loads)
      }
      // Q resident before the key loop (see the bf16 path)
#pragma unroll
      for (int i = 0; i < 18; ++i) require_vgpr(qf[i]);
      if (nrounds > 1) issue_round_f8(ring, 1, round_page_f8(ring, 1));
      if (nrounds > 2) issue_round_f8(ring, 2, round_page_f8(ring, 2));
      if (nrounds > 3) pg = round_page_f8(ring, 3);
      if (nrounds > 0) {
        barrier();   // round 0 from all waves
        widen_round_f8(smem, 0, k0, L, wave, lane);
      }
      for (int p = 0; p < nrounds; ++p) {
        if (p + 2 < nrounds) MLA_VM_WAIT(2);
        else MLA_VM_WAIT(0);
        barrier();   // round p widened and round p + 1 copied by all waves; round p - 1 done
        if (p + 3 < nrounds) issue_round_f8(ring, p + 3, pg);
        if (p + 1 < nrounds) widen_round_f8(smem, p + 1, k0 + kRoundTok * (p + 1), L, wave, lane);
        round_step<1>(smem, fr, Lds<1>::kPair + (p & 1) * kRoundBytes,
                      Lds<1>::kPairScale + (p & 1) * kRoundTok * 4, k0 + kRoundTok * p, lim,
                      lim_all, a.scale_log2, lane, flag_own, flag_par, seq, qf, acc, m, l);
        if (p + 4 < nrounds) pg = round_page_f8(ring, p + 4);
      }
    }

    // ---- epilogue: lane owns row l32, columns 256 hf + 32 cb + 8(r/4) + 4hl
    // + r%4 (cb = 0..7).  Both waves of a pair hold the same row sums; the
    // first half writes the LSE.  The lane's column offset goes through an
    // opaque copy of the lane id, so that the compiler does not hoist the
    // output addresses out of the item loop.
    {
      const int ln = opaque(lane);
      const int hle = ln >> 5;
      const int row = row_base + 32 * rg + (ln & 31);
      const bool valid = row < R;
      const int t = valid ? row / H : 0, h = valid ? row - t * H : 0;
      const float lt = pair_sum(l);
      const bool empty = !(lt > 0.f);
      const float inv = empty ? 0.f : 1.f / lt;
      const float lse_v = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
      if (valid) {
        uint8_t* op;
        if (slot < 0) {
          op = o + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDLatent * 2);
          if (lse && hle == 0 && hf == 0) lse[(b * a.max_q_len + t) * H + h] = lse_v;
        } else {
          // bf16 partials, merged by mla_combine_kernel_bf16
          const int rb = slot_row + 32 * rg + (ln & 31);
          op = reinterpret_cast<uint8_t*>(part_o) +
               ((int64_t)slot * kRowsPerBlock + rb) * (kDLatent * 2);
          if (hle == 0 && hf == 0) part_lse[(int64_t)slot * kRowsPerBlock + rb] = lse_v;
        }
        op += (256 * hf + 4 * hle) * 2;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * inv);
            *reinterpret_cast<bf16x4*>(op + (32 * cb + 8 * q4) * 2) = v;
          }
        }
      }
    }
    // every wave leaves the ring and its exchange slot before the next
    // item's prologue refills them
    barrier();
  }
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (a.phases != 1) return hipErrorInvalidValue;
  if (kv_dtype == 0) {
    hipLaunchKernelGGL((mla_decode_kernel_split<0>), dim3(a.num_wg), dim3(kThreads), 0, stream, a,
                       a.plan, a.q, a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o,
                       a.lse, a.part_o, a.part_lse);
  } else {
    hipLaunchKernelGGL((mla_decode_kernel_split<1>), dim3(a.num_wg), dim3(kThreads), 0, stream, a,
                       a.plan, a.q, a.kv, a.kv_scale, a.block_table, a.kv_lens, a.q_lens, a.o,
                       a.lse, a.part_o, a.part_lse);
  }
  return hipGetLastError();
}

}  // namespace mla
