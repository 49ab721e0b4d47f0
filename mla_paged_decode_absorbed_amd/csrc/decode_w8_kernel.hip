// Weight-absorbed MLA decode over a paged latent cache, two waves per SIMD:
// a candidate successor of mla_decode_kernel_pairs for bf16 caches and
// one-phase plans.  It computes what the library's decode kernels compute
// (same plan, same work items, same outputs and partials):
//   s_j = scale * <q, c_j> over the visible cached rows, O = softmax(s) .
//   latent, LSE (KsanaLLM 0.6.0 page, weight-absorbed MLA for decode;
//   PaddlePaddle 3.0 inference page, draft tokens verified in one pass;
//   FlashAttention-3 in DeepSeek-R1 page, chapter 2: LSE and split-K).
//
// Why: with one wave per SIMD, mla_decode_kernel_pairs serialises each
// wave's chain QK^T -> softmax -> PV, and the matrix unit sits idle during
// the softmax and the LDS waits.  Here the 128 rows of a work item are spread
// over eight waves of 16 rows, two per SIMD, so one wave's softmax and waits
// can run under the other wave's MFMAs.  A wave then has 256 registers:
// Q (16 rows x 576) takes 72, the output accumulator (16 rows x 512 fp32)
// 128.  Every wave reads every key tile from LDS (twice the LDS reads per key
// of the four-wave kernel; the layout keeps them free of bank conflicts).
//
// Mapping onto CDNA4:
//   * 512 threads (eight wave64s), one workgroup per CU, persistent over its
//     plan items; wave w owns rows 16w .. 16w + 15 of an item.
//   * Key tiles of 16 tokens stream HBM -> LDS through the same 8-stage ring
//     and tile layout as the library kernels, in rounds of four tiles: tile t
//     of a round is copied by waves t and t + 4, nine 1 KB copies each.
//   * Keys are processed 32 at a time (two ring stages).  QK^T: S^T[16 keys x
//     16 rows] = K . Q^T on v_mfma_f32_16x16x32_bf16 for each stage, 18 steps
//     of 32 dimensions sharing the Q fragment; a lane holds keys 4(lane/16) +
//     r of its row in each stage.
//   * PV: O^T[16 columns x 16 rows] += V^T . P^T on v_mfma_f32_16x16x32_bf16
//     for 32 column blocks.  The contraction takes a lane's own 8 keys (four
//     of each stage) in the order it holds them, so the probabilities are the
//     B operand with no lane exchange; V^T is read by ds_read_b64_tr_b16, four
//     keys of one stage per read.
//   * The softmax keeps the library kernels' fixed reference max and their
//     restart when a score overshoots it by more than 32 (log2 units).  The
//     waves agree on a restart through per-wave flags kept by round parity:
//     a wave publishes whether round j overshot before the barrier that
//     opens round j + 1, and every wave reads all flags of round j after that
//     barrier.  The next write to those flags (round j + 2) happens after the
//     barrier that opens round j + 2, which every reader has reached, so all
//     waves see the same flags and leave the round loop at the same barrier.
//     (A single flag, set while a slower wave may not yet have read it after
//     the same barrier, lets waves leave at different barriers.)
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
constexpr int kStages = 8;                    // two rounds in the ring
constexpr int kFlagOff = kStages * kTileBytes;   // overshoot flags [2][8] (round parity, wave)
constexpr int kSmemBytes = kFlagOff + 2 * 8 * 4;
constexpr float kRestartMargin = 32.0f;       // log2 units above the reference max
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

// Whether any of the 8 waves published an overshoot in the flags of one
// round parity (two 16-byte LDS reads).
__device__ __forceinline__ bool any_flag(volatile LDS_PTR(int) flags, int parity) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 a = *(const LDS_PTR(i32x4))((LDS_PTR(int))flags + parity * 8);
  const i32x4 b = *(const LDS_PTR(i32x4))((LDS_PTR(int))flags + parity * 8 + 4);
  const i32x4 o = a | b;
  return (o.x | o.y | o.z | o.w) != 0;
}

struct Ring {
  const uint8_t* kv;
  const int32_t* bt_row;
  uint32_t lds;        // LDS address of the ring
  int page_shift, k0, L, ntiles, lane;
};

// This wave's share of round j: half HALF (copies 9*HALF .. 9*HALF + 8) of
// tile `t` of the round, into its ring stage.  A tile past the item is a
// harmless dummy copy of the round's first key (every wave issues exactly
// nine copies per round, so each wave's vmcnt count is the same).  Copy ins
// fills the stage's 1 KB block ins: rows 8(ins&1) .. +7, bytes 128(ins>>1) ..
// +127 of each row, in the library's tile layout.
template <int HALF>
__device__ __forceinline__ void issue_half(const Ring& r, int t, int j) {
  const int tile = kRoundTiles * j + t;
  const int stage = tile % kStages;
  const int kr = r.k0 + kRoundTok * j;          // first key of the round (< L)
  const bool real = tile < r.ntiles;
  const int kt = real ? r.k0 + kTileTok * tile : kr;
  const int pmask = (1 << r.page_shift) - 1;
  const int row0 = (r.bt_row[kt >> r.page_shift] << r.page_shift) + (kt & pmask);
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

__device__ __forceinline__ void issue_round(const Ring& r, int t, int half, int j) {
  if (half) issue_half<1>(r, t, j);
  else issue_half<0>(r, t, j);
}

template <int KVD>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel_w8(
    const DecodeArgs a, const int32_t* __restrict__ plan, const uint8_t* __restrict__ qg,
    const uint8_t* __restrict__ kvg, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ q_lens,
    uint8_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  static_assert(KVD == 0, "bf16 caches only");
  constexpr int KW = 2;   // QK steps whose K fragments are in flight
  constexpr int VW = 3;   // PV column blocks whose V fragments are in flight
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
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
  const int kh = g4 >> 1, krh = l16 >> 3, kr8 = l16 & 7;
  const int kbase = krh * 1024 + (16 * kh + 8 * ((g4 & 1) ^ krh) + (kr8 ^ (4 * kh))) * 16;
  // V^T fragment of PV column block m (A operand, 16 columns x 4 keys of a
  // stage): the lane names row 4g4 + l16/4, columns 16m + 4(l16%4) .. +3 and
  // receives column 16m + l16, rows 4g4 .. 4g4 + 3; at vb[m&1] + 2048(m>>2) +
  // 256(m&3).
  const int vr = 4 * g4 + (l16 >> 2), vrh = vr >> 3, vr8 = vr & 7, vx = (l16 & 3) >> 1;
  const int vb_e = vrh * 1024 + 16 * (8 * (vx ^ vrh) + vr8) + 8 * (l16 & 1);
  const int vb_o = vrh * 1024 + 16 * (8 * (vx ^ vrh) + (vr8 ^ 4)) + 8 * (l16 & 1);
  volatile LDS_PTR(int) flags = (volatile LDS_PTR(int))(smem + kFlagOff);   // [parity][wave]

  for (int it = it_begin; it < it_end; ++it) {
    const int32_t* item = items + it * kItemWords;
    const int b = item[0], row_base = item[1], k0 = item[2], k1 = item[3], slot = item[4];
    const int slot_row = item[5];
    const int L = kv_lens[b];
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
    int lim_all = lim;
    lim_all = min(lim_all, __shfl_xor(lim_all, 1));
    lim_all = min(lim_all, __shfl_xor(lim_all, 2));
    lim_all = min(lim_all, __shfl_xor(lim_all, 4));
    lim_all = min(lim_all, __shfl_xor(lim_all, 8));
    lim_all = __builtin_amdgcn_readfirstlane(lim_all);

    // ---- Q^T fragments (B operand): row, dims 32c + 8g4 .. +7
    bf16x8 qf[18];
    {
      const uint8_t* qp = qg + ((int64_t)((b * a.max_q_len + t) * H + h)) * (kDQK * 2) + g4 * 16;
#pragma unroll
      for (int c = 0; c < 18; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 64);
    }

    Ring ring;
    ring.kv = kvg;
    ring.bt_row = block_table + (int64_t)b * a.max_pages;
    ring.lds = smem_base;
    ring.page_shift = a.page_shift;
    ring.k0 = k0;
    ring.L = L;
    ring.ntiles = ntiles;
    ring.lane = lane;

    f32x4 acc[32];
    float m = -INFINITY, l = 0.f;
    for (;;) {   // runs once unless a score overshoots the reference max
      if (nrounds > 0) issue_round(ring, tq, half, 0);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) acc[cb] = f32x4{};
      l = 0.f;
      bool again = false;       // workgroup-uniform: some wave overshot
      bool overshoot = false;   // wave-uniform: this wave overshot in the last round

      // Round j opens by publishing round j-1's overshoot, waiting for this
      // wave's copies and the barrier, and stopping the pass if any wave
      // overshot in round j-1; after the last round the same is done once more.
      for (int j = 0; j < nrounds; ++j) {
        if (j > 0 && lane == 0) flags[((j - 1) & 1) * 8 + wave] = overshoot ? 1 : 0;
        MLA_VM_WAIT(0);
        barrier();   // tiles of round j come from all waves
        if (j > 0 && any_flag(flags, (j - 1) & 1)) {
          again = true;
          break;
        }
        if (j + 1 < nrounds) issue_round(ring, tq, half, j + 1);
        overshoot = false;

#pragma unroll
        for (int pp = 0; pp < kRoundTiles / 2; ++pp) {
          const int tile = kRoundTiles * j + 2 * pp;   // first stage of the pair
          if (tile >= ntiles) break;
          const int kp = k0 + kTileTok * tile;          // first key of the pair
          // this pair's per-lane LDS bases: one add each per pair, through
          // opaque copies so that the compiler keeps three registers here
          // rather than precomputing a base per ring stage for the whole loop
          const int so = (tile % kStages) * kTileBytes;
          const int kb_s = opaque(kbase + so);
          const int ve_s = opaque(vb_e + so), vo_s = opaque(vb_o + so);

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
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[r] = SA[r] * a.scale_log2;
            s[4 + r] = SB[r] * a.scale_log2;
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
          if (__any(mx > m + kRestartMargin)) {
            m = fmaxf(m, mx);
            overshoot = true;
            break;
          }
          bf16x8 pf;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float p = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[r] - m);
            l += p;
            pf[r] = (__bf16)p;
          }

          // ---- O^T[512 x 16] += V^T . P^T: 32 column blocks of 16
          {
            auto vload = [&](int cm) -> bf16x8 {
              const int off = ((cm & 1) ? vo_s : ve_s) + 2048 * (cm >> 2) + 256 * (cm & 3);
              const bf16x4 v0 =
                  __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_PTR(bf16x4))(smem + off));
              const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (LDS_PTR(bf16x4))(smem + kTileBytes + off));
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
      }
      if (!again && nrounds > 0) {   // the loop ran out: check its last round
        if (lane == 0) flags[((nrounds - 1) & 1) * 8 + wave] = overshoot ? 1 : 0;
        MLA_VM_WAIT(0);
        barrier();
        again = any_flag(flags, (nrounds - 1) & 1);
      }
      // Every wave left at the same barrier with the same `again`; no copy is
      // in flight (the last wait drained them) and no wave reads the ring
      // after that barrier, so a new pass may refill it.
      if (!again) break;
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
          const int rb = slot_row + 16 * wave + l16;
          float* pp = part_o + ((int64_t)slot * kRowsPerBlock + rb) * kDLatent;
#pragma unroll
          for (int cm = 0; cm < 32; ++cm) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[cm][e] * inv;
            *reinterpret_cast<f32x4*>(pp + 16 * cm + 4 * ge) = v;
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

hipError_t launch_decode_w8(const DecodeArgs& a, hipStream_t stream) {
  if (a.phases != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mla_decode_kernel_w8<0>), dim3(a.num_wg), dim3(kThreads), 0, stream, a,
                     a.plan, a.q, a.kv, a.block_table, a.kv_lens, a.q_lens, a.o, a.lse, a.part_o,
                     a.part_lse);
  return hipGetLastError();
}

}  // namespace mla
