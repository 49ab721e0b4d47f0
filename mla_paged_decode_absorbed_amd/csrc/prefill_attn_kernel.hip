// SageAttention-style causal prefill attention (PaddlePaddle 3.0 inference
// page, long-sequence inference): INT8 Q K^T on the INT8 matrix cores, the
// INT32 scores dequantized in fp32, an online softmax, P quantized to e4m3
// and multiplied with the e4m3 V on the fp8 matrix cores, V's per-channel
// scale taken off each block's product.
//
// A workgroup takes 64 queries (half a 128-token query block) of one head;
// each of its 4 waves one 16-query tile.  Two workgroups share a CU, so
// their barrier-separated phases (staging, INT8 products, softmax, fp8
// products) overlap.  Key blocks of 128 (the same blocks that carry the
// scales of K and V) are staged in LDS in turn, up to the diagonal, the next
// block's codes already loading into registers while one is computed:
//
//  * scores: S^T[16 keys x 16 queries] = K Q^T on v_mfma_i32_16x16x64_i8,
//    3 steps over the 192 dims; Q's operands stay in registers.  In the
//    output, lane l holds keys 4 (l / 16) + r of query l % 16;
//  * s = S * q_scale * k_scale * softmax_scale (in log2 units; one key scale
//    per block), -inf for keys after the query or past the sequence; the row
//    max takes two lane swaps (the 4 lanes of a query), the running max, sum
//    and accumulator are rescaled by 2^(m_old - m_new);
//  * P = 2^(s - m) times 448 goes to e4m3 (hardware conversion, nearest
//    even): the 8 score tiles of a lane are exactly the 32 keys
//    16 a + 4 g + r the lane feeds to the PV instruction, so P never moves;
//  * O^T[16 channels x 16 queries] += V^T P^T on
//    v_mfma_scale_f32_16x16x128_f8f6f4, V^T read from LDS in the key order
//    mla_prefill_quantize wrote; V's power-of-two channel scales ride along
//    as the instruction's e8m0 scales of V^T's rows, so the product lands in
//    the accumulators already dequantized.
//
// The workgroups of the last (most expensive) query blocks start first, and
// consecutive workgroups are consecutive heads, so with H a multiple of 8
// every query block of a head runs on one XCD, whose L2 then holds that
// head's keys and values.  O = acc / (448 l), LSE = m ln 2 + ln l.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gfx950_asm.h"
#include "prefill.h"

namespace mla {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kKStride = 224;                 // LDS bytes per key row (192 + 32: fewer bank conflicts than + 16)
constexpr int kVStride = 144;                 // LDS bytes per channel row (128 + 16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2PScale = 8.807354922057604f;   // log2(448)
constexpr float kLnPScale = 6.104793232414985f;     // ln(448)
constexpr int kE8M0One = 127;                 // unit block scale of the fp8 instruction
constexpr int kWaves = 4;                     // waves per workgroup
constexpr int kTilesPerWave = 1;              // 16-query tiles per wave

// One key block: scores, online softmax, P V.  kMask: the block holds keys
// after some query (the diagonal block) or past the sequence's end.
template <int kU, bool kMask>
__device__ __forceinline__ void attend_block(const int8_t* ktile, const uint8_t* vtile,
                                             float kscale, const uint8_t* vexp,
                                             const i32x4 (&qop)[kU][3], const float (&qsc)[kU],
                                             const int (&qi)[kU], int key0, int n, int g, int col,
                                             float (&m)[kU], float (&lsum)[kU],
                                             f32x4 (&acc)[kU][8]) {
  // scores S^T: key 16 T + 4 g + r, query col, for every query tile
  i32x4 sacc[kU][8];
#pragma unroll
  for (int T = 0; T < 8; ++T) {
#pragma unroll
    for (int u = 0; u < kU; ++u) sacc[u][T] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int sg = 0; sg < 3; ++sg) {
      const i32x4 kop =
          *(const LDS_PTR(i32x4))(ktile + (16 * T + col) * kKStride + 64 * sg + 16 * g);
#pragma unroll
      for (int u = 0; u < kU; ++u)
        sacc[u][T] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, qop[u][sg], sacc[u][T], 0, 0, 0);
    }
  }
  // t = S; with the block's key scale times q_scale * softmax_scale * log2(e)
  // = c > 0 the log2-domain score is t * c, so the row max is c * max t
  float t[kU][8][4];
  float mx[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) mx[u] = -INFINITY;
#pragma unroll
  for (int T = 0; T < 8; ++T) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = float(sacc[u][T][r]);
        if (kMask) {
          const int key = key0 + 16 * T + 4 * g + r;
          if (!(key <= qi[u] && key < n)) v = -INFINITY;
        }
        t[u][T][r] = v;
        mx[u] = fmaxf(mx[u], v);
      }
  }
  float alpha[kU];
  i32x8 pop[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const float c = qsc[u] * kscale;
    float mt = fmaxf(mx[u], __shfl_xor(mx[u], 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(m[u], mt * c);
    const bool none = mnew == -INFINITY;          // nothing visible yet (padding queries)
    alpha[u] = none ? 1.f : __builtin_amdgcn_exp2f(m[u] - mnew);
    // 448 P = 2^(t qsc - (m - log2 448)), straight into e4m3.  mnew rounds
    // t qsc once more than the fused exponent below does, so the subtracted
    // max is raised by a bound on that rounding (|m| 2^-20 + 2^-16, under
    // 1e-5 of P): 448 P then stays below 448, the largest e4m3 value
    const float mb = none ? 0.f : mnew - kLog2PScale + (fabsf(mnew) * 0x1p-20f + 0x1p-16f);
    float ps = 0.f;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(t[u][T][r], c, -mb));
        if (kMask && t[u][T][r] == -INFINITY) p[r] = 0.f;
        ps += p[r];
      }
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
      pop[u][T] = w;
    }
    lsum[u] = lsum[u] * alpha[u] + ps;
    m[u] = mnew;
  }
  // once no query's max moves (the usual case after the first blocks) the
  // wave skips the rescale of its accumulators
  bool moved = false;
#pragma unroll
  for (int u = 0; u < kU; ++u) moved = moved || alpha[u] != 1.f;
  if (__any(moved)) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[u][ct] *= alpha[u];
  }
  // O^T += V^T P^T per 16-channel tile, straight into the accumulators: the
  // lanes of channel row col hand the instruction that channel's e8m0 scale
  // (its power-of-two exponent + 127), which it applies to the row of V^T
  const LDS_PTR(uint32_t) vx = (const LDS_PTR(uint32_t))(vexp + 8 * col);
  const uint32_t ex[2] = {vx[0], vx[1]};
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const LDS_PTR(i32x4) vr = (const LDS_PTR(i32x4))(vtile + (16 * ct + col) * kVStride + 32 * g);
    const i32x4 v0 = vr[0], v1 = vr[1];
    const i32x8 vop = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    const int sa = int((ex[ct >> 2] >> (8 * (ct & 3))) & 0xFFu);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      acc[u][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, pop[u], acc[u][ct], 0, 0,
                                                                    0, sa, 0, kE8M0One);
  }
}

// K codes, V codes and the scales of one key block, loaded to registers by
// the kThreads threads so the loads of the next block are in flight while
// this one is computed.
template <int kThreads>
struct BlockRegs {
  static constexpr int kK = kPfBlock * 12 / kThreads;      // 16-byte K chunks per thread
  static constexpr int kV = kPfDV * 8 / kThreads;          // 16-byte V chunks per thread
  static_assert(kK * kThreads == kPfBlock * 12 && kV * kThreads == kPfDV * 8, "chunking");
  i32x4 k[kK], v[kV];
  float ks;        // the block's key scale
  uint32_t vx;     // channel threadIdx.x's V scale as an e8m0 byte (first 128 threads)
};

template <int kThreads>
__device__ __forceinline__ void load_block(const PrefillAttnArgs& a, const PfBlock& blk, int kb,
                                           int h, BlockRegs<kThreads>& r) {
  const int H = a.num_heads;
  const int key0 = kb * kPfBlock;
  const int nk = min(kPfBlock, blk.n - key0);
#pragma unroll
  for (int j = 0; j < BlockRegs<kThreads>::kK; ++j) {
    const int c = int(threadIdx.x) + kThreads * j;
    const int key = c / 12, part = c - key * 12;
    r.k[j] = i32x4{0, 0, 0, 0};
    if (key < nk)
      r.k[j] = reinterpret_cast<const i32x4*>(a.kc + (int64_t(blk.t0 + key0 + key) * H + h) *
                                                         kPfDQK)[part];
  }
  const i32x4* vsrc =
      reinterpret_cast<const i32x4*>(a.vc + (int64_t(blk.b0 + kb) * H + h) * (kPfDV * kPfBlock));
#pragma unroll
  for (int j = 0; j < BlockRegs<kThreads>::kV; ++j) r.v[j] = vsrc[int(threadIdx.x) + kThreads * j];
  r.ks = a.ks[int64_t(blk.b0 + kb) * H + h];
  r.vx = 0u;
  if (threadIdx.x < kPfDV)   // the e8m0 byte of a power of two 2^e is its fp32 exponent field
    r.vx = (__float_as_uint(a.vs[(int64_t(blk.b0 + kb) * H + h) * kPfDV + threadIdx.x]) >> 23) &
           0xFFu;
}

template <int kThreads>
__device__ __forceinline__ void store_block(const BlockRegs<kThreads>& r, int8_t* ktile,
                                            uint8_t* vtile, uint8_t* vexp) {
#pragma unroll
  for (int j = 0; j < BlockRegs<kThreads>::kK; ++j) {
    const int c = int(threadIdx.x) + kThreads * j;
    const int key = c / 12, part = c - key * 12;
    *(LDS_PTR(i32x4))(ktile + key * kKStride + 16 * part) = r.k[j];
  }
#pragma unroll
  for (int j = 0; j < BlockRegs<kThreads>::kV; ++j) {
    const int c = int(threadIdx.x) + kThreads * j;
    *(LDS_PTR(i32x4))(vtile + (c >> 3) * kVStride + 16 * (c & 7)) = r.v[j];
  }
  // channel c = 16 ct + col goes to byte 8 col + ct: a lane reads its 8 in one
  if (threadIdx.x < kPfDV)
    *(LDS_PTR(uint8_t))(vexp + 8 * (threadIdx.x & 15) + (threadIdx.x >> 4)) = uint8_t(r.vx);
}

// kW waves of kU 16-query tiles each: a workgroup covers kQ = 16 kW kU
// queries, kSplit workgroups one 128-query block.
// At most 256 VGPRs: two waves per SIMD, so two workgroups share a CU and
// their load / MFMA / softmax phases overlap instead of running in lockstep.
template <int kW, int kU>
__global__ __launch_bounds__(kW * 64, 2) void mla_prefill_attn_kernel(const PrefillAttnArgs a) {
  constexpr int kQ = 16 * kW * kU;
  constexpr int kSplit = kPfBlock / kQ;
  static_assert(kSplit * kQ == kPfBlock, "workgroups tile a query block");
  constexpr int kThreads = kW * 64;
  __shared__ __attribute__((aligned(16))) int8_t ktile[kPfBlock * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kPfDV * kVStride];
  __shared__ __attribute__((aligned(16))) uint8_t vexp[kPfDV];
  const int H = a.num_heads;
  const int rest = int(blockIdx.x) / H;
  const int h = int(blockIdx.x) - rest * H;
  const int wi = rest / kSplit, part = rest - wi * kSplit;
  const int i = a.num_blocks - 1 - wi;          // the last blocks carry the most keys
  PfBlock blk;
  if (!pf_find_block(a.cu, a.num_seqs, a.num_tokens, a.num_blocks, i, &blk)) return;
  const int qb = blk.kb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;

  BlockRegs<kThreads> regs;
  load_block<kThreads>(a, blk, 0, h, regs);

  // this lane's queries (one per 16-query tile) and their Q operands
  int qi[kU];
  float qsc[kU];
  i32x4 qop[kU][3];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    qi[u] = qb * kPfBlock + part * kQ + wave * 16 * kU + u * 16 + col;
    qsc[u] = 0.f;
#pragma unroll
    for (int sg = 0; sg < 3; ++sg) qop[u][sg] = i32x4{0, 0, 0, 0};
    if (qi[u] < blk.n) {
      const int64_t row = int64_t(blk.t0 + qi[u]) * H + h;
      const i32x4* src = reinterpret_cast<const i32x4*>(a.qc + row * kPfDQK);
#pragma unroll
      for (int sg = 0; sg < 3; ++sg) qop[u][sg] = src[4 * sg + g];
      qsc[u] = a.qs[row] * a.sm_scale * kLog2e;
    }
  }

  float m[kU], lsum[kU];
  f32x4 acc[kU][8];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    m[u] = -INFINITY;
    lsum[u] = 0.f;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb = 0; kb <= qb; ++kb) {
    __syncthreads();                              // the previous block's reads are done
    store_block<kThreads>(regs, ktile, vtile, vexp);
    const float kscale = regs.ks;
    __syncthreads();
    if (kb < qb) load_block<kThreads>(a, blk, kb + 1, h, regs);
    // blocks below the diagonal are whole and wholly visible
    if (kb < qb)
      attend_block<kU, false>(ktile, vtile, kscale, vexp, qop, qsc, qi, kb * kPfBlock, blk.n, g,
                              col, m, lsum, acc);
    else
      attend_block<kU, true>(ktile, vtile, kscale, vexp, qop, qsc, qi, kb * kPfBlock, blk.n, g,
                             col, m, lsum, acc);
  }

#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float l = lsum[u];                            // 448 times the softmax sum
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qi[u] >= blk.n) continue;
    const int64_t row = int64_t(blk.t0 + qi[u]) * H + h;
    const float inv = 1.f / l;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f32x4 o = acc[u][ct] * inv;
      const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      *reinterpret_cast<bf16x4*>(a.o + row * (kPfDV * 2) + (16 * ct + 4 * g) * 2) = ob;
    }
    if (g == 0) a.lse[row] = m[u] * kLn2 + logf(l) - kLnPScale;
  }
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t stream) {
  const int64_t wgs = int64_t(a.num_blocks) * a.num_heads * (kPfBlock / (16 * kWaves * kTilesPerWave));
  if (wgs <= 0) return hipSuccess;
  if (wgs > int64_t(0x7FFFFFFF)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mla_prefill_attn_kernel<kWaves, kTilesPerWave>), dim3(unsigned(wgs)),
                     dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
