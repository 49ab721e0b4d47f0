// Device-side planner: builds, from device-resident lengths, the same plan
// image as the host planner for a fixed launch shape (mla_decode_plan_fixed),
// so a decode step whose lengths were produced on the GPU (accepted draft
// tokens, for instance) needs no copy of them to the host.
//
// One workgroup of one wave.  All lanes stage the lengths in LDS and check
// them.  The whole wave then runs the planner's loops (plan_core.h, the code
// the host planner runs) in step: their sequential reads come from arrays
// cached 64 elements at a time in the lanes' registers and read out with
// readlane, so the loops run on the scalar unit with one LDS access per 64
// elements; lane 0 stores the results to LDS.  With one workgroup per
// processor (the default) all lanes then write the plan image at once;
// otherwise lane 0 writes it with the host's writer.  Lengths that the host
// planner would reject yield an empty plan (no items: the decode writes
// nothing) and MLA_ERR_BAD_SHAPE in *status.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode.h"
#include "plan_core.h"
#include "plan_device.h"

namespace mla {
namespace {

__host__ __device__ inline int64_t align16(int64_t x) { return (x + 15) / 16 * 16; }

struct PlanLds {
  int64_t kvl, ql, units, pieces, ufp, slot, comb, total;
};

__host__ __device__ inline PlanLds plan_lds_layout(int64_t B, int64_t MU, int64_t P) {
  PlanLds l;
  l.kvl = 0;
  l.ql = l.kvl + align16(4 * B);
  l.units = l.ql + align16(4 * B);
  l.pieces = l.units + align16(int64_t(sizeof(PlanUnit)) * MU);
  l.ufp = l.pieces + align16(int64_t(sizeof(PlanPiece)) * (MU + P + 1));
  l.slot = l.ufp + align16(4 * (MU + 1));
  l.comb = l.slot + align16(4 * (MU + P + 1));
  l.total = l.comb + align16(4 * kCombineWords * MU);
  return l;
}

__device__ inline int32_t lane_value(int32_t v, int32_t l) {
  return __builtin_amdgcn_readlane(v, l);
}

// Sequential reads of an LDS array by the whole wave: lane l holds element
// base + l of the current 64-element chunk, and element i is read from lane
// i % 64 into a scalar register, so a run of reads costs one LDS access per
// 64 elements.  i is uniform over the wave.
struct IntCache {
  const int32_t* a;
  int32_t n, lane, base, mine;
  __device__ IntCache(const int32_t* a_, int32_t n_, int32_t lane_)
      : a(a_), n(n_), lane(lane_), base(-64), mine(0) {}
  __device__ int32_t operator()(int32_t i) {
    if ((i & ~63) != base) {
      base = i & ~63;
      mine = base + lane < n ? a[base + lane] : 0;
    }
    return lane_value(mine, i & 63);
  }
};

struct UnitCache {
  const PlanUnit* a;
  int32_t n, lane, base;
  PlanUnit mine;
  __device__ UnitCache(const PlanUnit* a_, int32_t n_, int32_t lane_)
      : a(a_), n(n_), lane(lane_), base(-64), mine{0, 0, 0, 0, 0} {}
  __device__ PlanUnit operator()(int32_t i) {
    if ((i & ~63) != base) {
      base = i & ~63;
      mine = base + lane < n ? a[base + lane] : PlanUnit{0, 0, 0, 0, 0};
    }
    const int32_t l = i & 63;
    return {lane_value(mine.b, l), lane_value(mine.row0, l), lane_value(mine.rows, l),
            lane_value(mine.L, l), lane_value(mine.rounds, l)};
  }
};

// The plan image with one workgroup per processor (phases 1), written by all
// lanes at once: item i is piece i, and workgroup g's items start at the
// number of pieces on processors below g.  Same words as plan_write_image.
__device__ void write_image_one_phase(const PlanUnit* units, const PlanPiece* pieces,
                                      int32_t n_pieces, const int32_t* slot, const int32_t* comb,
                                      int32_t n_comb, int32_t n_partials, int32_t G_out,
                                      int32_t* out, int32_t lane) {
  const int64_t off_wg = kHeaderWords;
  const int64_t off_items = off_wg + plan_round_up8(G_out + 1);
  const int64_t off_comb = off_items + int64_t(n_pieces) * kItemWords;
  if (lane < kHeaderWords) {
    int32_t v = 0;
    switch (lane) {
      case kWMagic: v = kPlanMagic; break;
      case kWVersion: v = kPlanVersion; break;
      case kWNumWg: v = G_out; break;
      case kWNumItems: v = n_pieces; break;
      case kWNumCombine: v = n_comb; break;
      case kWNumPartials: v = n_partials; break;
      case kWTile: v = kTileTokens; break;
      case kWRowsPerBlock: v = kRowsPerBlock; break;
      case kWOffWgStart: v = int32_t(off_wg); break;
      case kWOffItems: v = int32_t(off_items); break;
      case kWOffCombine: v = int32_t(off_comb); break;
      case kWPhases: v = 1; break;
      default: break;
    }
    out[lane] = v;
  }
  for (int64_t g = lane; g < off_items - off_wg; g += 64) {
    int32_t v = 0;
    if (g <= G_out) {   // pieces on processors below g (pieces are in processor order)
      int32_t lo = 0, hi = n_pieces;
      while (lo < hi) {
        const int32_t mid = (lo + hi) / 2;
        if (pieces[mid].proc < g) lo = mid + 1; else hi = mid;
      }
      v = lo;
    }
    out[off_wg + g] = v;
  }
  for (int32_t i = lane; i < n_pieces; i += 64) {
    const PlanPiece pc = pieces[i];
    const PlanUnit u = units[pc.unit];
    int32_t* it = out + off_items + int64_t(i) * kItemWords;
    it[0] = u.b;
    it[1] = u.row0;
    it[2] = pc.k0;
    it[3] = pc.k1;
    it[4] = slot[i];
    it[5] = 0;
    it[6] = 0;
    it[7] = 0;
  }
  for (int32_t w = lane; w < n_comb * kCombineWords; w += 64) out[off_comb + w] = comb[w];
}

__global__ __launch_bounds__(64) void mla_plan_kernel(const PlanDeviceArgs a, int64_t max_units) {
  __shared__ __attribute__((aligned(16))) char lds[kPlanLdsBytes];
  __shared__ int bad;
  const PlanLds l = plan_lds_layout(a.batch, max_units, a.P);
  int32_t* kvl = reinterpret_cast<int32_t*>(lds + l.kvl);
  int32_t* ql = reinterpret_cast<int32_t*>(lds + l.ql);
  const int lane = threadIdx.x;
  if (lane == 0) bad = 0;
  __syncthreads();
  for (int b = lane; b < a.batch; b += 64) {
    const int32_t L = a.kv_lens[b];
    const int32_t q = a.q_lens ? a.q_lens[b] : a.max_q_len;
    kvl[b] = L;
    ql[b] = q;
    // the host planner's length checks
    if (L < 0 || q < 0 || q > a.max_q_len || L > a.cap || (a.causal && q > 0 && L < q)) bad = 1;
  }
  __syncthreads();

  PlanUnit* units = reinterpret_cast<PlanUnit*>(lds + l.units);
  PlanPiece* pieces = reinterpret_cast<PlanPiece*>(lds + l.pieces);
  int32_t* ufp = reinterpret_cast<int32_t*>(lds + l.ufp);
  int32_t* slot = reinterpret_cast<int32_t*>(lds + l.slot);
  int32_t* comb = reinterpret_cast<int32_t*>(lds + l.comb);
  int32_t n_units = 0, n_pieces = 0, C = 0, n_partials = 0;
  const bool lengths_bad = plan_uniform(bad) != 0;
  if (!lengths_bad) {
    // every lane computes the same sequence of units; lane 0 stores them
    IntCache kv_at(kvl, a.batch, lane), q_at(ql, a.batch, lane);
    for (int32_t b = 0; b < a.batch; ++b)
      n_units += plan_units_of(b, q_at(b), kv_at(b), a.num_heads,
                               lane == 0 ? units + n_units : nullptr);
    __syncthreads();
    auto put_piece = [&](int32_t i, const PlanPiece& pc) {
      if (lane == 0) pieces[i] = pc;
    };
    auto put_first = [&](int32_t u, int32_t i) {
      if (lane == 0) ufp[u] = i;
      if (u == n_units) n_pieces = i;
    };
    const int64_t total = plan_total(UnitCache(units, n_units, lane), n_units, a.item_cost);
    // budgets stay below total + per-piece costs: 32-bit scalar arithmetic when
    // that fits (budgets, processors and rounds of any real shape), else 64-bit
    if (total + int64_t(a.P) * (a.item_cost + kMinPieceRounds + 1) < (int64_t(1) << 30)) {
      const int32_t per_proc = plan_per_proc<int32_t>(UnitCache(units, n_units, lane), n_units,
                                                      total, a.item_cost, a.P);
      plan_fill<int32_t>(UnitCache(units, n_units, lane), n_units, per_proc, a.item_cost, a.P,
                         true, put_piece, put_first);
    } else {
      const int64_t per_proc = plan_per_proc<int64_t>(UnitCache(units, n_units, lane), n_units,
                                                      total, a.item_cost, int64_t(a.P));
      plan_fill<int64_t>(UnitCache(units, n_units, lane), n_units, per_proc, a.item_cost,
                         int64_t(a.P), true, put_piece, put_first);
    }
    __syncthreads();
    plan_slots(
        UnitCache(units, n_units, lane), IntCache(ufp, n_units + 1, lane), n_units,
        [&](int32_t p, int32_t v) {
          if (lane == 0) slot[p] = v;
        },
        [&](int32_t e, int32_t b, int32_t row0, int32_t first, int32_t n) {
          if (lane == 0) {
            int32_t* c = comb + int64_t(e) * kCombineWords;
            c[0] = b;
            c[1] = row0;
            c[2] = first;
            c[3] = n;
          }
        },
        &C, &n_partials);
    __syncthreads();
  }
  // an empty plan when the lengths are bad (no pieces: every workgroup idle)
  int64_t words = 0;
  if (a.PH == 1) {
    const int64_t need = kHeaderWords + plan_round_up8(a.P + 1) +
                         int64_t(n_pieces) * kItemWords + int64_t(C) * kCombineWords;
    words = need <= a.plan_words ? need : -1;
    if (words > 0)
      write_image_one_phase(units, pieces, n_pieces, slot, comb, C, n_partials, a.P, a.plan,
                            lane);
  } else if (lane == 0) {
    words = plan_write_image(units, pieces, n_pieces, slot, comb, C, n_partials, a.PH,
                             a.P * a.PH, a.plan, a.plan_words);
  }
  if (a.status && lane == 0)
    *a.status = lengths_bad ? int32_t(MLA_ERR_BAD_SHAPE)
                            : (words < 0 ? int32_t(MLA_ERR_PLAN_TOO_SMALL) : int32_t(MLA_OK));
}

}  // namespace

int64_t plan_lds_bytes(int64_t batch, int64_t max_units, int64_t P) {
  return plan_lds_layout(batch, max_units, P).total;
}

hipError_t launch_plan(const PlanDeviceArgs& a, int64_t max_units, hipStream_t stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(64), 0, stream, a, max_units);
  return hipGetLastError();
}

}  // namespace mla
