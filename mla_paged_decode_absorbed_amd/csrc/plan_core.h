// Split-KV planner core, shared by the host planner (plan.cpp) and the device
// planner (plan_kernel.hip): plain loops over caller-provided arrays, so both
// build the same plan image from the same lengths.
//
// A unit is 128 consecutive query rows of one sequence (row r is token r / H,
// head r % H); all its rows share one key stream.  Units are dealt, in order,
// to "processors" of `phases` consecutive workgroups: a processor's
// workgroups each take 128/phases of the unit's rows over the same keys.
// Every processor gets a budget of per_proc round-costs (a round is 64 keys;
// each piece also costs a fixed item_cost for its query load and epilogue).
// A unit that does not fit the remaining budget is cut at a round boundary,
// never leaving a piece under kMinPieceRounds; each piece of a cut unit
// writes a partial (O, LSE) and the unit gets a combine entry.  The smallest
// per_proc whose fill fits P processors is used.  This is the split-K
// partition with a log-sum-exp merge of the FlashAttention-3 in DeepSeek-R1
// page (chapter 2), scheduled so that sequences of any length mix balance
// across CUs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_layout.h"

namespace mla {

struct PlanUnit {
  int32_t b, row0, rows, L, rounds;
};

struct PlanPiece {
  int32_t proc, unit, k0, k1;
};

// Fixed cost of one piece, in rounds: the query load and the epilogue's write.
constexpr int kItemCostRounds = 2;
// A cut never leaves a piece shorter than this many rounds on either side.
constexpr int kMinPieceRounds = 2;

__host__ __device__ inline int64_t plan_round_up8(int64_t x) { return (x + 7) / 8 * 8; }

// A value every lane of the device planner's wave holds alike: on the GPU it
// is read from the first lane, so the loops below run on the scalar unit.
__host__ __device__ inline int32_t plan_uniform(int32_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(v);
#else
  return v;
#endif
}

__host__ __device__ inline PlanUnit plan_load(const PlanUnit& u) {
  return {plan_uniform(u.b), plan_uniform(u.row0), plan_uniform(u.rows), plan_uniform(u.L),
          plan_uniform(u.rounds)};
}

__host__ __device__ inline PlanPiece plan_load(const PlanPiece& p) {
  return {plan_uniform(p.proc), plan_uniform(p.unit), plan_uniform(p.k0), plan_uniform(p.k1)};
}

// Units of sequence b (q query tokens, L keys): ceil(q * H / 128) of them.
// Writes them to out (if not null) and returns their number.
__host__ __device__ inline int32_t plan_units_of(int32_t b, int32_t q, int32_t L, int32_t H,
                                                 PlanUnit* out) {
  if (q <= 0) return 0;
  const int32_t rows = q * H;
  const int32_t rounds = (L + kRoundTokens - 1) / kRoundTokens;
  int32_t n = 0;
  for (int32_t r0 = 0; r0 < rows; r0 += kRowsPerBlock, ++n)
    if (out) out[n] = {b, r0, rows - r0 < kRowsPerBlock ? rows - r0 : kRowsPerBlock, L, rounds};
  return n;
}

// The loops below read units through unit_at(i) and write results through
// put_*(...) callables, so the host can run them over plain arrays and the
// device planner over arrays it caches in registers.

// Greedy fill with a budget of per_proc per processor.  Returns the number
// of processors used; without recording it stops early and returns P + 2 as
// soon as more than P are needed.  Recording passes the pieces (in unit
// order, so also in processor order) to put_piece(index, piece) and the
// first piece of every unit to put_first(unit, index), with
// put_first(n_units, piece count) last.
// I is the integer type of the budgets: int64_t always works; int32_t (fast
// scalar compares on the GPU) when the total cost of all units fits in it.
template <class I, class UnitAt, class PutPiece, class PutFirst>
__host__ __device__ inline I plan_fill(UnitAt&& unit_at, int32_t n_units, I per_proc,
                                       int32_t item_cost, I P, bool record,
                                       PutPiece&& put_piece, PutFirst&& put_first) {
  I proc = 0;
  I budget = per_proc;
  int32_t np = 0;
  for (int32_t ui = 0; ui < n_units; ++ui) {
    const PlanUnit u = unit_at(ui);
    if (record) put_first(ui, np);
    int32_t k = 0;   // rounds of u already placed
    for (;;) {
      const I rem = u.rounds - k;
      const I avail = budget - item_cost;
      if (rem <= avail + kMinPieceRounds / 2) {
        if (record) put_piece(np++, PlanPiece{int32_t(proc), ui, k * kRoundTokens, u.L});
        budget -= rem + item_cost;
        break;
      }
      if (avail >= kMinPieceRounds && rem - avail >= kMinPieceRounds) {
        if (record) {
          const int64_t k1 = (int64_t(k) + avail) * kRoundTokens;
          put_piece(np++, PlanPiece{int32_t(proc), ui, k * kRoundTokens,
                                    int32_t(k1 < u.L ? k1 : u.L)});
        }
        k += int32_t(avail);
      }
      ++proc;
      budget = per_proc;
      if (!record && proc > P) return proc + 1;
    }
    if (budget <= item_cost) {
      ++proc;
      budget = per_proc;
    }
  }
  if (record) put_first(n_units, np);
  return proc + (budget < per_proc ? 1 : 0);
}

// Total cost of all units: rounds plus the per-piece cost of one piece each.
template <class UnitAt>
__host__ __device__ inline int64_t plan_total(UnitAt&& unit_at, int32_t n_units,
                                              int32_t item_cost) {
  int64_t total = 0;
  for (int32_t ui = 0; ui < n_units; ++ui) total += unit_at(ui).rounds + item_cost;
  return total;
}

// The smallest budget, from the even share up, whose fill fits P processors.
template <class I, class UnitAt>
__host__ __device__ inline I plan_per_proc(UnitAt&& unit_at, int32_t n_units, int64_t total,
                                           int32_t item_cost, I P) {
  const int64_t Pd = P > 1 ? P : 1;
  I per_proc = I((total + Pd - 1) / Pd);
  if (per_proc < item_cost + kMinPieceRounds) per_proc = item_cost + kMinPieceRounds;
  auto none = [](int32_t, auto) {};
  while (plan_fill<I>(unit_at, n_units, per_proc, item_cost, P, false, none, none) > P)
    ++per_proc;
  return per_proc;
}

// Partial slots and combine entries, both in unit order: the pieces of a unit
// cut in several get consecutive slots (put_slot(piece, slot)) and the unit a
// combine entry put_comb(entry, b, row0, first slot, pieces); a unit in one
// piece gets slot -1.  first_at(u) is the unit's first piece (first_at(n_units)
// the piece count).
template <class UnitAt, class FirstAt, class PutSlot, class PutComb>
__host__ __device__ inline void plan_slots(UnitAt&& unit_at, FirstAt&& first_at, int32_t n_units,
                                           PutSlot&& put_slot, PutComb&& put_comb,
                                           int32_t* n_comb, int32_t* n_partials) {
  int32_t np = 0, nc = 0;
  int32_t p0 = n_units > 0 ? first_at(0) : 0;
  for (int32_t ui = 0; ui < n_units; ++ui) {
    const int32_t p1 = first_at(ui + 1);
    if (p1 - p0 <= 1) {
      for (int32_t p = p0; p < p1; ++p) put_slot(p, -1);
    } else {
      const PlanUnit u = unit_at(ui);
      put_comb(nc++, u.b, u.row0, np, p1 - p0);
      for (int32_t p = p0; p < p1; ++p) put_slot(p, np++);
    }
    p0 = p1;
  }
  *n_comb = nc;
  *n_partials = np;
}

// Writes the plan image for G_out workgroups (processor p owns workgroups
// p * PH .. p * PH + PH - 1; the k-th takes rows k * 128/PH.. of each of its
// pieces, skipped where the unit has no such rows).  Returns the number of
// words written, or -1 if they exceed out_words.
__host__ __device__ inline int64_t plan_write_image(
    const PlanUnit* units, const PlanPiece* pieces, int32_t n_pieces, const int32_t* slot,
    const int32_t* comb, int32_t n_comb, int32_t n_partials, int32_t PH, int32_t G_out,
    int32_t* out, int64_t out_words) {
  const int32_t rows_per_item = kRowsPerBlock / PH;
  int64_t N = 0;
  for (int32_t i = 0; i < n_pieces; ++i) {
    const int32_t rows = plan_uniform(units[plan_uniform(pieces[i].unit)].rows);
    for (int32_t k = 0; k < PH && k * rows_per_item < rows; ++k) ++N;
  }
  const int64_t off_wg = kHeaderWords;
  const int64_t off_items = off_wg + plan_round_up8(G_out + 1);
  const int64_t off_comb = off_items + N * kItemWords;
  const int64_t words = off_comb + int64_t(n_comb) * kCombineWords;
  if (words > out_words) return -1;
  for (int64_t w = 0; w < off_items; ++w) out[w] = 0;
  out[kWMagic] = kPlanMagic;
  out[kWVersion] = kPlanVersion;
  out[kWNumWg] = G_out;
  out[kWNumItems] = int32_t(N);
  out[kWNumCombine] = n_comb;
  out[kWNumPartials] = n_partials;
  out[kWTile] = kTileTokens;
  out[kWRowsPerBlock] = kRowsPerBlock;
  out[kWOffWgStart] = int32_t(off_wg);
  out[kWOffItems] = int32_t(off_items);
  out[kWOffCombine] = int32_t(off_comb);
  out[kWPhases] = PH;
  int32_t* wg_start = out + off_wg;
  int32_t* items = out + off_items;
  int32_t n = 0, i = 0;
  for (int32_t p = 0; p < G_out / PH; ++p) {
    const int32_t i0 = i;
    while (i < n_pieces && plan_uniform(pieces[i].proc) == p) ++i;
    for (int32_t k = 0; k < PH; ++k) {
      wg_start[p * PH + k] = n;
      for (int32_t j = i0; j < i; ++j) {
        const PlanPiece pc = plan_load(pieces[j]);
        const PlanUnit u = plan_load(units[pc.unit]);
        const int32_t off = k * rows_per_item;
        if (off >= u.rows) continue;
        int32_t* it = items + int64_t(n++) * kItemWords;
        it[0] = u.b;
        it[1] = u.row0 + off;
        it[2] = pc.k0;
        it[3] = pc.k1;
        it[4] = plan_uniform(slot[j]);
        it[5] = off;
        it[6] = 0;
        it[7] = 0;
      }
    }
  }
  for (int32_t g = (G_out / PH) * PH; g <= G_out; ++g) wg_start[g] = n;
  for (int64_t w = 0; w < int64_t(n_comb) * kCombineWords; ++w)
    out[off_comb + w] = plan_uniform(comb[w]);
  return words;
}

}  // namespace mla
