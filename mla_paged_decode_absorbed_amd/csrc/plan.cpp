// Split-KV planner (host side): deals (sequence, row block, key range) work to
// a fixed set of persistent workgroups so that each gets about the same number
// of key rounds.  The loops live in plan_core.h, shared with the device
// planner; this file adds the host-side lengths, tuning knobs and bounds.
// Pure host code; no HIP calls.  The processors of `phases` consecutive
// workgroups sit on one XCD, so the cache a processor's workgroups share is
// fetched from HBM once and the other reads hit that XCD's L2.
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "mla_decode.h"
#include "plan_core.h"
#include "plan_layout.h"
#include "validate.h"

namespace mla {

namespace {

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

// Phases per processor.  Measured on MI355X, sharing a unit's keys between
// 2 or 4 workgroups (one 16-key tile per wave and round, one round in flight)
// is slower than splitting the key range of whole 128-row units and merging
// the partials, for every shape tried (DeepSeek-V3 decode 126 vs 181 us/call,
// long-context e4m3 255 vs 1383 us/call), so 1 is the default; MLA_PHASES=2
// or 4 selects the shared-key schedule.
int choose_phases(int32_t G) {
  const int forced = env_int("MLA_PHASES", 0);
  if ((forced == 2 || forced == 4) && G % forced == 0) return forced;
  return 1;
}

}  // namespace

uint64_t plan_words_bound(const mla_shape& s, int32_t G) {
  const int64_t units = max_units(s);
  // pieces <= units + processors; every piece expands to at most 4 items
  return uint64_t(kHeaderWords + round_up8(G + 1) + 4 * (units + G) * kItemWords +
                  (units + G) * kCombineWords + 8);
}

uint64_t partial_bytes(int64_t n_partials) {
  const uint64_t o = uint64_t(n_partials) * kRowsPerBlock * kDLatent * sizeof(float);
  const uint64_t lse = uint64_t(n_partials) * kRowsPerBlock * sizeof(float);
  return o + (lse + 255) / 256 * 256;
}

void fixed_launch_info(const mla_shape& s, int32_t G, int32_t PH, mla_plan_info* info) {
  // Bounds that hold for every lengths of the shape: at most 2 (P - 1)
  // partials (a processor boundary cuts at most one unit, and a cut unit has
  // one partial per piece), one combine entry per 128-row unit, and at most
  // (units + P) pieces of PH items each.
  const int32_t P = std::max(1, G / PH);
  const int32_t G_out = P * PH;
  const int64_t unit_bound = max_units(s);
  info->num_workgroups = G_out;
  info->num_items = int32_t(std::min<int64_t>((unit_bound + P) * PH, INT32_MAX));
  info->num_partials = 2 * G_out;
  info->num_combine = int32_t(unit_bound);
  info->tile_tokens = kTileTokens;
  info->rows_per_block = kRowsPerBlock;
  info->phases = PH;
  info->plan_bytes = plan_words_bound(s, G_out) * sizeof(int32_t);
  info->workspace_bytes = partial_bytes(2 * int64_t(G_out));
}

int64_t max_units(const mla_shape& s) {
  const int64_t rows = int64_t(s.max_q_len) * s.num_heads;
  return int64_t(s.batch) * ((rows + kRowsPerBlock - 1) / kRowsPerBlock);
}

void plan_launch_params(int32_t* G, int32_t* PH, int32_t* item_cost) {
  const int force_wg = env_int("MLA_NUM_WORKGROUPS", 0);
  if (force_wg > 0) *G = force_wg;
  *PH = choose_phases(*G);
  *item_cost = std::max(0, env_int("MLA_ITEM_COST_ROUNDS", kItemCostRounds));
}

mla_status build_plan(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens,
                      int32_t G, int32_t* out, uint64_t out_words, mla_plan_info* info,
                      bool fixed_shape) {
  int32_t PH = 1, item_cost = kItemCostRounds;
  plan_launch_params(&G, &PH, &item_cost);
  const int32_t P = std::max(1, G / PH);            // processors

  std::vector<PlanUnit> units;
  for (int b = 0; b < s.batch; ++b) {
    const int32_t q = q_lens ? q_lens[b] : s.max_q_len;
    const int32_t n = plan_units_of(b, q, kv_lens[b], s.num_heads, nullptr);
    units.resize(units.size() + n);
    plan_units_of(b, q, kv_lens[b], s.num_heads, units.data() + units.size() - n);
  }
  const int32_t n_units = int32_t(units.size());

  auto unit_at = [&](int32_t i) { return units[size_t(i)]; };
  const int64_t total = plan_total(unit_at, n_units, item_cost);
  const int64_t per_proc = plan_per_proc<int64_t>(unit_at, n_units, total, item_cost, P);
  std::vector<PlanPiece> pieces(size_t(n_units) + P + 1);
  std::vector<int32_t> unit_first_piece(size_t(n_units) + 1, 0);
  const int64_t used = plan_fill<int64_t>(
      unit_at, n_units, per_proc, item_cost, P, true,
      [&](int32_t i, const PlanPiece& pc) { pieces[size_t(i)] = pc; },
      [&](int32_t u, int32_t i) { unit_first_piece[size_t(u)] = i; });
  const int32_t n_pieces = unit_first_piece[size_t(n_units)];
  const int32_t P_eff = std::max<int32_t>(1, int32_t(used));
  // a fixed launch shape keeps all P processors (those past P_eff get no items)
  const int32_t G_out = (fixed_shape ? P : P_eff) * PH;

  std::vector<int32_t> slot(size_t(n_pieces) + 1), comb(size_t(n_units) * kCombineWords + 1);
  int32_t C = 0, n_partials = 0;
  plan_slots(
      unit_at, [&](int32_t u) { return unit_first_piece[size_t(u)]; }, n_units,
      [&](int32_t p, int32_t v) { slot[size_t(p)] = v; },
      [&](int32_t e, int32_t b, int32_t row0, int32_t first, int32_t n) {
        int32_t* c = comb.data() + size_t(e) * kCombineWords;
        c[0] = b;
        c[1] = row0;
        c[2] = first;
        c[3] = n;
      },
      &C, &n_partials);
  const int64_t words = plan_write_image(units.data(), pieces.data(), n_pieces, slot.data(),
                                         comb.data(), C, n_partials, PH, G_out, out,
                                         int64_t(out_words));
  if (words < 0) return MLA_ERR_PLAN_TOO_SMALL;

  if (fixed_shape) {
    fixed_launch_info(s, G, PH, info);
    return MLA_OK;
  }
  info->num_workgroups = G_out;
  info->num_items = out[kWNumItems];
  info->num_partials = n_partials;
  info->num_combine = C;
  info->tile_tokens = kTileTokens;
  info->rows_per_block = kRowsPerBlock;
  info->phases = PH;
  info->plan_bytes = uint64_t(words) * sizeof(int32_t);
  info->workspace_bytes = partial_bytes(n_partials);
  return MLA_OK;
}

}  // namespace mla
