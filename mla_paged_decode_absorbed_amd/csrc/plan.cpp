// Split-KV planner: deals (sequence, row block, key range) work to a fixed set
// of persistent workgroups so that each gets about the same number of key
// rounds.  Pure host code; no HIP calls.
//
// A unit is 128 consecutive query rows of one sequence (row r is token r / H,
// head r % H); all its rows share one key stream.  Units are dealt to
// "processors" of `phases` consecutive workgroups on one XCD: a processor's
// workgroups each take 128/phases of the unit's rows over the same keys, so
// the cache is fetched from HBM once and the other reads hit that XCD's L2.
// When a unit's key range does not fit a processor's remaining budget it is
// cut at a round boundary (64 keys); every piece then writes a partial
// (O, LSE) and the unit gets a combine entry.  This is the split-K partition
// with a log-sum-exp merge from the FlashAttention-3 page (chapter 2),
// scheduled so that variable-length sequences balance across CUs.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla_decode.h"
#include "plan_layout.h"
#include "validate.h"

namespace mla {

namespace {

struct Unit {
  int32_t b, row0, rows, L, rounds;
};

struct Piece {
  int32_t proc, unit, k0, k1;
};

// Fixed cost of one piece, in rounds: the query load and the epilogue's write.
constexpr int kItemCostRounds = 2;
// A cut never leaves a piece shorter than this many rounds on either side.
constexpr int kMinPieceRounds = 2;

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

std::vector<Unit> make_units(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens) {
  std::vector<Unit> units;
  for (int b = 0; b < s.batch; ++b) {
    const int q = q_lens ? q_lens[b] : s.max_q_len;
    if (q <= 0) continue;
    const int rows = q * s.num_heads;
    const int L = kv_lens[b];
    const int rounds = (L + kRoundTokens - 1) / kRoundTokens;
    for (int r0 = 0; r0 < rows; r0 += kRowsPerBlock)
      units.push_back({b, r0, std::min(kRowsPerBlock, rows - r0), L, rounds});
  }
  return units;
}

// Phases per processor.  Measured on MI355X, sharing a unit's keys between
// 2 or 4 workgroups (one 16-key tile per wave and round, one round in flight)
// is slower than splitting the key range of whole 128-row units and merging
// the partials, for every shape tried (DeepSeek-V3 decode 126 vs 181 us/call,
// long-context e4m3 255 vs 1383 us/call), so 1 is the default; MLA_PHASES=2
// or 4 selects the shared-key schedule.
int choose_phases(int64_t /*n_units*/, int32_t G) {
  const int forced = env_int("MLA_PHASES", 0);
  if ((forced == 2 || forced == 4) && G % forced == 0) return forced;
  return 1;
}

}  // namespace

uint64_t plan_words_bound(const mla_shape& s, int32_t G) {
  const int64_t rows = int64_t(s.max_q_len) * s.num_heads;
  const int64_t units = int64_t(s.batch) * ((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  // pieces <= units + processors; every piece expands to at most 4 items
  return uint64_t(kHeaderWords + round_up8(G + 1) + 4 * (units + G) * kItemWords +
                  (units + G) * kCombineWords + 8);
}

uint64_t partial_bytes(int64_t n_partials) {
  const uint64_t o = uint64_t(n_partials) * kRowsPerBlock * kDLatent * sizeof(float);
  const uint64_t lse = uint64_t(n_partials) * kRowsPerBlock * sizeof(float);
  return o + (lse + 255) / 256 * 256;
}

mla_status build_plan(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens,
                      int32_t G, int32_t* out, uint64_t out_words, mla_plan_info* info,
                      bool fixed_shape) {
  std::vector<Unit> units = make_units(s, kv_lens, q_lens);

  const int force_wg = env_int("MLA_NUM_WORKGROUPS", 0);
  if (force_wg > 0) G = force_wg;
  const int PH = choose_phases(int64_t(units.size()), G);
  const int P = std::max(1, G / PH);            // processors
  const int item_cost = std::max(0, env_int("MLA_ITEM_COST_ROUNDS", kItemCostRounds));

  int64_t total = 0;
  for (const Unit& u : units) total += u.rounds + item_cost;

  // Greedy fill of processors in unit order with a per-processor budget of
  // per_proc round-costs; the smallest budget whose fill fits in P
  // processors is used.  Cutting a unit adds one piece (and its fixed cost).
  std::vector<Piece> pieces;
  std::vector<int32_t> unit_first_piece(units.size() + 1, 0);
  auto fill = [&](int64_t per_proc, bool record) -> int64_t {
    int64_t proc = 0;
    int64_t budget = per_proc;
    for (size_t ui = 0; ui < units.size(); ++ui) {
      const Unit& u = units[ui];
      if (record) unit_first_piece[ui] = int32_t(pieces.size());
      int k = 0;   // rounds of u already placed
      for (;;) {
        const int rem = u.rounds - k;
        const int64_t avail = budget - item_cost;
        if (rem <= avail + kMinPieceRounds / 2) {
          if (record)
            pieces.push_back({int32_t(proc), int32_t(ui), k * kRoundTokens, u.L});
          budget -= rem + item_cost;
          break;
        }
        if (avail >= kMinPieceRounds && rem - avail >= kMinPieceRounds) {
          if (record)
            pieces.push_back({int32_t(proc), int32_t(ui), k * kRoundTokens,
                              std::min(u.L, int((k + avail) * kRoundTokens))});
          k += int(avail);
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
    return proc + (budget < per_proc ? 1 : 0);
  };
  int64_t per_proc =
      std::max<int64_t>((total + P - 1) / std::max(P, 1), item_cost + kMinPieceRounds);
  while (fill(per_proc, false) > P) ++per_proc;
  const int32_t P_eff = std::max<int32_t>(1, int32_t(fill(per_proc, true)));
  unit_first_piece[units.size()] = int32_t(pieces.size());
  // a fixed launch shape keeps all P processors (those past P_eff get no items)
  const int32_t G_eff = (fixed_shape ? P : P_eff) * PH;

  // Slots and combine entries (per unit with more than one piece).
  std::vector<int32_t> slot(pieces.size(), -1);
  std::vector<int32_t> comb;   // flattened combine entries
  int32_t n_partials = 0;
  for (size_t ui = 0; ui < units.size(); ++ui) {
    const int32_t p0 = unit_first_piece[ui], p1 = unit_first_piece[ui + 1];
    if (p1 - p0 <= 1) continue;
    comb.insert(comb.end(), {units[ui].b, units[ui].row0, n_partials, p1 - p0});
    for (int32_t p = p0; p < p1; ++p) slot[p] = n_partials++;
  }
  const int32_t C = int32_t(comb.size() / kCombineWords);

  // Expand pieces into per-workgroup items: workgroup proc*PH + k takes rows
  // row0 + k*(128/PH) .. of the piece (skipped when they hold no valid row).
  const int rows_per_item = kRowsPerBlock / PH;
  std::vector<std::vector<int32_t>> per_wg(G_eff);
  int32_t N = 0;
  for (size_t i = 0; i < pieces.size(); ++i) {
    const Piece& pc = pieces[i];
    const Unit& u = units[pc.unit];
    for (int k = 0; k < PH; ++k) {
      const int off = k * rows_per_item;
      if (off >= u.rows) break;
      std::vector<int32_t>& v = per_wg[pc.proc * PH + k];
      v.insert(v.end(), {u.b, u.row0 + off, pc.k0, pc.k1, slot[i], off, 0, 0});
      ++N;
    }
  }

  const int64_t off_wg = kHeaderWords;
  const int64_t off_items = off_wg + round_up8(G_eff + 1);
  const int64_t off_comb = off_items + int64_t(N) * kItemWords;
  const int64_t words = off_comb + int64_t(C) * kCombineWords;
  if (uint64_t(words) > out_words) return MLA_ERR_PLAN_TOO_SMALL;

  std::memset(out, 0, size_t(words) * sizeof(int32_t));
  out[kWMagic] = kPlanMagic;
  out[kWVersion] = kPlanVersion;
  out[kWNumWg] = G_eff;
  out[kWNumItems] = N;
  out[kWNumCombine] = C;
  out[kWNumPartials] = n_partials;
  out[kWTile] = kTileTokens;
  out[kWRowsPerBlock] = kRowsPerBlock;
  out[kWOffWgStart] = int32_t(off_wg);
  out[kWOffItems] = int32_t(off_items);
  out[kWOffCombine] = int32_t(off_comb);
  out[kWPhases] = PH;
  int32_t* wg_start = out + off_wg;
  int32_t* items = out + off_items;
  int32_t n = 0;
  for (int32_t g = 0; g < G_eff; ++g) {
    wg_start[g] = n;
    std::memcpy(items + int64_t(n) * kItemWords, per_wg[g].data(),
                per_wg[g].size() * sizeof(int32_t));
    n += int32_t(per_wg[g].size() / kItemWords);
  }
  wg_start[G_eff] = n;
  if (!comb.empty()) std::memcpy(out + off_comb, comb.data(), comb.size() * sizeof(int32_t));

  info->num_workgroups = G_eff;
  info->num_items = N;
  info->num_partials = n_partials;
  info->num_combine = C;
  info->tile_tokens = kTileTokens;
  info->rows_per_block = kRowsPerBlock;
  info->phases = PH;
  info->plan_bytes = uint64_t(words) * sizeof(int32_t);
  info->workspace_bytes = partial_bytes(n_partials);
  if (fixed_shape) {
    // launch bounds that hold for every lengths of this shape: at most
    // 2 (P - 1) partials (a cut at each processor boundary adds at most two)
    // and one combine entry per 128-row unit; the kernels read the plan's
    // own counts on the device
    const int64_t rows = int64_t(s.max_q_len) * s.num_heads;
    const int64_t unit_bound = int64_t(s.batch) * ((rows + kRowsPerBlock - 1) / kRowsPerBlock);
    info->num_items = int32_t(std::max<int64_t>(N, 1));
    info->num_partials = 2 * G_eff;
    info->num_combine = int32_t(unit_bound);
    info->plan_bytes = plan_words_bound(s, G_eff) * sizeof(int32_t);
    info->workspace_bytes = partial_bytes(2 * int64_t(G_eff));
  }
  return MLA_OK;
}

}  // namespace mla
