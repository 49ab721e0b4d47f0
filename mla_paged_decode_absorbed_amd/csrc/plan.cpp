// Split-KV planner: deals (sequence, row block, key range) work items to a
// fixed set of persistent workgroups so that each gets about the same number
// of key tiles.  Pure host code; no HIP calls.
//
// A row block is 128 consecutive query rows of one sequence (row r is token
// r / H, head r % H).  All rows of a block share one key stream, so a block is
// the unit whose keys are streamed once.  When a block's key range does not
// fit the workgroup's remaining budget it is cut; every piece then writes a
// partial (O, LSE) and the block gets a combine entry.  This is the split-K
// partition with a log-sum-exp merge from the FlashAttention-3 page
// (chapter 2), scheduled so that variable-length sequences balance across CUs.
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
  int32_t b, row0, L, tiles;
};

struct Piece {
  int32_t wg, b, row0, k0, k1;
};

// Fixed cost of one work item, in tiles: the 128-row query load (144 KiB,
// about four bf16 tiles) plus the epilogue's output write.
constexpr int kItemCostTiles = 4;
// A cut never leaves a piece shorter than this many tiles on either side.
constexpr int kMinPieceTiles = 2;

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

std::vector<Unit> make_units(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens,
                             int tile) {
  std::vector<Unit> units;
  for (int b = 0; b < s.batch; ++b) {
    const int q = q_lens ? q_lens[b] : s.max_q_len;
    if (q <= 0) continue;
    const int rows = q * s.num_heads;
    const int L = kv_lens[b];
    const int tiles = (L + tile - 1) / tile;
    for (int r0 = 0; r0 < rows; r0 += kRowsPerBlock) units.push_back({b, r0, L, tiles});
  }
  return units;
}

}  // namespace

uint64_t plan_words_bound(const mla_shape& s, int32_t G) {
  const int64_t rows = int64_t(s.max_q_len) * s.num_heads;
  const int64_t units = int64_t(s.batch) * ((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  return uint64_t(kHeaderWords + round_up8(G + 1) + (units + G) * kItemWords +
                  int64_t(G) * kCombineWords + 8);
}

uint64_t partial_bytes(int64_t n_partials) {
  const uint64_t o = uint64_t(n_partials) * kRowsPerBlock * kDLatent * sizeof(float);
  const uint64_t lse = uint64_t(n_partials) * kRowsPerBlock * sizeof(float);
  return o + (lse + 255) / 256 * 256;
}

mla_status build_plan(const mla_shape& s, const int32_t* kv_lens, const int32_t* q_lens,
                      int32_t G, int32_t* out, uint64_t out_words, mla_plan_info* info) {
  const int tile = tile_tokens_for(s.kv_dtype);
  std::vector<Unit> units = make_units(s, kv_lens, q_lens, tile);

  const int item_cost = std::max(0, env_int("MLA_ITEM_COST_TILES", kItemCostTiles));
  int64_t total = 0;
  for (const Unit& u : units) total += u.tiles + item_cost;

  // Optional override of the workgroup count (tuning / tests).
  const int force_wg = env_int("MLA_NUM_WORKGROUPS", 0);
  if (force_wg > 0) G = force_wg;

  // Greedy fill of workgroups in unit order with a per-workgroup budget of
  // per_wg tile-costs; the smallest budget whose fill fits in G workgroups is
  // used.  Cutting a unit adds one item (and its fixed cost) on each side.
  std::vector<Piece> pieces;
  std::vector<int32_t> unit_first_piece(units.size() + 1, 0);
  auto fill = [&](int64_t per_wg, bool record) -> int64_t {
    int64_t wg = 0;
    int64_t budget = per_wg;
    for (size_t ui = 0; ui < units.size(); ++ui) {
      const Unit& u = units[ui];
      if (record) unit_first_piece[ui] = int32_t(pieces.size());
      int k = 0;
      for (;;) {
        const int rem = u.tiles - k;
        const int64_t avail = budget - item_cost;
        if (rem <= avail + kMinPieceTiles / 2) {
          if (record) pieces.push_back({int32_t(wg), u.b, u.row0, k * tile, u.L});
          budget -= rem + item_cost;
          break;
        }
        if (avail >= kMinPieceTiles && rem - avail >= kMinPieceTiles) {
          if (record)
            pieces.push_back({int32_t(wg), u.b, u.row0, k * tile,
                              std::min(u.L, int((k + avail) * tile))});
          k += int(avail);
        }
        ++wg;
        budget = per_wg;
        if (!record && wg > G) return wg + 1;
      }
      if (budget <= item_cost) {
        ++wg;
        budget = per_wg;
      }
    }
    return wg + (budget < per_wg ? 1 : 0);
  };
  int64_t per_wg = std::max<int64_t>((total + G - 1) / std::max(G, 1), item_cost + kMinPieceTiles);
  while (fill(per_wg, false) > G) ++per_wg;
  const int32_t G_eff = std::max<int32_t>(1, int32_t(fill(per_wg, true)));
  unit_first_piece[units.size()] = int32_t(pieces.size());

  // Slots and combine entries.
  std::vector<int32_t> slot(pieces.size(), -1);
  std::vector<int32_t> comb;   // flattened combine entries
  int32_t n_partials = 0;
  for (size_t ui = 0; ui < units.size(); ++ui) {
    const int32_t p0 = unit_first_piece[ui], p1 = unit_first_piece[ui + 1];
    if (p1 - p0 <= 1) continue;
    comb.insert(comb.end(), {units[ui].b, units[ui].row0, n_partials, p1 - p0});
    for (int32_t p = p0; p < p1; ++p) slot[p] = n_partials++;
  }
  const int32_t N = int32_t(pieces.size());
  const int32_t C = int32_t(comb.size() / kCombineWords);

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
  out[kWTile] = tile;
  out[kWRowsPerBlock] = kRowsPerBlock;
  out[kWOffWgStart] = int32_t(off_wg);
  out[kWOffItems] = int32_t(off_items);
  out[kWOffCombine] = int32_t(off_comb);
  int32_t* wg_start = out + off_wg;
  for (int32_t i = 0; i < N; ++i) wg_start[pieces[i].wg + 1]++;
  for (int32_t g = 0; g < G_eff; ++g) wg_start[g + 1] += wg_start[g];
  int32_t* items = out + off_items;
  for (int32_t i = 0; i < N; ++i) {
    int32_t* it = items + int64_t(i) * kItemWords;
    it[0] = pieces[i].b;
    it[1] = pieces[i].row0;
    it[2] = pieces[i].k0;
    it[3] = pieces[i].k1;
    it[4] = slot[i];
  }
  std::memcpy(out + off_comb, comb.data(), comb.size() * sizeof(int32_t));

  info->num_workgroups = G_eff;
  info->num_items = N;
  info->num_partials = n_partials;
  info->num_combine = C;
  info->tile_tokens = tile;
  info->rows_per_block = kRowsPerBlock;
  info->plan_bytes = uint64_t(words) * sizeof(int32_t);
  info->workspace_bytes = partial_bytes(n_partials);
  return MLA_OK;
}

}  // namespace mla
