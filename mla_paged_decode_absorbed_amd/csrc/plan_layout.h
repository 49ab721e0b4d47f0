// Plan image layout shared by the host planner and the device kernels.
//
// The plan is a flat array of int32 words:
//
//   [0]  kPlanMagic            [1] kPlanVersion
//   [2]  num_workgroups (G)    [3] num_items (N)
//   [4]  num_combine (C)       [5] num_partials
//   [6]  tile_tokens           [7] rows_per_block
//   [8]  offset of wg_start    [9] offset of items     [10] offset of combine
//   [11] phases                [12..15] reserved
//   wg_start[G + 1]            items of workgroup g are [wg_start[g], wg_start[g+1])
//   items[N][kItemWords]       {b, row0, k0, k1, slot, slot_row, 0, 0}
//                              rows row0 .. row0 + 128/phases - 1 of sequence b,
//                              keys [k0, k1); slot < 0: write O/LSE directly,
//                              else partial slot, rows from slot_row on
//   combine[C][kCombineWords]  {b, row0, first_slot, n_splits}
//
// Offsets are in words and multiples of 8 (32-byte aligned items).
#pragma once
#include <stdint.h>

namespace mla {

constexpr int32_t kPlanMagic = 0x504C414D;  // "MALP" little-endian
constexpr int32_t kPlanVersion = 2;
constexpr int kHeaderWords = 16;
constexpr int kItemWords = 8;
constexpr int kCombineWords = 4;
constexpr int kRowsPerBlock = 128;   // query rows of one planner unit / partial slot
constexpr int kTileTokens = 16;      // keys per kernel tile
constexpr int kRoundTokens = 64;     // keys per ring round; key splits fall on multiples
constexpr int kDLatent = 512;
constexpr int kDRope = 64;
constexpr int kDQK = kDLatent + kDRope;

enum PlanWord : int {
  kWMagic = 0, kWVersion, kWNumWg, kWNumItems, kWNumCombine, kWNumPartials,
  kWTile, kWRowsPerBlock, kWOffWgStart, kWOffItems, kWOffCombine, kWPhases
};

inline int64_t round_up8(int64_t x) { return (x + 7) / 8 * 8; }

// Tokens per pipeline tile for a cache dtype (0 = bf16, 1 = fp8).
inline int tile_tokens_for(int /*kv_dtype*/) { return kTileTokens; }
// Smallest page size the kernels take: a tile (bf16) or a whole ring round
// (e4m3, whose 64 per-token scales are fetched with one copy) per page.
inline int min_page_size_for(int kv_dtype) { return kv_dtype == 1 ? kRoundTokens : kTileTokens; }

}  // namespace mla
