// Plan image layout shared by the host planner and the device kernels.
//
// The plan is a flat array of int32 words:
//
//   [0]  kPlanMagic            [1] kPlanVersion
//   [2]  num_workgroups (G)    [3] num_items (N)
//   [4]  num_combine (C)       [5] num_partials
//   [6]  tile_tokens           [7] rows_per_block
//   [8]  offset of wg_start    [9] offset of items     [10] offset of combine
//   [11..15] reserved
//   wg_start[G + 1]            items of workgroup g are [wg_start[g], wg_start[g+1])
//   items[N][kItemWords]       {b, row0, k0, k1, slot, 0, 0, 0}
//                              slot < 0: write O/LSE directly; else partial slot
//   combine[C][kCombineWords]  {b, row0, first_slot, n_splits}
//
// Offsets are in words and multiples of 8 (32-byte aligned items).
#pragma once
#include <stdint.h>

namespace mla {

constexpr int32_t kPlanMagic = 0x504C414D;  // "MALP" little-endian
constexpr int32_t kPlanVersion = 1;
constexpr int kHeaderWords = 16;
constexpr int kItemWords = 8;
constexpr int kCombineWords = 4;
constexpr int kRowsPerBlock = 128;   // query rows handled by one work item
constexpr int kDLatent = 512;
constexpr int kDRope = 64;
constexpr int kDQK = kDLatent + kDRope;

enum PlanWord : int {
  kWMagic = 0, kWVersion, kWNumWg, kWNumItems, kWNumCombine, kWNumPartials,
  kWTile, kWRowsPerBlock, kWOffWgStart, kWOffItems, kWOffCombine
};

inline int64_t round_up8(int64_t x) { return (x + 7) / 8 * 8; }

// Tokens per pipeline tile for a cache dtype (0 = bf16, 1 = fp8).
inline int tile_tokens_for(int kv_dtype) { return kv_dtype == 1 ? 64 : 32; }

}  // namespace mla
