// Host side of the key-range split: how many splits a launch uses, and the layout of the
// caller-owned split workspace (per-tile arrival counters, then the split partials) that
// the splits merge through.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xstage {

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Launch mode of the attention kernel's paced persistent variant (the kernel's own modes
// 0..4 are the product and the traced variants).
constexpr int kAttnModePaced = 5;

struct SplitPlan {
  int n_split = 1;          // key-range splits per (b, h, m-tile); 1 = no merge
  int kvb_per_split = 0;    // 64-key blocks per split (the last split may get fewer)
  void* partial = nullptr;  // n_tiles * n_split partial records
  uint32_t* counters = nullptr;  // n_tiles arrival counters, zero between launches
};

// Largest split-partial area a plan may use (the workspace size query reports plans up to
// this; a launch given less workspace splits less).
constexpr size_t kSplitPartialCap = size_t(128) << 20;

// Bytes of split partials of one (tile, split) unit: 4 waves x (2 fp16 O chunks per 32-wide
// d tile + one (m, l, scale) chunk) x 64 lanes x 16 B.
inline size_t partial_bytes_per_unit(int D) { return (size_t)4 * (2 * (D / 32) + 1) * 64 * 16; }

// Workspace layout, the same for every shape: kSplitMaxTiles uint32 arrival counters (tile t
// uses counter t), then the partials.  The counters of any later call, whatever its shape,
// therefore never overlap an earlier call's partials, and every call leaves them at zero.
// Shapes with more tiles are not split (they fill the device without it).
constexpr int kSplitMaxTiles = 4096;
constexpr size_t kCounterAreaBytes = (size_t)kSplitMaxTiles * 4;

// Width rule of an attention launch: true when it runs 8-wave workgroups over 256 query rows
// instead of 4-wave ones over 128.  even_tiles: every (b, h) has an even number of 128-row
// tiles; units4: 128-row tiles x key splits; kvb: 64-key blocks per key range; cus: compute
// units of the device.
bool wide_rule(bool even_tiles, long units4, int n_split, int kvb, int cus);

// Picks the key-split count of `n_tiles` tiles of 128 query rows over `nkv` blocks of 64
// keys (head dimension D) on the current device, from a cost model of rounds of
// co-resident workgroups (two per compute unit) and of the merge of split tiles, among the
// plans whose partials fit `partial_capacity` bytes (0: no split).
SplitPlan choose_split(int n_tiles, int nkv, int D, size_t partial_capacity);

// Plan with exactly n_split key splits (1: none) and the workspace bytes it uses (0 for
// n_split = 1).  False when n_split is outside 1..15, the shape has more than kSplitMaxTiles
// tiles (n_split > 1), nkv 64-key blocks cannot form exactly n_split non-empty equal ranges,
// or the partials exceed kSplitPartialCap.
bool plan_forced(int n_tiles, int nkv, int D, int n_split, SplitPlan* plan, size_t* used);

// Plan of a launch given `ws_bytes` of split workspace (ws_bytes = 0: no workspace): the
// counters take kCounterAreaBytes, the partials at most the rest (and at most
// kSplitPartialCap); more than kSplitMaxTiles tiles are never split.  Returns the workspace bytes the plan uses in *used (0 without split).
SplitPlan plan_with_workspace(int n_tiles, int nkv, int D, unsigned long long ws_bytes, size_t* used);

// Per-workgroup work of a launch whose workgroups all fit on the device at once.  Workgroups
// are dispatched in index order, round-robin over the 8 XCDs (i % 8), and each XCD fills
// every CU once before it places a second workgroup on any: with c CUs per XCD and n
// workgroups on it, slots (i / 8) 0 .. n-c-1 share their CU with slots c .. n-1, and the
// slots in between have a CU to themselves.  Two workgroups on one CU do not progress
// alike: the older one (lower slot) keeps most of the issue slots.  Measured per-block
// rates relative to a lone workgroup (MI355X, D = 128): older sharer 0.864, younger sharer
// 0.58.  The table assigns every workgroup a (tile, split, key-block range) so that each
// tile mixes these classes and its blocks are shared out to minimise the time its slowest
// split needs (blocks / rate): the splits of a tile then finish together and no tile waits
// on an all-younger-sharer group.  Only
// speed depends on this; any table that partitions every tile's keys is correct.
constexpr int kUnitTableCap = 512;
struct UnitTable {
  uint32_t e[kUnitTableCap];  // tile | split << 10 | j0 << 14 | j1 << 23
};
constexpr uint32_t unit_entry(int tile, int split, int j0, int j1) {
  return (uint32_t)tile | (uint32_t)split << 10 | (uint32_t)j0 << 14 | (uint32_t)j1 << 23;
}

// Table for n_tiles tiles of n_split splits over nkv key blocks on `cus` compute units, or
// false when the launch is outside its scope (more workgroups than fit at once, no more
// than one per CU, more than kUnitTableCap workgroups, nkv > 511, fewer than 2 blocks per
// split, CU count not a multiple of 8).
bool build_unit_table(int n_tiles, int nkv, int n_split, int cus, UnitTable* table);

// Cached build_unit_table for the current device (nullptr when out of scope).
const UnitTable* unit_table(int n_tiles, int nkv, int n_split);


}  // namespace xstage
