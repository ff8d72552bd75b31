// Host side of the key-range split: how many splits a launch uses, and the library-owned
// buffers (split partials, per-tile arrival counters) that the splits merge through.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xstage {

struct SplitPlan {
  int n_split = 1;          // key-range splits per (b, h, m-tile); 1 = no merge
  int kvb_per_split = 0;    // 64-key blocks per split (the last split may get fewer)
  void* partial = nullptr;  // n_tiles * n_split partial records
  uint32_t* counters = nullptr;  // n_tiles arrival counters, zero between launches
};

// Picks the key-split count of `n_tiles` tiles of 128 query rows over `nkv` blocks of 64
// keys (head dimension D) on the current device, from a cost model of rounds of
// co-resident workgroups (two per compute unit) and of the merge of split tiles.
SplitPlan choose_split(int n_tiles, int nkv, int D, size_t partial_bytes_per_unit);

// Returns buffers of at least `partial_bytes` and `n_counters` zeroed counters owned by the
// library for (current device, stream).  Grows them on demand: growing synchronizes
// `stream` first (the old buffers may still be read by earlier launches on it).
int acquire_workspace(hipStream_t stream, size_t partial_bytes, int n_counters, void** partial,
                      uint32_t** counters);

}  // namespace xstage
