// Host side of the fused attention kernel (attn_a2a.hip): the launch used by every attention
// entry point, and the work decomposition queries.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace xstage {

// Launches the fused attention + slab epilogue.  ws / ws_bytes: the caller's split workspace
// (NULL: no key split).  mode: 0 product, 1..4 traced variants, kAttnModePaced the paced
// persistent variant (with pace_chunks chunks per tile).  stamps: traced modes only.
// layout: source shards and destination head layout (NULL: contiguous [B, S, H, D] inputs,
// [S/P, H, D] slabs).  force_split > 0: exactly that many key splits instead of the
// model's choice (XSTAGE_ERR_INVALID if unavailable or the workspace is too small).
int launch_attn_any(const void* q, const void* k, const void* v, const SlabTable& slabs, int B, int S, int H, int D,
                    int P, float scale, void* ws, unsigned long long ws_bytes, hipStream_t stream, int mode = 0,
                    unsigned long long* stamps = nullptr, const Layout* layout = nullptr, int pace_chunks = 0,
                    int force_split = 0);
// Workgroups of a product launch given ws_bytes of split workspace; *n_split may be NULL.
int attn_workgroups(int B, int S, int H, int D, unsigned long long ws_bytes, int* n_split);
// Query rows per workgroup of that launch: 128 (4 waves) or 256 (8 waves).
int attn_wg_rows(int B, int S, int H, int D, unsigned long long ws_bytes);
// Workgroups of a paced launch in *n_wg (0 if the occupancy query failed); returns the tiles.
int attn_paced_workgroups(int B, int S, int H, int D, int* n_wg);
// Split-workspace bytes of a launch forced to n_split key splits (force_split above); *ok
// false when that split count is not available for the shape (see plan_forced).
unsigned long long attn_ws_forced(int B, int S, int H, int D, int n_split, bool* ok);
// Split-workspace bytes a launch of this shape uses given ws_bytes (~0: the full plan's).
unsigned long long attn_ws_used(int B, int S, int H, int D, unsigned long long ws_bytes);
// Per-workgroup (tile, split, j0, j1) of a product launch (tiles of attn_wg_rows query rows);
// returns the workgroup count.
int attn_schedule(int B, int S, int H, int D, unsigned long long ws_bytes, int cap, int* tile, int* split, int* j0,
                  int* j1);

}  // namespace xstage
