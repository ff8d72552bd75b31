// Host side of the expert-wave grouped-GEMM stand-in (see moe_waves.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "common.hpp"

namespace xstage {

constexpr int kMoeMaxWaveExperts = 32;  // experts per wave (kernel-argument tables)

// Kernel arguments of one launch: its Linear-1 experts (type 0) and Linear-2 experts
// (type 1), each a contiguous expert range with per-expert tile prefix sums.
struct MoeLaunchArgs {
  const uint16_t* x;
  const uint16_t* w1;
  const uint16_t* w2;
  uint16_t* h;
  const int* dst_slab;
  const int* dst_row;
  SlabTable out;
  int out_rows[XSTAGE_MAX_P];
  int P, d_model, d_ff;
  int n_tiles[2];
  int mix;  // positions [0, mix) interleave the Linear-1 tiles with Linear-2 tiles
  int n_exp[2];
  int exp_id[2][kMoeMaxWaveExperts];
  int exp_off[2][kMoeMaxWaveExperts];
  int exp_rows[2][kMoeMaxWaveExperts];
  int tile_pre[2][kMoeMaxWaveExperts + 1];
  unsigned long long* stamps;  // optional: [run-wide tile][4 waves][4]
  int stamp_base[2];           // run-wide index of this launch's first tile of each type
};

struct MoeShape {
  int E, d_model, d_ff, experts_per_wave;
  const int* offsets;  // E + 1 token offsets (host)
  const int* rows;     // E token counts (host)
};

struct MoeBuffers {
  const uint16_t* x;
  const uint16_t* w1;
  const uint16_t* w2;
  uint16_t* h;
  const int* dst_slab;
  const int* dst_row;
  int P;
  uint16_t* out[XSTAGE_MAX_P];
  int out_rows[XSTAGE_MAX_P];
  unsigned long long* stamps;
};

// One launch of a schedule: Linear-1 tiles of experts [l1_begin, l1_end) and Linear-2 tiles
// of experts [l2_begin, l2_end).
struct MoeLaunch {
  int l1_begin, l1_end, l2_begin, l2_end;
};

// Output tiles of an expert with `rows` tokens and `n_cols` output columns.
int moe_tiles(int rows, int n_cols);

// The launches of a schedule (0 = expert waves, 1 = interleaved); returns their number.
int moe_plan(const MoeShape& sh, int schedule, std::vector<MoeLaunch>* launches);

int launch_moe(const MoeShape& sh, const MoeBuffers& buf, int schedule, hipStream_t stream);

}  // namespace xstage
