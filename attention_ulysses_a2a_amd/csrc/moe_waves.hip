// Grouped-GEMM stand-in for the interleaved expert-wave scheduling of the X-Stage explainer
// (gist.science, arXiv 2607.23264), "Contributions", MegaMoE (reshaping) item, and
// "Results", MegaMoE optimisation: a mixture-of-experts layer runs Linear-1 (compute whose
// output stays local) and Linear-2 (whose epilogue issues the combine all-to-all's stores)
// over waves of experts.  The expert-wave baseline runs, per wave, all Linear-1 tiles and
// then all Linear-2 tiles, so the stores come in concentrated bursts; the interleaved
// schedule runs the Linear-2 tiles of wave w together with the Linear-1 tiles of wave w+1,
// so that on every CU store bursts run beside Linear-1 compute.  On one GPU the P
// destinations are buffers in local HBM.
//
// One kernel computes a launch's mixed list of 128 x 128 output tiles, Y = X W^T with bf16
// inputs and fp32 accumulation (weights [N, K], K contiguous, as a linear layer stores
// them): v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand, so a lane holds
// four consecutive output columns of one token row; operands go global -> LDS with
// buffer_load_dwordx4 ... lds, XOR-swizzled, weight blocks two ahead (three slots), token
// blocks one ahead (two slots); the tile is restaged through
// LDS so every store is a 16-byte chunk of a 256-byte row segment.  Linear-1 tiles write H
// (bf16, [tokens, d_ff]); Linear-2 tiles send each token row to (dst_slab[t], dst_row[t]).
// Linear-2 of an expert reads H written by an earlier launch, so stream order carries the
// only dependency: no workgroup ever waits on another.
#include <algorithm>
#include <vector>

#include "common.hpp"
#include "moe_waves.hpp"

namespace xstage {

namespace {

constexpr int kTM = 128;   // token rows per tile
constexpr int kTN = 128;   // output columns per tile
constexpr int kTK = 64;    // k per LDS block
[[maybe_unused]] constexpr int kSlot = kTM * kTK * 2;  // bytes of one operand block (16 KiB)
// Positions of a mixed launch over which its Linear-1 tiles are spread, per Linear-1 tile.
// 1: the Linear-1 tiles take the first positions, so each starts at once (while they fit
// the co-resident slots) and the Linear-2 tiles fill the other slots and the tail.  Spreading
// them wider starts some long Linear-1 tiles late: on MI355X at the DeepSeek-V3-sized layer
// 1 gives 0.81 ms, 2 gives 0.98 ms, an even spread over the whole launch 0.99 ms (expert
// waves: 0.94 ms).
constexpr int kMixPerL1 = 1;

}  // namespace

__global__ __launch_bounds__(256, 2) void moe_gemm_kernel(const MoeLaunchArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  // Weight (A) blocks in three slots, token (B) blocks in two, as separate LDS objects (the
  // compiler then tracks the asynchronous copies per slot); 80 KiB, two workgroups per CU.
  __shared__ __attribute__((aligned(16))) char lds_w0[kSlot];
  __shared__ __attribute__((aligned(16))) char lds_w1[kSlot];
  __shared__ __attribute__((aligned(16))) char lds_w2[kSlot];
  __shared__ __attribute__((aligned(16))) char lds_x0[kSlot];
  __shared__ __attribute__((aligned(16))) char lds_x1[kSlot];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  unsigned long long t_start = 0;
  if (a.stamps) t_start = __builtin_amdgcn_s_memrealtime();

  // Tile of this workgroup.  Positions [0, mix) interleave all n1 Linear-1 tiles evenly with
  // mix - n1 Linear-2 tiles (position i is Linear-2 when floor((i+1) m2 / mix) exceeds
  // floor(i m2 / mix)); the remaining positions are Linear-2 tiles.  Workgroups start in
  // position order, so the long Linear-1 tiles start early and short tiles fill the tail.
  const int n1 = a.n_tiles[0], mix = a.mix, i = blockIdx.x;
  int type, idx;
  if (i < mix) {
    const int m2 = mix - n1;
    const int c0 = (int)((long long)i * m2 / mix), c1 = (int)((long long)(i + 1) * m2 / mix);
    type = c1 > c0 ? 1 : 0;
    idx = type ? c0 : i - c0;
  } else {
    type = 1;
    idx = mix - n1 + (i - mix);
  }
  int j = 0;
  while (j + 1 < a.n_exp[type] && idx >= a.tile_pre[type][j + 1]) ++j;
  const int K = type ? a.d_ff : a.d_model;
  const int N = type ? a.d_model : a.d_ff;
  const int NT = N / kTN;
  const int loc = idx - a.tile_pre[type][j];
  const int mt = loc / NT, nt = loc - mt * NT;
  const int e = a.exp_id[type][j], off = a.exp_off[type][j], rows = a.exp_rows[type][j];
  const int m0 = mt * kTM;
  const int xrows = min(kTM, rows - m0);

  const uint16_t* wsrc = (type ? a.w2 : a.w1) + ((size_t)e * N + (size_t)nt * kTN) * K;
  const uint16_t* xsrc = (type ? a.h : a.x) + ((size_t)off + m0) * K;
  // Token rows past the expert's last read as zeros (range check of the buffer resource).
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void*)wsrc, (short)0, kTN * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)xsrc, (short)0, xrows * K * 2, 0x00020000);

  // Instruction l of wave w fills the 1 KiB LDS segment (4l + w) of a block: chunk
  // c = (4l + w) * 64 + lane holds row c / 8, logical 16-byte chunk (c % 8) ^ sw(row) with
  // sw(row) = (row / 2) % 8.  A 128-byte row is half of the 64 banks, so rows of one parity
  // share a bank half; sw gives the 8 rows of each parity among any 16 consecutive rows 8
  // different chunk positions, and a 16-lane group of operand reads (16 rows, one logical
  // chunk) touches all 64 banks once (with (row % 8) rows r and r + 8 collide: ~4 conflict
  // cycles per LDS instruction, against 0.08 now; the time is the same either way).
  uint32_t ld_off[4];
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const int c = (l * 4 + w) * 64 + lane;
    const int row = c >> 3, lc = (c & 7) ^ ((row >> 1) & 7);
    ld_off[l] = (uint32_t)row * K * 2u + lc * 16u;
  }
  auto wslot = [&](int s) -> char* { return s == 0 ? lds_w0 : s == 1 ? lds_w1 : lds_w2; };
  auto xslot = [&](int s) -> char* { return s ? lds_x1 : lds_x0; };
  auto load_w = [&](int s, int kb) {
#pragma unroll
    for (int l = 0; l < 4; ++l)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(wslot(s) + (l * 4 + wu) * 1024),
                                               16, ld_off[l] + kb * (kTK * 2), 0, 0, 0);
  };
  auto load_x = [&](int s, int kb) {
#pragma unroll
    for (int l = 0; l < 4; ++l)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xslot(s) + (l * 4 + wu) * 1024),
                                               16, ld_off[l] + kb * (kTK * 2), 0, 0, 0);
  };

  // Wave w computes output columns wn .. wn+63 (weight rows) of token rows wm .. wm+63.
  const int wn = (w >> 1) * 64, wm = (w & 1) * 64;
  const int r32 = lane & 31;
  int aoff[4];  // byte offset of this lane's operand chunk for k-step ks, row r32 of a 32-row block
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = r32 * (kTK * 2) + (((2 * ks + hl) ^ ((r32 >> 1) & 7)) << 4);
  f32x16 acc[2][2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[ii][jj] = f32x16{};

  auto compute = [&](int sw, int sx) {
    const char* W = wslot(sw);
    const char* X = xslot(sx);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) af[ii] = *reinterpret_cast<const bf16x8*>(W + (wn + 32 * ii) * (kTK * 2) + aoff[ks]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) bf[jj] = *reinterpret_cast<const bf16x8*>(X + (wm + 32 * jj) * (kTK * 2) + aoff[ks]);
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ii], bf[jj], acc[ii][jj], 0, 0, 0);
    }
  };

  // Weight blocks (streamed from HBM) run two ahead, token blocks (mostly L2 hits) one ahead.
  // At the start of block kb the token copy of kb+1 is issued before the weight copy of kb+2;
  // copies complete in issue order, so the wait at the end of the block can leave the latter
  // (4 copies per thread) outstanding.  The block ends with a bare s_barrier after that wait:
  // __syncthreads()'s fence would wait for every outstanding copy into LDS.  Slot reuse: the
  // copies issued at the start of block kb go to the slots read in block kb - 1, which every
  // wave has finished (its reads consumed by its MFMAs, lgkmcnt(0), then the barrier).
  const int nkb = K / kTK;
  load_x(0, 0);
  load_w(0, 0);
  if (1 < nkb) load_w(1, 1);
  if (1 < nkb) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  auto step = [&](int kb, const int SW, const int SX) {
    // SW = kb % 3, SX = kb % 2 (literals after unrolling)
    if (kb + 1 < nkb) load_x(1 - SX, kb + 1);
    if (kb + 2 < nkb) load_w((SW + 2) % 3, kb + 2);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before the block's reads
    compute(SW, SX);
    // own copies of block kb+1 landed (only the 4 of block kb+2 may be outstanding); the
    // block's LDS reads were consumed by its MFMAs; then a bare barrier (no LDS fence, which
    // would wait for every outstanding copy)
    if (kb + 2 < nkb) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  };
  int kb = 0;
  for (; kb + 6 <= nkb; kb += 6) {
    step(kb, 0, 0);
    step(kb + 1, 1, 1);
    step(kb + 2, 2, 0);
    step(kb + 3, 0, 1);
    step(kb + 4, 1, 0);
    step(kb + 5, 2, 1);
  }
  for (; kb < nkb; ++kb) {
    const int r = kb % 6;
    if (r == 0) step(kb, 0, 0);
    else if (r == 1) step(kb, 1, 1);
    else if (r == 2) step(kb, 2, 0);
    else if (r == 3) step(kb, 0, 1);
    else step(kb, 1, 0);
  }
  unsigned long long t_loop = 0;
  if (a.stamps) t_loop = __builtin_amdgcn_s_memrealtime();

  // Restage as bf16 token rows of 256 bytes (16 chunks, chunk index XOR row % 16): rows
  // 0..63 in the weight slot 0, rows 64..127 in weight slot 1 (both free after the loop).
  {
    char* st = wm ? lds_w1 : lds_w0;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 32 * jj + r32;                     // token row within the wave's 64
          const int col = wn + 32 * ii + 8 * q + 4 * hl;     // first of 4 consecutive columns
          const f32x16& x = acc[ii][jj];
          const u32x2 v = {pack_bf16x2(x[4 * q + 0], x[4 * q + 1]), pack_bf16x2(x[4 * q + 2], x[4 * q + 3])};
          *reinterpret_cast<u32x2*>(st + row * 256 + (((col >> 3) ^ (row & 15)) << 4) + (col & 7) * 2) = v;
        }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int lin = it * 256 + tid;
    const int row = lin >> 4, ch = lin & 15;  // token row in the tile, 16-byte chunk in the row
    const char* st = row < 64 ? lds_w0 : lds_w1;
    const int rr = row & 63;
    const u32x4 v = *reinterpret_cast<const u32x4*>(st + rr * 256 + ((ch ^ (rr & 15)) << 4));
    if (row < xrows) {
      const int t = off + m0 + row;
      if (type == 0) {
        *(g_u32x4*)(a.h + (size_t)t * a.d_ff + nt * kTN + ch * 8) = v;
      } else {
        const int p = a.dst_slab[t], r = a.dst_row[t];
        if ((unsigned)p < (unsigned)a.P && (unsigned)r < (unsigned)a.out_rows[p])
          *(g_u32x4*)(a.out.p[p] + (size_t)r * a.d_model + nt * kTN + ch * 8) = v;
      }
    }
  }
  if (a.stamps && lane == 0) {
    const unsigned long long t_issued = __builtin_amdgcn_s_memrealtime();
    unsigned long long* sp = a.stamps + ((size_t)(a.stamp_base[type] + idx) * 4 + w) * 4;
    sp[0] = t_start;
    sp[1] = t_loop;
    sp[2] = t_issued;
    sp[3] = (unsigned long long)type;
  }
#endif
}

int moe_tiles(int rows, int n_cols) { return ((rows + kTM - 1) / kTM) * (n_cols / kTN); }

int moe_plan(const MoeShape& sh, int schedule, std::vector<MoeLaunch>* launches) {
  const int E = sh.E, W = (E + sh.experts_per_wave - 1) / sh.experts_per_wave;
  launches->clear();
  auto wave = [&](int w, int* e0, int* e1) {
    *e0 = w * sh.experts_per_wave;
    *e1 = std::min(E, *e0 + sh.experts_per_wave);
  };
  auto add = [&](int l1_wave, int l2_wave) {
    MoeLaunch L;
    L.l1_begin = L.l1_end = L.l2_begin = L.l2_end = 0;
    if (l1_wave >= 0) wave(l1_wave, &L.l1_begin, &L.l1_end);
    if (l2_wave >= 0) wave(l2_wave, &L.l2_begin, &L.l2_end);
    launches->push_back(L);
  };
  if (schedule == 0) {  // expert waves: Linear-1 of the wave, then its Linear-2
    for (int w = 0; w < W; ++w) {
      add(w, -1);
      add(-1, w);
    }
  } else {  // interleaved: Linear-2 of wave w together with Linear-1 of wave w+1
    add(0, -1);
    for (int w = 0; w < W; ++w) add(w + 1 < W ? w + 1 : -1, w);
  }
  return (int)launches->size();
}

int launch_moe(const MoeShape& sh, const MoeBuffers& buf, int schedule, hipStream_t stream) {
  std::vector<MoeLaunch> plan;
  moe_plan(sh, schedule, &plan);
  // run-wide stamp index: all Linear-1 tiles (expert order), then all Linear-2 tiles
  std::vector<int> pre1(sh.E + 1, 0), pre2(sh.E + 1, 0);
  for (int e = 0; e < sh.E; ++e) {
    pre1[e + 1] = pre1[e] + moe_tiles(sh.rows[e], sh.d_ff);
    pre2[e + 1] = pre2[e] + moe_tiles(sh.rows[e], sh.d_model);
  }
  for (const MoeLaunch& L : plan) {
    MoeLaunchArgs a = {};
    a.x = buf.x;
    a.w1 = buf.w1;
    a.w2 = buf.w2;
    a.h = buf.h;
    a.dst_slab = buf.dst_slab;
    a.dst_row = buf.dst_row;
    a.P = buf.P;
    for (int p = 0; p < buf.P; ++p) {
      a.out.p[p] = buf.out[p];
      a.out_rows[p] = buf.out_rows[p];
    }
    a.d_model = sh.d_model;
    a.d_ff = sh.d_ff;
    const int b[2] = {L.l1_begin, L.l2_begin}, en[2] = {L.l1_end, L.l2_end};
    for (int t = 0; t < 2; ++t) {
      a.n_exp[t] = en[t] - b[t];
      a.tile_pre[t][0] = 0;
      for (int q = 0; q < a.n_exp[t]; ++q) {
        const int e = b[t] + q;
        a.exp_id[t][q] = e;
        a.exp_off[t][q] = sh.offsets[e];
        a.exp_rows[t][q] = sh.rows[e];
        a.tile_pre[t][q + 1] = a.tile_pre[t][q] + moe_tiles(sh.rows[e], t ? sh.d_model : sh.d_ff);
      }
      a.n_tiles[t] = a.tile_pre[t][a.n_exp[t]];
    }
    a.mix = std::min(a.n_tiles[0] + a.n_tiles[1], kMixPerL1 * a.n_tiles[0]);
    a.stamps = buf.stamps;
    a.stamp_base[0] = pre1[b[0]];
    a.stamp_base[1] = pre1[sh.E] + pre2[b[1]];
    const int n = a.n_tiles[0] + a.n_tiles[1];
    if (n == 0) continue;
    hipLaunchKernelGGL(moe_gemm_kernel, dim3(n), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return XSTAGE_ERR_HIP;
  }
  return XSTAGE_OK;
}

}  // namespace xstage
