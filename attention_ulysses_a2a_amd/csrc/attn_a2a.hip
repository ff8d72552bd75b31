// Fused non-causal attention + Ulysses post-attention all-to-all epilogue for gfx950.
//
// Method: X-Stage explainer (gist.science, arXiv 2607.23264), technical summary,
// "Contributions", FlashAttention-A2A (piggybacking) item: the post-attention all-to-all is
// fused into FlashAttention; the owner of an output tile issues the stores of that tile
// toward its destinations and at once goes on with the next tile's query loop, which gives
// the stores time to drain; no wave is set aside for communication.  Here the P
// destinations are P receive buffers ("slabs") in local HBM.
//
// Work decomposition (one workgroup = NW waves = 32 NW query rows of one (batch, head); NW = 4,
// or 8 for launches that give every CU two 4-wave workgroups' worth of work without the
// one-round unit table):
//   * each wave owns 32 query rows and keeps them in registers as the B operand of
//     v_mfma_f32_32x32x16_bf16; scores are computed transposed, S^T = K Q^T, so that one
//     lane holds 32 keys of ONE query: the row max is a max over the lane's registers plus
//     one swap of wave halves, and the row sum never leaves the lane until the end;
//   * K and V blocks of 64 keys are staged in LDS (double-buffered, XOR-swizzled 16-byte
//     chunks) by all threads of the workgroup, and every wave reads them: 8 waves halve the
//     copies per query row; the next block's global loads are in flight while the current
//     block is computed;
//   * O^T = V^T P^T: P^T comes straight out of the score accumulators (converted to bf16),
//     and V^T operands are read from the natural [key][d] LDS layout with
//     ds_read_b64_tr_b16, the gfx950 transposing LDS read;
//   * epilogue: normalise, round to bf16, restage the tile through LDS and write each row's
//     16-byte chunks straight into the slab owning that sequence row.  The stores are not
//     waited on.
#include <algorithm>
#include <atomic>
#include <math.h>

#include "attn_a2a.hpp"
#include "common.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace xstage {

template <int D, int NW = 4>
struct AttnCfg {
  static constexpr int BM = 32 * NW;     // query rows per workgroup
  static constexpr int BN = 64;          // keys per block
  static constexpr int THREADS = 64 * NW;  // NW waves of 64
  static constexpr int KS = D / 16;     // 16-wide k-steps of the score product
  static constexpr int DT = D / 32;     // 32-wide tiles of the output dimension
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int ROWB = D * 2;    // bytes per staged row
  static constexpr int BLKB = BN * ROWB;
  static constexpr int NLD = BN * CH / THREADS;  // 16-byte loads per thread, per block and tensor
};

// XOR pattern applied to the 16-byte chunk index of LDS row `row`.  It makes three access
// patterns conflict-free: 16 consecutive rows reading the same logical chunk (score A
// operand), the transposing V reads (8 rows x 64 bytes per instruction) and full-row
// writes/reads (any permutation of a row's chunks).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  }
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  SlabTable slabs;
  int B, S, H, S_P;
  int n_mtiles;
  int n_units;       // workgroups: (b, h, m-tile) tiles x key splits
  int n_split;       // key-range splits per tile (1: no merge)
  int kvb_per_split; // 64-key blocks per split (uniform splits)
  int use_table;     // 1: per-workgroup (tile, split, key range) from the unit table
  // Input layout: n_src sequence shards of src_rows rows each (n_src = 1: q, k, v above),
  // rows of src_hs heads, this call's heads starting at src_h0.  Output layout: P slabs of
  // S_P rows, rows of dst_hs heads, this call's heads written from column dst_h0 on.
  int src_rows, src_hs, src_h0;
  int dst_hs, dst_h0;
  float c;           // |scale| * log2(e): scores are turned into base-2 logits
  uint32_t qflip;    // 0x80008000 for a negative scale: Q is negated on load
  void* partial;      // split partials: [tile][split][wave][chunk][64 lanes] (n_split > 1)
  int partial_bytes;  // bytes of the partial area (< 2^31)
  int pace_chunks;    // paced mode: chunks per output tile (a divisor of the stores per lane)
  uint32_t* counters;  // per-tile arrival counters, zero between launches (n_split > 1)
  unsigned long long* stamps;  // traced modes: [workgroup][wave][4] wall-clock ticks
  int clock_stamps;  // traced modes: entries 2, 3 hold shader-clock ticks at start / loop end
};

// Kernel modes.  kRun is the product path.  The traced modes record, per wave, the
// wall-clock time at start, at the end of the key loop, after the last epilogue store was
// issued and (kCoupled) after those stores completed: kTraced changes nothing else;
// kCoupled makes every wave wait for its stores before it ends (the completion-coupled
// counterfactual: the issuer blocks until its stores are visible); kNoStore issues no output
// store at all (the unbounded-asynchronous bound: stores cost nothing; nothing is written).
// kPaced is the paced persistent mode: each workgroup runs several tiles in turn, keeps the
// finished tile's rows in LDS and issues them in pace_chunks chunks, one at the start of each
// of the next tile's first key-loop iterations (two 64-key blocks each), so that the store
// burst is spread over the next tile's compute; the last tile's rows are issued at the end.
// Splits are not used (one unit per tile), and the results equal the unsplit product path's.
enum AttnMode { kRun = 0, kTraced = 1, kCoupled = 2, kNoStore = 3, kPaced = kAttnModePaced };
// Host-side launch mode: kTraced with shader-clock stamps in entries 2 and 3.
constexpr int kTracedClock = 4;

// A pointer read through a wave-uniform index, kept in scalar registers.
__device__ __forceinline__ uint16_t* uniform_ptr(uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<uint16_t*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  return uniform_ptr(const_cast<uint16_t*>(p));
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

struct NoSrc {};

// Where q, k, v come from: kPlain = contiguous [B, S, H, D] tensors (a.q, a.k, a.v);
// kShards = Q, K and V read in place from P sequence shards (the SrcTable); kShardQ = Q from
// the shards, K and V from contiguous [B, S, H, D] tensors (a.k, a.v).
enum SrcMode { kPlain = 0, kShards = 1, kShardQ = 2 };

// NW = 4: two workgroups per CU (two waves per SIMD); NW = 8: one workgroup per CU, also two
// waves per SIMD; the paced mode holds 96 KiB of LDS, one 4-wave workgroup per CU.
template <int D, int MODE, int SRC, int NW = 4>
__global__ __launch_bounds__(64 * NW, (MODE == kPaced || NW == 8) ? 1 : 2) void attn_a2a_kernel(const AttnArgs a, const UnitTable tab,
                                                          const std::conditional_t<SRC != kPlain, SrcTable, NoSrc> src) {
  // The body names device-only types (the buffer resource), which the host pass of a
  // template cannot instantiate; the host pass only needs the launch signature.
#if defined(__HIP_DEVICE_COMPILE__)
  using C = AttnCfg<D, NW>;
  static_assert(NW == 4 || (NW == 8 && MODE != kPaced), "4-wave workgroups, or 8 outside the paced mode");
  // K0 K1 V0 V1 as four LDS objects rather than one array: the compiler then knows that the
  // reads of one slot do not alias the asynchronous global->LDS copies into another, and
  // does not wait for those copies before every read.  Slots are named by the byte offsets
  // they would have in one array (compile-time constants after inlining).
  __shared__ __attribute__((aligned(16))) char lds_k0[C::BLKB];
  __shared__ __attribute__((aligned(16))) char lds_k1[C::BLKB];
  __shared__ __attribute__((aligned(16))) char lds_v0[C::BLKB];
  __shared__ __attribute__((aligned(16))) char lds_v1[C::BLKB];
  auto sp = [&](int slot_byte) -> char* {
    return slot_byte < C::BLKB ? lds_k0 : slot_byte < 2 * C::BLKB ? lds_k1 : slot_byte < 3 * C::BLKB ? lds_v0 : lds_v1;
  };
  constexpr bool kPace = MODE == kPaced;
  constexpr bool kStamped = MODE == kTraced || MODE == kCoupled || MODE == kNoStore;
  // Paced mode: the finished tile's rows (4 waves x 32 rows, restaged as in the epilogue)
  // wait here while the next tile's key loop runs.
  __shared__ __attribute__((aligned(16))) char lds_out[kPace ? NW * 32 * C::ROWB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;  // half of the wave
  // Traced modes: each stamp is stored (by lane 0) as soon as it is taken, so that no
  // stamp stays live across the key loop and the merge.
  auto stamp = [&](int slot, unsigned long long v) {
    if constexpr (kStamped) {
      if (lane == 0) a.stamps[((size_t)blockIdx.x * NW + w) * 4 + slot] = v;
    }
  };
  // Entries 2 and 3 start at 0: a workgroup that stores no output (a split that does not
  // merge, rows past S, the no-store mode) leaves them so.
  if constexpr (kStamped) {
    stamp(0, __builtin_amdgcn_s_memrealtime());
    if (a.clock_stamps) {
      stamp(2, __builtin_amdgcn_s_memtime());
    } else {
      stamp(2, 0);
      stamp(3, 0);
    }
  }

  const int nkv = (a.S + C::BN - 1) / C::BN;

  // Paced mode: the tile whose rows wait in lds_out (wave-uniform; pend_row0 < 0: none) and
  // the next of its chunks to issue.  issue_pending(n) issues chunks pend_next .. n-1: each
  // is stores [k * per, (k + 1) * per) of the wave's 8 (D = 128) or 4 (D = 64) 16-byte
  // stores per lane, every row to the slab that owns it.
  constexpr int NST = 32 * C::CH / 64;  // 16-byte stores per lane for a wave's 32 rows
  int pend_row0 = -1, pend_b = 0, pend_h = 0, pend_next = 0;
  auto issue_pending = [&](int upto) {
    if constexpr (kPace) {
      if (pend_row0 < 0) return;
      const char* const pst = lds_out + __builtin_amdgcn_readfirstlane(w) * 32 * C::ROWB;
      const int per = NST / a.pace_chunks;
      const int p_lo = pend_row0 / a.S_P, p_hi = min(pend_row0 + 31, a.S - 1) / a.S_P;
      for (; pend_next < upto; ++pend_next) {
        for (int i = pend_next * per; i < (pend_next + 1) * per; ++i) {
          const int lin = i * 64 + lane;
          const int row = lin / C::CH, ch = lin % C::CH;
          const u32x4 val = *reinterpret_cast<const u32x4*>(pst + row * C::ROWB + ((ch ^ swz<D>(row)) << 4));
          const int s_row = pend_row0 + row;
          const int p = s_row / a.S_P;
          const int r = s_row - p * a.S_P;
          const uint32_t off = (((uint32_t)pend_b * a.S_P + r) * a.dst_hs + a.dst_h0 + pend_h) * D + ch * 8;
          // slab pointers are read at wave-uniform indices only
          for (int pp = p_lo; pp <= p_hi; ++pp)
            if (s_row < a.S && p == pp) *(g_u32x4*)(uniform_ptr(a.slabs.p[pp]) + off) = val;
        }
      }
    }
  };

  // One pass per unit; the paced mode runs units blockIdx.x, blockIdx.x + gridDim.x, ...
  for (int unit = blockIdx.x;; unit += gridDim.x) {
  if constexpr (kPace) {
    if (unit != (int)blockIdx.x) __syncthreads();  // the previous unit's LDS reads are done
  }
  // This workgroup's tile, split and key-block range [j0, j1).  One-round launches take
  // them from the unit table (kernel arguments: one scalar load, issued with the others).
  // Otherwise the order is XCD-aware: workgroup i runs on XCD i % 8; each XCD gets a
  // contiguous range of (b, h, m-tile) units so that one head's K/V stays in one XCD's L2,
  // and the splits are uniform.
  int tile, split, j0, j1;
  {
    const int i = unit;
    const uint32_t e = tab.e[i < kUnitTableCap ? i : 0];
    if (a.use_table) {
      tile = e & 1023;
      split = (e >> 10) & 15;
      j0 = (e >> 14) & 511;
      j1 = e >> 23;
    } else {
      const int n = a.n_units;
      const int q8 = n >> 3, r8 = n & 7, xcd = i & 7, slot = i >> 3;
      const int L = xcd < r8 ? xcd * (q8 + 1) + slot : r8 * (q8 + 1) + (xcd - r8) * q8 + slot;
      tile = L / a.n_split;
      split = L - tile * a.n_split;
      j0 = split * a.kvb_per_split;
      j1 = min(j0 + a.kvb_per_split, nkv);
    }
  }
  const int mt = tile % a.n_mtiles;
  const int bh = tile / a.n_mtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int m0 = mt * C::BM;
  const int S = a.S;
  // Q rows: rq elements apart; qhead0 = offset of (b, first row of a shard, this head) within
  // a shard (the whole tensor when it is not sharded).  K/V rows: the same unless kShardQ.
  const uint32_t rq = (uint32_t)a.src_hs * D;
  const uint32_t qhead0 = ((uint32_t)b * a.src_rows * a.src_hs + a.src_h0 + h) * D;
  const uint32_t rs = SRC == kShardQ ? (uint32_t)a.H * D : rq;  // elements between K/V rows
  const uint32_t head0 = SRC == kShardQ ? ((uint32_t)b * S * a.H + h) * D : qhead0;
  const int kv_rows = SRC == kShardQ ? S : a.src_rows;  // rows per K/V buffer

  // Q fragment (B operand of the score MFMA): lane holds query (lane & 31), d = 16ks + 8*hl + 0..7
  const int wave_u32 = __builtin_amdgcn_readfirstlane(w);
  bf16x8 qf[C::KS];
  if constexpr (SRC == kPlain) {
    const int qrow = m0 + w * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < S) x = *reinterpret_cast<const u32x4*>(a.q + qhead0 + (uint32_t)qrow * rq + ks * 16 + hl * 8);
      x ^= a.qflip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  } else {
    // Q from the sequence shards.  The shard pointer is not a per-lane load: when a shard
    // holds at least 32 rows, a wave's rows lie in at most two shards, whose pointers are
    // read as wave-uniform scalar values.  The loads are branch-free (a row past S loads row
    // S - 1 and is zeroed by a select) and global rather than flat accesses, so neither they
    // nor the pointer fetch are waited on before the first K/V copies are issued.
    const int qrow = m0 + w * 32 + (lane & 31);
    const bool q_ok = qrow < S;
    const int qr = q_ok ? qrow : S - 1;
    const int p = qr / a.src_rows;
    const int r = qr - p * a.src_rows;
    const uint16_t* qb;
    if (a.src_rows >= 32) {
      const int p_lo = __builtin_amdgcn_readfirstlane(min(m0 + wave_u32 * 32, S - 1) / a.src_rows);
      const int p_hi = __builtin_amdgcn_readfirstlane(min(p_lo + 1, S / a.src_rows - 1));
      const uint16_t* const b_lo = uniform_ptr(src.q[p_lo]);
      const uint16_t* const b_hi = uniform_ptr(src.q[p_hi]);
      qb = (p == p_lo ? b_lo : b_hi) + qhead0;
    } else {
      qb = src.q[p] + qhead0;
    }
    const uint16_t* const qp = qb + (uint32_t)r * rq + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = *(const g_u32x4*)(qp + ks * 16);
      x = q_ok ? x : u32x4{0u, 0u, 0u, 0u};
      x ^= a.qflip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // K/V blocks go from global memory straight into LDS (buffer_load_dwordx4 ... lds: no
  // registers).  One instruction of wave w fills the 1 KiB LDS segment (i*NW + w) of a
  // block, lane by lane, so each lane fetches the global chunk that belongs at its LDS slot
  // under the swizzle.  The range check covers the per-lane offset (the scalar offset
  // stays 0), and a resource ends where the head's S rows end: rows past the end of the
  // sequence read as zeros — no clamping, no branches.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t head_bytes = (uint32_t)kv_rows * rs * 2u;  // one K/V buffer's rows of this head
  auto make_rsrc = [&](const uint16_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + head0), (short)0, (int)head_bytes, 0x00020000);
  };
  // K/V in one buffer (kPlain, kShardQ): every block gets a resource that starts at its
  // first row and spans the rows left in the head (wave-uniform scalar arithmetic), so the
  // per-lane offsets stay fixed through the loop and the range check still zeroes rows past
  // the end.  K/V in shards (kShards): the resources are built from the shard pointers
  // (kernel arguments, scalar loads) and the block offset is in the per-lane offset.
  const uint16_t* const kbase = SRC != kShards ? a.k + head0 : nullptr;
  const uint16_t* const vbase = SRC != kShards ? a.v + head0 : nullptr;
  // Shard cursors (kShards): the shard holding the K (V) stream's current block; blocks only
  // move forward, from j0.  The cursor is an index, and each load builds its buffer resource
  // from the shard pointer read at that index made wave-uniform (readfirstlane): a resource
  // carried across the loop as a value is not provably uniform to the compiler, which then
  // wraps every copy in a loop over the lanes' resources.
  int k_p = 0, v_p = 0;
  if constexpr (SRC == kShards) k_p = v_p = j0 * C::BN / a.src_rows;
  // Byte offset of this lane's chunk from the block's first key, for its first load; load i
  // of the lane is RSTEP rows further on (the swizzle repeats every 16 rows, so the chunk
  // column is the same): one per-lane register, the rest is a wave-uniform offset.
  constexpr int RSTEP = NW * 64 / C::CH;
  static_assert(RSTEP % 16 == 0, "the swizzle must repeat between a lane's loads");
  const int ld_row = (w * 64 + lane) / C::CH;
  const uint32_t ld_voff = ((uint32_t)ld_row * rs + (uint32_t)((((w * 64 + lane) % C::CH) ^ swz<D>(ld_row)) * 8)) * 2u;
  const uint32_t ld_step = (uint32_t)RSTEP * rs * 2u;
  // base: kbase or vbase (unused with shards: the slot names the stream).
  auto dload = [&](const uint16_t* base, int slot_byte, int n0) {
    if constexpr (SRC != kShards) {
      const uint32_t boff = (uint32_t)n0 * rs * 2u;  // < head_bytes: n0 < S
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(base + (size_t)n0 * rs), (short)0, (int)(head_bytes - boff), 0x00020000);
#pragma unroll
      for (int i = 0; i < C::NLD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(sp(slot_byte) + (i * NW + wu) * 1024), 16,
            ld_voff + i * ld_step, 0, 0, 0);
    } else {
      // The stream's cursor (K or V: which one is fixed by the slot, a constant after
      // inlining) names the shard holding its current block.  A block inside that shard is
      // one resource; the rows past S of the last block lie beyond the last shard's range
      // and read as zeros.  A block reaching into the next shard(s) loads from shards
      // p0 .. p1, each lane from exactly one of them (every LDS chunk written once), and
      // moves the cursor to the shard of its last row.
      const bool is_k = slot_byte < 2 * C::BLKB;
      int& cur_p = is_k ? k_p : v_p;
      const uint16_t* const* tbl = is_k ? src.k : src.v;
      const int cp = __builtin_amdgcn_readfirstlane(cur_p);
      const int cur_lo = cp * a.src_rows;
      const int last = min(n0 + C::BN, S) - 1;
      if (last < cur_lo + a.src_rows) {
        const __amdgpu_buffer_rsrc_t cur_r = make_rsrc(uniform_ptr(tbl[cp]));
        const uint32_t boff = (uint32_t)(n0 - cur_lo) * rs * 2u;
#pragma unroll
        for (int i = 0; i < C::NLD; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              cur_r, (__attribute__((address_space(3))) void*)(sp(slot_byte) + (i * NW + wu) * 1024), 16,
              ld_voff + (i * ld_step + boff), 0, 0, 0);
      } else {
        const int p0 = __builtin_amdgcn_readfirstlane(n0 / a.src_rows);
        const int p1 = __builtin_amdgcn_readfirstlane(last / a.src_rows);
        for (int p = p0; p <= p1; ++p) {
          const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr(tbl[__builtin_amdgcn_readfirstlane(p)]));
          const int lo = p * a.src_rows - n0;                        // first block row in shard p
          const int hi = p == p1 ? C::BN : (p + 1) * a.src_rows - n0;  // one past its last
          const uint32_t boff = (uint32_t)(n0 - p * a.src_rows) * rs * 2u;
#pragma unroll
          for (int i = 0; i < C::NLD; ++i) {
            const int row = ld_row + i * RSTEP;
            if (row >= lo && row < hi)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  r, (__attribute__((address_space(3))) void*)(sp(slot_byte) + (i * NW + wu) * 1024), 16,
                  ld_voff + (i * ld_step + boff), 0, 0, 0);
          }
        }
        cur_p = p1;
      }
    }
  };

  // LDS slots: K at byte 0 and BLKB, V at 2*BLKB and 3*BLKB.  Every per-lane read address
  // below is a fixed per-lane base plus a compile-time offset (slot, tile), so the reads
  // carry their offsets as immediates.
  constexpr int KSLOT0 = 0, VSLOT0 = 2 * C::BLKB;
  const int krow = lane & 31;
  const int kswz = swz<D>(krow);
  int kaddr[C::KS];  // score A operand: row krow, logical chunk 2ks + hl
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) kaddr[ks] = krow * C::ROWB + (((2 * ks + hl) ^ kswz) << 4);
  // transposing V reads: lane group g = lane/16, s4 = lane%16
  int vaddr[C::DT][2];
  {
    const int g = lane >> 4, s4 = lane & 15;
    const int vrow1 = 4 * (g >> 1) + (s4 >> 2);
    const int vrow2 = vrow1 + 8;
    const int vc0 = 2 * (g & 1) + ((s4 & 3) >> 1);  // chunk within a 32-wide d tile
    const int vbyte = (s4 & 1) * 8;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      vaddr[dt][0] = vrow1 * C::ROWB + (((4 * dt + vc0) ^ swz<D>(vrow1)) << 4) + vbyte;
      vaddr[dt][1] = vrow2 * C::ROWB + (((4 * dt + vc0) ^ swz<D>(vrow2)) << 4) + vbyte;
    }
  }

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  // c = |scale| log2(e), kept >= FLT_MIN so that a masked score (-inf) * c stays -inf; for
  // scale = 0 every real score times FLT_MIN is below 2^-100 in magnitude, so all weights
  // are exp2(0) = 1 in fp32 exactly as with c = 0.
  const float c = __builtin_fmaxf(a.c, 1.17549435e-38f);

  // S^T = K Q^T for one 64-key block held in K slot `ks_byte` (two 32-key tiles)
  auto qk = [&](int ks_byte, f32x16* st) {
    st[0] = f32x16{};
    st[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sp(ks_byte) + kaddr[ks] + t * 32 * C::ROWB);
        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[t], 0, 0, 0);
      }
    }
  };

  // Online softmax, base 2 with the scale folded into c, split in two steps so that the
  // exponentials of block j can share one basic block with the score MFMAs of block j+1:
  //  * rescale(): block max; the running max is only raised when the block exceeds it by
  //    more than kLazy (log2 units), so weights stay below 2^kLazy (exact after the final
  //    division) and the O rescale, one multiply per accumulator, is skipped for most blocks;
  //  * exp_pack(): weights, bf16 packing into the B operand of the PV MFMA, and the row sum
  //    of the packed (bf16) weights, i.e. of exactly the weights the PV product uses.
  // Keys past S exist only in the very last block (`tail`): their scores become -inf, so
  // they drop out of the max and get weight exp2(-inf) = 0 (c > 0 always, see above).
  constexpr float kLazy = 8.0f;
  auto key_of = [&](int n0, int t, int r) { return n0 + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3); };
  auto mask_tail = [&](f32x16* st, int n0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key_of(n0, t, r) >= S) st[t][r] = -INFINITY;
  };
  auto blockmax = [&](const f32x16* st) {
    float mx = __builtin_fmaxf(st[0][0], st[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, st[0][r]), st[0][r + 1]);
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, st[1][r]), st[1][r + 1]);
    return max_with_partner32(mx) * c;
  };
  auto rescale_to = [&](float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
  };
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  auto exp_pack = [&](f32x16* st, bf16x8* pb) {
    const float neg_m = -m_run;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[t][r], c, neg_m));
    // The row sum accumulates straight into l_run (one chain of 16 dot products: no
    // zero-initialised partial sums to add up afterwards).
    float l = l_run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& x = st[q >> 1];
      const int r0 = (q & 1) * 8;
      // (each packed word goes to the dot product as its own value: feeding it as an element
      // of the 4-word vector has been miscompiled into four dot products of the first word)
      const uint32_t w0 = pack_bf16x2(x[r0 + 0], x[r0 + 1]), w1 = pack_bf16x2(x[r0 + 2], x[r0 + 3]);
      const uint32_t w2 = pack_bf16x2(x[r0 + 4], x[r0 + 5]), w3 = pack_bf16x2(x[r0 + 6], x[r0 + 7]);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, l, false);
      pb[q] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
    }
    l_run = l;
  };

  // O^T += V^T P^T, four 16-key steps; k-step t uses pb[t] = registers 8*(t&1)..+7 of the
  // score tile t>>1, i.e. keys 16t + 8*(jj/4) + 4*hl + jj%4 for slot jj.
  auto pv = [&](int vs_byte, const bf16x8* pb) {
#pragma unroll
    for (int t = 0; t < C::BN / 16; ++t) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const bf16x4 lo = lds_read_tr(sp(vs_byte) + vaddr[dt][0] + 16 * t * C::ROWB);
        const bf16x4 hi = lds_read_tr(sp(vs_byte) + vaddr[dt][1] + 16 * t * C::ROWB);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t], o[dt], 0, 0, 0);
      }
    }
  };

  // Software pipeline over the split's key blocks [j0, j1).  Step j holds the raw scores
  // of block j (and their max) in registers and, in LDS, K of block j+1 and V of block j.
  // It starts the loads of K(j+2) and V(j+1) into the slots freed by step j-1, settles the
  // running max, computes the scores of block j+1 (MFMA) alongside the exponentials of
  // block j (VALU), then O += V(j)^T P(j)^T alongside the max of block j+1, waits for its
  // loads and meets the other waves at the barrier.  Slot parity alternates with j - j0;
  // the loop is unrolled by two so it is static.  Rows past S (zeros) are only in the last
  // block, handled after the loop: there the max is recomputed with those keys at -inf.
  f32x16 s_a[2], s_b[2];
  bf16x8 pb[4];
  float mx;
  dload(kbase, KSLOT0, j0 * C::BN);
  dload(vbase, VSLOT0, j0 * C::BN);
  if (j0 + 1 < j1) dload(kbase, KSLOT0 + C::BLKB, (j0 + 1) * C::BN);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(KSLOT0, s_a);
  mx = blockmax(s_a);
  __syncthreads();  // K slot 0 is refilled by the first step

  // PAR = (j - j0) & 1 is a literal at every call, so after inlining the slot offsets fold.
  auto step = [&](int j, const int PAR, f32x16* s_cur, f32x16* s_nxt) {
    if (j + 2 < j1) dload(kbase, KSLOT0 + PAR * C::BLKB, (j + 2) * C::BN);
    dload(vbase, VSLOT0 + (1 - PAR) * C::BLKB, (j + 1) * C::BN);
    rescale_to(mx);
    qk(KSLOT0 + (1 - PAR) * C::BLKB, s_nxt);
    exp_pack(s_cur, pb);
    pv(VSLOT0 + PAR * C::BLKB, pb);
    mx = blockmax(s_nxt);
    // Interleave: score MFMAs with their operand reads kept 4 ahead and the exponentials;
    // the slots of the last four score MFMAs already issue the first 8 transposing V reads,
    // which then run 4 MFMAs ahead of the PV MFMAs, interleaved with the next max.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 4 < 2 * C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
#pragma unroll
    for (int i = 0; i < 4 * C::DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 4 < 4 * C::DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int j = j0;
  for (; j + 2 < j1; j += 2) {
    if constexpr (kPace) issue_pending(min(pend_next + 1, a.pace_chunks));
    step(j, 0, s_a, s_b);
    step(j + 1, 1, s_b, s_a);
  }
  const bool tail = j1 * C::BN > S;
  auto last_block = [&](int jl, f32x16* st, int vs_byte) {
    if (tail) {
      mask_tail(st, jl * C::BN);
      mx = blockmax(st);
    }
    rescale_to(mx);
    exp_pack(st, pb);
    pv(vs_byte, pb);
  };
  if (j + 1 < j1) {
    step(j, 0, s_a, s_b);
    last_block(j + 1, s_b, VSLOT0 + C::BLKB);
  } else {
    last_block(j, s_a, VSLOT0);
  }

  if constexpr (kStamped) {
    stamp(1, __builtin_amdgcn_s_memrealtime());
    if (a.clock_stamps) stamp(3, __builtin_amdgcn_s_memtime());
  }

  // ---- key-range splits: every split stores its partial (O, m, l); the last to arrive
  // merges them (rescaling by exp2(m_s - m)) and runs the epilogue for the tile.
  if (!kPace && a.n_split > 1) {
    __shared__ int last_flag;
    // One record per (tile, split, wave), in lane-major 16-byte chunks: the lane's
    // unnormalised O rounded to fp16 (two chunks per 32-wide d tile, accumulator registers
    // 0..7 and 8..15), then (m, l, 2^E) in fp32.  16-bit values halve the bytes written here
    // and read back by the merge, both of which sit on the tail of the kernel; fp16's 11-bit
    // significand keeps each partial within 2^-11 of itself (bf16 would allow 2^-8 + 2^-9 per
    // output, more than a 1e-2 bound leaves beside the output's own bf16 rounding once |O|
    // reaches 2).  A lane whose largest |O| reaches 2^15 stores O * 2^-E instead, E >= 1
    // chosen so that the values stay below 2^15 (fp16 overflows at 65520); otherwise E = 0.
    // Values that fall below fp16's normal range lose at most 2^-25 absolutely, and the merged
    // sum of weights L is at least 1, so the output loses no more.
    constexpr int OCH = 2 * C::DT;
    constexpr int PREC = OCH + 1;
    // The workspace is ordinary device memory, cached in each XCD's own L2, and the splits of a
    // tile may run on different XCDs.  Every access to a record therefore has device scope
    // (sc1): stores write through the local L2 to the device's coherence point, loads are
    // served from there, never from a stale local line.  Ordering (see the arrival below):
    // a wave's record stores complete before the barrier, the barrier before the arrival
    // count, the count before the last arriver's loads; no cache write-back or invalidate.
    constexpr int kDeviceScope = 16;  // cache policy bits: sc1
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(a.partial, (short)0, a.partial_bytes, 0x00020000);
    auto rec = [&](int sp) { return (((uint32_t)(tile * a.n_split + sp) * (uint32_t)NW + (uint32_t)w) * PREC * 64u + (uint32_t)lane) * 16u; };
    u32x4 own[OCH];  // this split's record, kept for the merge should it arrive last
    float own_unscale;
    {
      float mx = 0.f;  // largest |O| of the lane (NaN ignored)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(o[dt][e]));
      // E = exponent of mx beyond 2^15 (mx < 2^(15 + E)); an infinite mx takes the largest
      // finite one's E, so that the finite values beside it keep their place
      int ex = (mx == __builtin_inff() ? 128 : __builtin_amdgcn_frexp_expf(mx)) - 15;
      ex = ex < 0 ? 0 : ex;
      own_unscale = __builtin_ldexpf(1.0f, ex);
      const uint32_t r = rec(split);
      const bool scaled = __builtin_amdgcn_ballot_w64(ex > 0) != 0;  // wave-uniform
      const float sc = __builtin_ldexpf(1.0f, -ex);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& x = o[dt];
          const int e0 = 8 * hh;
          own[2 * dt + hh] =
              scaled ? u32x4{pack_f16x2(x[e0 + 0] * sc, x[e0 + 1] * sc), pack_f16x2(x[e0 + 2] * sc, x[e0 + 3] * sc),
                             pack_f16x2(x[e0 + 4] * sc, x[e0 + 5] * sc), pack_f16x2(x[e0 + 6] * sc, x[e0 + 7] * sc)}
                     : u32x4{pack_f16x2(x[e0 + 0], x[e0 + 1]), pack_f16x2(x[e0 + 2], x[e0 + 3]),
                             pack_f16x2(x[e0 + 4], x[e0 + 5]), pack_f16x2(x[e0 + 6], x[e0 + 7])};
          __builtin_amdgcn_raw_buffer_store_b128(own[2 * dt + hh], prs, r + (2 * dt + hh) * 1024u, 0, kDeviceScope);
        }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{m_run, l_run, own_unscale, 0.f}), prs,
                                             r + OCH * 1024u, 0, kDeviceScope);
    }
    const f32x4 own_ml = {m_run, l_run, own_unscale, 0.f};
    // Wait until this wave's record stores have completed (device-scope stores complete once
    // they reach the coherence point); the barrier then orders all four waves' records before
    // the arrival count, an agent-scope atomic performed at the coherence point.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int is_last = prev == (uint32_t)(a.n_split - 1);
      if (is_last) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = is_last;
    }
    __syncthreads();
    if (!last_flag) return;
    // The last arriver saw every other split's count, each issued after that split's records
    // had completed; its device-scope loads, issued after the count returned, read them.
    // Merge in split order (own partial included, as the bits of its record), so the result
    // does not depend on which split arrived last.  The records of NB splits are requested
    // together and folded in with a running-max rescale, so that up to NB splits cost one
    // round trip to the coherence point.
    constexpr int NB = 4;
    float m_acc = -INFINITY, l_acc = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
    for (int s0 = 0; s0 < a.n_split; s0 += NB) {
      u32x4 ob[NB][OCH];
      f32x4 ml[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (s0 + i == split) {  // own record: the same bits, from registers
          ml[i] = own_ml;
#pragma unroll
          for (int ch = 0; ch < OCH; ++ch) ob[i][ch] = own[ch];
        } else if (s0 + i < a.n_split) {
          const uint32_t r = rec(s0 + i);
          ml[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, r + OCH * 1024u, 0, kDeviceScope));
#pragma unroll
          for (int ch = 0; ch < OCH; ++ch) ob[i][ch] = __builtin_amdgcn_raw_buffer_load_b128(prs, r + ch * 1024u, 0, kDeviceScope);
        } else {
          ml[i] = f32x4{-INFINITY, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ch = 0; ch < OCH; ++ch) ob[i][ch] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      float m_new = m_acc;
#pragma unroll
      for (int i = 0; i < NB; ++i) m_new = __builtin_fmaxf(m_new, ml[i][0]);
      const float fo = m_acc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_acc - m_new);
      l_acc *= fo;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] *= fo;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float f = __builtin_amdgcn_exp2f(ml[i][0] - m_new);
        l_acc += ml[i][1] * f;
        const float fs = f * ml[i][2];  // the record holds O * 2^-E; ml[i][2] = 2^E (1 unless scaled)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              // copied to a scalar first: this compiler reads element 0 for a bit cast applied
              // to a vector element directly, whatever the index
              const uint32_t wv = ob[i][2 * dt + hh][k];
              const f16x2 hv = __builtin_bit_cast(f16x2, wv);
              o[dt][8 * hh + 2 * k] += (float)hv[0] * fs;
              o[dt][8 * hh + 2 * k + 1] += (float)hv[1] * fs;
            }
      }
      m_acc = m_new;
    }
    m_run = m_acc;
    l_run = l_acc;
  }

  // ---- epilogue: normalise, bf16, restage per wave, store rows into their slabs ----------
  const float inv = 1.0f / sum_with_partner32(l_run);
  // wave-private [32][D] restage area: 4 waves use the K slots (no wave reads them after the
  // loop's last barrier); 8 waves need the V slots too, which the other waves may still be
  // reading in the last block's PV product until this barrier; paced mode: in lds_out, once
  // the previous tile's rows have all been issued from there
  if constexpr (kPace) issue_pending(a.pace_chunks);
  if constexpr (NW > 4) __syncthreads();
  char* stage = kPace ? lds_out + w * 32 * C::ROWB
                      : (NW > 4 ? sp((w >> 1) * C::BLKB) : (w < 2 ? lds_k0 : lds_k1)) + (w & 1) * 32 * C::ROWB;
  {
    const int n = lane & 31;
    const int sw = swz<D>(n);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const u32x2 val = {pack_bf16x2(o[dt][4 * rq + 0] * inv, o[dt][4 * rq + 1] * inv),
                           pack_bf16x2(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv)};
        const int ch = 4 * dt + rq;
        *reinterpret_cast<u32x2*>(stage + n * C::ROWB + ((ch ^ sw) << 4) + hl * 8) = val;
      }
  }
  __builtin_amdgcn_wave_barrier();

  if constexpr (kPace) {
    const int row0 = m0 + wu * 32;
    pend_row0 = row0 < S ? row0 : -1;
    pend_b = b;
    pend_h = h;
    pend_next = 0;
  } else {
  // Destination of each restaged row.  The wave's 32 rows are consecutive sequence rows, so
  // unless a slab holds fewer than 32 rows they touch at most two slabs, whose pointers are
  // read once as wave-uniform (scalar) values: the stores then issue back to back with no
  // wait between them.  Tiny slabs (fewer than 32 rows) take a per-row-pointer path.
  // wu: this wave's index as a wave-uniform value (defined with the loads above)
  const int row0 = m0 + wu * 32;
  if (row0 >= S || MODE == kNoStore) return;
  const int rowN = min(row0 + 31, S - 1);
  const int p_lo = row0 / a.S_P, p_hi = rowN / a.S_P;
  const bool full = row0 + 31 < S;
  if (p_hi - p_lo <= 1) {
    uint16_t* const base_lo = uniform_ptr(a.slabs.p[p_lo]);
    uint16_t* const base_hi = uniform_ptr(a.slabs.p[p_hi]);
    g_u32x4* dst[NST];
    u32x4 val[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int lin = i * 64 + lane;
      const int row = lin / C::CH, ch = lin % C::CH;
      val[i] = *reinterpret_cast<const u32x4*>(stage + row * C::ROWB + ((ch ^ swz<D>(row)) << 4));
      const int s_row = row0 + row;
      const bool hi = s_row >= p_hi * a.S_P;
      const int r = s_row - (hi ? p_hi : p_lo) * a.S_P;
      const uint32_t off = (((uint32_t)b * a.S_P + r) * a.dst_hs + a.dst_h0 + h) * D + ch * 8;
      dst[i] = (g_u32x4*)((hi ? base_hi : base_lo) + off);
    }
    if (full) {
#pragma unroll
      for (int i = 0; i < NST; ++i) *dst[i] = val[i];
    } else {
#pragma unroll
      for (int i = 0; i < NST; ++i)
        if (row0 + (i * 64 + lane) / C::CH < S) *dst[i] = val[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int lin = i * 64 + lane;
      const int row = lin / C::CH, ch = lin % C::CH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * C::ROWB + ((ch ^ swz<D>(row)) << 4));
      const int s_row = row0 + row;
      if (s_row < S) {
        const int p = s_row / a.S_P;
        const int r = s_row - p * a.S_P;
        const uint32_t off = (((uint32_t)b * a.S_P + r) * a.dst_hs + a.dst_h0 + h) * D + ch * 8;
        *reinterpret_cast<u32x4*>(a.slabs.p[p] + off) = val;
      }
    }
  }
  if constexpr (kStamped) {
    const unsigned long long t_issued = __builtin_amdgcn_s_memrealtime();
    unsigned long long t_done = 0;
    if constexpr (MODE == kCoupled) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      t_done = __builtin_amdgcn_s_memrealtime();
    }
    if (!a.clock_stamps) {
      stamp(2, t_issued);
      stamp(3, t_done);
    }
  }
  }  // end of the non-paced epilogue
  if constexpr (!kPace) {
    break;
  } else {
    if (unit + (int)gridDim.x >= a.n_units) break;
  }
  }  // units
  // paced mode: the last tile's rows
  if constexpr (kPace) issue_pending(a.pace_chunks);
#endif
}

// Workgroups of the paced kernel that fit on one CU at once (LDS-bound: one), cached per D
// (it does not depend on the device); 0 if the query fails.
template <int D>
static int paced_per_cu() {
  static std::atomic<int> per_cu{0};
  int n = per_cu.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_a2a_kernel<D, kPaced, kPlain>, AttnCfg<D>::THREADS, 0) !=
            hipSuccess ||
        n < 1)
      return 0;
    per_cu.store(n, std::memory_order_relaxed);
  }
  return n;
}

// One launch: the key-split plan (counted in 128-row tiles, as the split cost model and the
// workspace layout count them) and the workgroup width.
struct AttnLaunch {
  SplitPlan plan;
  int nw = 4;       // waves per workgroup; query rows per workgroup = 32 nw
  int n_tiles = 0;  // (b, h, 32nw-row tile) units
  int n_units = 0;  // workgroups = n_tiles * n_split
  size_t used = 0;  // split workspace bytes the plan uses
};

// force_split > 0: exactly that many splits (false if impossible or the workspace is too
// small); otherwise the model's plan for ws_bytes of workspace.
static bool attn_launch(int B, int S, int H, int D, unsigned long long ws_bytes, int force_split, bool allow_wide,
                        AttnLaunch* L) {
  const int n_tiles4 = B * H * ((S + 127) / 128);
  const int nkv = (S + 63) / 64;
  if (force_split > 0) {
    if (!plan_forced(n_tiles4, nkv, D, force_split, &L->plan, &L->used)) return false;
    if (L->used > 0 && ws_bytes < L->used) return false;
  } else {
    L->plan = plan_with_workspace(n_tiles4, nkv, D, ws_bytes, &L->used);
  }
  // width rule (workspace.hip, beside the split cost model that prices it)
  L->nw = allow_wide && wide_rule(((S + 127) / 128) % 2 == 0, (long)n_tiles4 * L->plan.n_split, L->plan.n_split,
                                  L->plan.kvb_per_split, cu_count())
              ? 8
              : 4;
  L->n_tiles = L->nw == 8 ? n_tiles4 / 2 : n_tiles4;
  L->n_units = L->n_tiles * L->plan.n_split;
  return true;
}

// The one-round unit table (4-wave launches only; nullptr when out of its scope).
static const UnitTable* launch_table(const AttnLaunch& L, int S) {
  return L.nw == 4 && L.plan.n_split > 1 ? unit_table(L.n_tiles, (S + 63) / 64, L.plan.n_split) : nullptr;
}

unsigned long long attn_ws_forced(int B, int S, int H, int D, int n_split, bool* ok) {
  SplitPlan plan;
  size_t used = 0;
  *ok = plan_forced(B * H * ((S + 127) / 128), (S + 63) / 64, D, n_split, &plan, &used);
  return *ok ? used : 0;
}

// Workgroups of a paced launch (each runs tiles i, i + n, i + 2n, ...); returns the tile count
// and sets *n_wg (0 if the occupancy query failed).
int attn_paced_workgroups(int B, int S, int H, int D, int* n_wg) {
  const int n_tiles = B * H * ((S + 127) / 128);
  const int per = D == 128 ? paced_per_cu<128>() : paced_per_cu<64>();
  *n_wg = per < 1 ? 0 : std::min(n_tiles, cu_count() * per);
  return n_tiles;
}

template <int D, int NW>
static int launch_attn(const void* q, const void* k, const void* v, const SlabTable& slabs, int B, int S, int H,
                       int P, float scale, const AttnLaunch& L, int mode, unsigned long long* stamps,
                       const Layout& lay, int pace_chunks, hipStream_t stream) {
  using C = AttnCfg<D, NW>;
  const SplitPlan& plan = L.plan;
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slabs = slabs;
  a.B = B;
  a.S = S;
  a.H = H;
  a.S_P = S / P;
  a.n_mtiles = (S + C::BM - 1) / C::BM;
  a.n_split = plan.n_split;
  a.kvb_per_split = plan.kvb_per_split;
  a.n_units = L.n_units;
  a.c = fabsf(scale) * kLog2e;
  a.qflip = std::signbit(scale) ? 0x80008000u : 0u;
  a.partial = plan.partial;
  a.partial_bytes = (int)((size_t)a.n_units * (NW / 4) * partial_bytes_per_unit(D));
  a.counters = plan.counters;
  a.pace_chunks = pace_chunks;
  a.stamps = stamps;
  a.clock_stamps = mode == kTracedClock;
  if (mode == kTracedClock) mode = kTraced;
  a.src_rows = lay.src ? S / P : S;
  a.src_hs = lay.src_heads > 0 ? lay.src_heads : H;
  a.src_h0 = lay.src_head0;
  a.dst_hs = lay.dst_heads > 0 ? lay.dst_heads : H;
  a.dst_h0 = lay.dst_head0;
  static const UnitTable kNoTable = {};
  const UnitTable* tab = launch_table(L, S);
  a.use_table = tab != nullptr;
  const UnitTable& t = tab ? *tab : kNoTable;
  const dim3 grid(a.n_units), block(C::THREADS);
  const NoSrc none;
  if constexpr (NW == 4) {
    if (mode == kPaced) {  // persistent: as many workgroups as fit at once, each runs several tiles
      if (lay.src || plan.n_split != 1) return XSTAGE_ERR_INVALID;
      const int n = paced_per_cu<D>();
      if (n < 1) return XSTAGE_ERR_HIP;
      const dim3 pgrid(std::min(a.n_units, cu_count() * n));
      hipLaunchKernelGGL((attn_a2a_kernel<D, kPaced, kPlain>), pgrid, block, 0, stream, a, t, none);
      return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
    }
  } else {
    if (mode == kPaced) return XSTAGE_ERR_INVALID;
  }
  if (lay.src) {  // shards: product mode only
    if (mode != kRun) return XSTAGE_ERR_INVALID;
    if (lay.kv_contiguous)
      hipLaunchKernelGGL((attn_a2a_kernel<D, kRun, kShardQ, NW>), grid, block, 0, stream, a, t, *lay.src);
    else
      hipLaunchKernelGGL((attn_a2a_kernel<D, kRun, kShards, NW>), grid, block, 0, stream, a, t, *lay.src);
  } else {
    switch (mode) {
      case kTraced: hipLaunchKernelGGL((attn_a2a_kernel<D, kTraced, kPlain, NW>), grid, block, 0, stream, a, t, none); break;
      case kCoupled: hipLaunchKernelGGL((attn_a2a_kernel<D, kCoupled, kPlain, NW>), grid, block, 0, stream, a, t, none); break;
      case kNoStore: hipLaunchKernelGGL((attn_a2a_kernel<D, kNoStore, kPlain, NW>), grid, block, 0, stream, a, t, none); break;
      default: hipLaunchKernelGGL((attn_a2a_kernel<D, kRun, kPlain, NW>), grid, block, 0, stream, a, t, none); break;
    }
  }
  return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
}

int attn_workgroups(int B, int S, int H, int D, unsigned long long ws_bytes, int* n_split) {
  AttnLaunch L;
  attn_launch(B, S, H, D, ws_bytes, 0, true, &L);
  if (n_split) *n_split = L.plan.n_split;
  return L.n_units;
}

int attn_wg_rows(int B, int S, int H, int D, unsigned long long ws_bytes) {
  AttnLaunch L;
  attn_launch(B, S, H, D, ws_bytes, 0, true, &L);
  return 32 * L.nw;
}

// Workspace bytes a launch of this shape uses given ws_bytes of workspace (0: no split);
// ws_bytes = ~0 gives the bytes of the unconstrained plan.
unsigned long long attn_ws_used(int B, int S, int H, int D, unsigned long long ws_bytes) {
  AttnLaunch L;
  attn_launch(B, S, H, D, ws_bytes, 0, true, &L);
  return L.used;
}

int attn_schedule(int B, int S, int H, int D, unsigned long long ws_bytes, int cap, int* tile, int* split, int* j0,
                  int* j1) {
  AttnLaunch L;
  attn_launch(B, S, H, D, ws_bytes, 0, true, &L);
  const int n = L.n_units;
  if (n > cap) return n;
  const int nkv = (S + 63) / 64;
  const UnitTable* tab = launch_table(L, S);
  for (int i = 0; i < n; ++i) {
    if (tab) {
      const uint32_t e = tab->e[i];
      tile[i] = e & 1023;
      split[i] = (e >> 10) & 15;
      j0[i] = (e >> 14) & 511;
      j1[i] = e >> 23;
    } else {  // the kernel's XCD-contiguous order with uniform splits
      const int q8 = n / 8, r8 = n % 8, x = i % 8, slot = i / 8;
      const int Lx = x < r8 ? x * (q8 + 1) + slot : r8 * (q8 + 1) + (x - r8) * q8 + slot;
      tile[i] = Lx / L.plan.n_split;
      split[i] = Lx % L.plan.n_split;
      j0[i] = split[i] * L.plan.kvb_per_split;
      j1[i] = std::min(j0[i] + L.plan.kvb_per_split, nkv);
    }
  }
  return n;
}

int launch_attn_any(const void* q, const void* k, const void* v, const SlabTable& slabs, int B, int S, int H, int D,
                    int P, float scale, void* ws, unsigned long long ws_bytes, hipStream_t stream, int mode,
                    unsigned long long* stamps, const Layout* layout, int pace_chunks, int force_split) {
  static const Layout kDefaultLayout;
  const Layout& lay = layout ? *layout : kDefaultLayout;
  AttnLaunch L;
  if (!attn_launch(B, S, H, D, ws ? ws_bytes : 0ull, force_split, mode != kPaced, &L)) return XSTAGE_ERR_INVALID;
  if (L.plan.n_split > 1) {
    L.plan.counters = static_cast<uint32_t*>(ws);
    L.plan.partial = static_cast<char*>(ws) + kCounterAreaBytes;
  }
  if (D == 128)
    return L.nw == 8 ? launch_attn<128, 8>(q, k, v, slabs, B, S, H, P, scale, L, mode, stamps, lay, pace_chunks, stream)
                     : launch_attn<128, 4>(q, k, v, slabs, B, S, H, P, scale, L, mode, stamps, lay, pace_chunks, stream);
  return L.nw == 8 ? launch_attn<64, 8>(q, k, v, slabs, B, S, H, P, scale, L, mode, stamps, lay, pace_chunks, stream)
                   : launch_attn<64, 4>(q, k, v, slabs, B, S, H, P, scale, L, mode, stamps, lay, pace_chunks, stream);
}

}  // namespace xstage
