// Fused non-causal attention + Ulysses post-attention all-to-all epilogue for gfx950.
//
// Method: X-Stage explainer (gist.science, arXiv 2607.23264), technical summary,
// "Contributions", FlashAttention-A2A (piggybacking) item: the post-attention all-to-all is
// fused into FlashAttention; the owner of an output tile issues the stores of that tile
// toward its destinations and at once goes on with the next tile's query loop, which gives
// the stores time to drain; no wave is set aside for communication.  Here the P
// destinations are P receive buffers ("slabs") in local HBM.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one (batch, head)):
//   * each wave owns 32 query rows and keeps them in registers as the B operand of
//     v_mfma_f32_32x32x16_bf16; scores are computed transposed, S^T = K Q^T, so that one
//     lane holds 32 keys of ONE query: the row max is a max over the lane's registers plus
//     one swap of wave halves, and the row sum never leaves the lane until the end;
//   * K and V blocks of 64 keys are staged in LDS (double-buffered, XOR-swizzled 16-byte
//     chunks) by all 256 threads; the next block's global loads are in flight while the
//     current block is computed;
//   * O^T = V^T P^T: P^T comes straight out of the score accumulators (converted to bf16),
//     and V^T operands are read from the natural [key][d] LDS layout with
//     ds_read_b64_tr_b16, the gfx950 transposing LDS read;
//   * epilogue: normalise, round to bf16, restage the tile through LDS and write each row's
//     16-byte chunks straight into the slab owning that sequence row.  The stores are not
//     waited on.
#include <math.h>

#include "common.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace xstage {

template <int D>
struct AttnCfg {
  static constexpr int BM = 128;        // query rows per workgroup
  static constexpr int BN = 64;         // keys per block
  static constexpr int THREADS = 256;   // 4 waves of 64
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
  int kvb_per_split; // 64-key blocks per split
  float c;           // |scale| * log2(e): scores are turned into base-2 logits
  uint32_t qflip;    // 0x80008000 for a negative scale: Q is negated on load
  f32x4* partial;    // split partials: [tile][split][wave][PREC chunks][64 lanes] (n_split > 1)
  uint32_t* counters;  // per-tile arrival counters, zero between launches (n_split > 1)
};

// A pointer read through a wave-uniform index, kept in scalar registers.
__device__ __forceinline__ uint16_t* uniform_ptr(uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<uint16_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_a2a_kernel(const AttnArgs a) {
  using C = AttnCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[4 * C::BLKB];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;  // half of the wave

  // XCD-aware unit order: workgroup i runs on XCD i % 8; give each XCD a contiguous range
  // of (b, h, m-tile) units so that one head's K/V stays in one XCD's L2.
  int L;
  {
    const int i = blockIdx.x, n = a.n_units;
    const int q8 = n >> 3, r8 = n & 7, xcd = i & 7, slot = i >> 3;
    L = xcd < r8 ? xcd * (q8 + 1) + slot : r8 * (q8 + 1) + (xcd - r8) * q8 + slot;
  }
  const int tile = L / a.n_split;
  const int split = L - tile * a.n_split;
  const int mt = tile % a.n_mtiles;
  const int bh = tile / a.n_mtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int m0 = mt * C::BM;
  const int S = a.S;
  const uint32_t rs = (uint32_t)a.H * D;  // elements between consecutive rows of one head
  const uint32_t head0 = ((uint32_t)b * S * a.H + h) * D;
  const uint16_t* qb = a.q + head0;
  const uint16_t* kb = a.k + head0;
  const uint16_t* vb = a.v + head0;

  // Q fragment (B operand of the score MFMA): lane holds query (lane & 31), d = 16ks + 8*hl + 0..7
  bf16x8 qf[C::KS];
  {
    const int qrow = m0 + w * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < S) x = *reinterpret_cast<const u32x4*>(qb + (uint32_t)qrow * rs + ks * 16 + hl * 8);
      x ^= a.qflip;
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> register -> LDS staging of one K/V block (16-byte chunks).
  u32x4 kr[C::NLD], vr[C::NLD];
  // Keys past the end are clamped to row S-1: their scores are masked and their weights
  // set to exactly zero, so the duplicated (finite) rows contribute nothing.  No branches.
  auto gload = [&](int n0) {
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int lin = i * C::THREADS + tid;
      const int row = lin / C::CH, ch = lin % C::CH;
      const int key = min(n0 + row, S - 1);
      const uint32_t off = (uint32_t)key * rs + ch * 8;
      kr[i] = *reinterpret_cast<const u32x4*>(kb + off);
      vr[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  auto lstore = [&](char* kbuf, char* vbuf) {
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int lin = i * C::THREADS + tid;
      const int row = lin / C::CH, ch = lin % C::CH;
      const int off = row * C::ROWB + ((ch ^ swz<D>(row)) << 4);
      *reinterpret_cast<u32x4*>(kbuf + off) = kr[i];
      *reinterpret_cast<u32x4*>(vbuf + off) = vr[i];
    }
  };

  // Per-lane LDS offsets (loop invariant).
  const int krow = lane & 31;
  const int kswz = swz<D>(krow);
  // transposing V reads: lane group g = lane/16, s4 = lane%16
  const int g = lane >> 4, s4 = lane & 15;
  const int vrow1 = 4 * (g >> 1) + (s4 >> 2);
  const int vrow2 = vrow1 + 8;
  const int vc0 = 2 * (g & 1) + ((s4 & 3) >> 1);  // chunk within a 32-wide d tile
  const int vbyte = (s4 & 1) * 8;
  const int vsw1 = swz<D>(vrow1), vsw2 = swz<D>(vrow2);

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.c;

  const int nkv = (S + C::BN - 1) / C::BN;
  const int j0 = split * a.kvb_per_split;
  const int j1 = min(j0 + a.kvb_per_split, nkv);
  gload(j0 * C::BN);
  lstore(smem, smem + C::BLKB);
  __syncthreads();

  for (int j = j0; j < j1; ++j) {
    const char* kbuf = smem + ((j - j0) & 1) * 2 * C::BLKB;
    const char* vbuf = kbuf + C::BLKB;
    const bool more = j + 1 < j1;
    if (more) gload((j + 1) * C::BN);

    // S^T (keys x queries) for two 32-key tiles
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char* p = kbuf + (t * 32 + krow) * C::ROWB + (((2 * ks + hl) ^ kswz) << 4);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(p);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
      }
    }

    // keys beyond S in the last block: excluded from the max here, weight forced to zero below
    const int n0 = j * C::BN;
    const bool tail = n0 + C::BN > S;
    if (tail) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= S) s[t][r] = -INFINITY;
        }
    }

    // online softmax in base 2 (exp(x) = exp2(x * log2 e); scale folded into c)
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[t][r]);
    mx = max_with_partner32(mx);
    const float m_new = __builtin_fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float neg_m = -m_new;
    float rsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, neg_m));
    if (tail) {  // (-inf) * c is NaN when scale == 0: zero the masked weights explicitly
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= S) s[t][r] = 0.f;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) rsum += s[t][r];
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T, four 16-key steps; k-step t uses registers 8*(t&1)..+7 of s[t>>1],
    // i.e. keys 16t + 8*(jj/4) + 4*hl + jj%4 for slot jj.
#pragma unroll
    for (int t = 0; t < C::BN / 16; ++t) {
      const f32x16& st = s[t >> 1];
      const int rb = 8 * (t & 1);
      const u32x4 pk = {pack_bf16x2(st[rb + 0], st[rb + 1]), pack_bf16x2(st[rb + 2], st[rb + 3]),
                        pack_bf16x2(st[rb + 4], st[rb + 5]), pack_bf16x2(st[rb + 6], st[rb + 7])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
      const char* vt = vbuf + 16 * t * C::ROWB;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int ch = 4 * dt + vc0;
        const bf16x4 lo = lds_read_tr(vt + vrow1 * C::ROWB + ((ch ^ vsw1) << 4) + vbyte);
        const bf16x4 hi = lds_read_tr(vt + vrow2 * C::ROWB + ((ch ^ vsw2) << 4) + vbyte);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dt], 0, 0, 0);
      }
    }

    if (more) {
      char* nk = smem + ((j + 1 - j0) & 1) * 2 * C::BLKB;
      lstore(nk, nk + C::BLKB);
    }
    __syncthreads();
  }

  // ---- key-range splits: every split stores its partial (O, m, l); the last to arrive
  // merges them (exact rescaling by exp2(m_s - m)) and runs the epilogue for the tile.
  if (a.n_split > 1) {
    __shared__ int last_flag;
    constexpr int PREC = 4 * C::DT + 1;  // 16-byte chunks per lane: O registers, then (m, l)
    auto rec = [&](int sp) { return a.partial + ((size_t)(tile * a.n_split + sp) * 4 + w) * PREC * 64 + lane; };
    {
      f32x4* r = rec(split);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          r[(dt * 4 + q4) * 64] = f32x4{o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]};
      r[(PREC - 1) * 64] = f32x4{m_run, l_run, 0.f, 0.f};
    }
    // Each wave's stores complete (workgroup-scope release), then ONE device-scope release
    // for the whole workgroup before its arrival is counted: a device-scope fence writes
    // back the XCD's L2, which is far too costly to repeat per wave.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t prev = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int is_last = prev == (uint32_t)(a.n_split - 1);
      if (is_last) {
        __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next launch
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other splits' partials
      }
      last_flag = is_last;
    }
    __syncthreads();
    if (!last_flag) return;
    // Merge in split order from memory (own partial included), so the result does not
    // depend on which split arrived last.
    float m_all = -INFINITY;
    for (int sp = 0; sp < a.n_split; ++sp) m_all = __builtin_fmaxf(m_all, rec(sp)[(PREC - 1) * 64][0]);
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};
    for (int sp = 0; sp < a.n_split; ++sp) {
      const f32x4* r = rec(sp);
      const f32x4 ml = r[(PREC - 1) * 64];
      const float f = __builtin_amdgcn_exp2f(ml[0] - m_all);
      l_run += ml[1] * f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = r[(dt * 4 + q4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[dt][4 * q4 + e] += x[e] * f;
        }
    }
    m_run = m_all;
  }

  // ---- epilogue: normalise, bf16, restage per wave, store rows into their slabs ----------
  const float inv = 1.0f / sum_with_partner32(l_run);
  char* stage = smem + w * 32 * C::ROWB;  // wave-private [32][D] (buffers are free after the loop)
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

  // Destination of each restaged row.  The wave's 32 rows are consecutive sequence rows, so
  // unless a slab holds fewer than 32 rows they touch at most two slabs, whose pointers are
  // read once as wave-uniform (scalar) values: the stores then issue back to back with no
  // wait between them.  Tiny slabs (fewer than 32 rows) take a per-row-pointer path.
  constexpr int NST = 32 * C::CH / 64;  // 16-byte stores per lane
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int row0 = m0 + wu * 32;
  if (row0 >= S) return;
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
      const uint32_t off = (((uint32_t)b * a.S_P + r) * a.H + h) * D + ch * 8;
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
        const uint32_t off = (((uint32_t)b * a.S_P + r) * a.H + h) * D + ch * 8;
        *reinterpret_cast<u32x4*>(a.slabs.p[p] + off) = val;
      }
    }
  }
}

template <int D>
static int launch_attn(const void* q, const void* k, const void* v, const SlabTable& slabs, int B, int S, int H,
                       int P, float scale, const SplitPlan& plan, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.slabs = slabs;
  a.B = B;
  a.S = S;
  a.H = H;
  a.S_P = S / P;
  a.n_mtiles = (S + AttnCfg<D>::BM - 1) / AttnCfg<D>::BM;
  a.n_split = plan.n_split;
  a.kvb_per_split = plan.kvb_per_split;
  a.n_units = B * H * a.n_mtiles * plan.n_split;
  a.c = fabsf(scale) * kLog2e;
  a.qflip = std::signbit(scale) ? 0x80008000u : 0u;
  a.partial = static_cast<f32x4*>(plan.partial);
  a.counters = plan.counters;
  hipLaunchKernelGGL(attn_a2a_kernel<D>, dim3(a.n_units), dim3(AttnCfg<D>::THREADS), 0, stream, a);
  return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
}

// Bytes of split partials for one tile and one split (4 waves x PREC chunks x 64 lanes x 16 B).
static size_t partial_bytes_per_unit(int D) { return (size_t)4 * (4 * (D / 32) + 1) * 64 * 16; }

int launch_attn_any(const void* q, const void* k, const void* v, const SlabTable& slabs, int B, int S, int H, int D,
                    int P, float scale, hipStream_t stream) {
  const int n_tiles = B * H * ((S + 127) / 128);
  const int nkv = (S + 63) / 64;
  SplitPlan plan = choose_split(n_tiles, nkv, partial_bytes_per_unit(D));
  if (plan.n_split > 1) {
    const int st = acquire_workspace(stream, (size_t)n_tiles * plan.n_split * partial_bytes_per_unit(D), n_tiles,
                                     &plan.partial, &plan.counters);
    if (st != XSTAGE_OK) return st;
  }
  if (D == 128) return launch_attn<128>(q, k, v, slabs, B, S, H, P, scale, plan, stream);
  return launch_attn<64>(q, k, v, slabs, B, S, H, P, scale, plan, stream);
}

}  // namespace xstage
