// The serial baseline's separate all-to-all send step, and the Burst-Gap store
// microbenchmark (X-Stage explainer, gist.science, arXiv 2607.23264, technical summary:
// "Results", FlashAttention-A2A, serial execution; "Methodology", Burst-Gap model;
// "Contributions", characterisation by parameterised microbenchmarks).
#include "common.hpp"

namespace xstage {

// ---------------------------------------------------------------------------------------
// Scatter: for every (b, p) the rows [p*S/P, (p+1)*S/P) of batch b are one contiguous run of
// S/P*H*D elements in the source and in slab p, so the step is B*P plain copies.  Each
// workgroup copies one 16 KiB piece (4 x 16 bytes per thread) of one (b, p) run.
struct ScatterArgs {
  const uint16_t* in;
  SlabTable slabs;
  uint32_t S, S_P, HD;       // HD = H * D
  uint32_t seg_chunks;       // 16-byte chunks per (b, p) run
  uint32_t blocks_per_seg;
  int P;
};

constexpr int kScatterThreads = 256;
constexpr int kScatterUnroll = 4;

__global__ __launch_bounds__(256) void a2a_scatter_kernel(const ScatterArgs a) {
  const uint32_t seg = blockIdx.x / a.blocks_per_seg;
  const uint32_t piece = blockIdx.x - seg * a.blocks_per_seg;
  const uint32_t b = seg / a.P, p = seg - b * a.P;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.in + ((size_t)b * a.S + (size_t)p * a.S_P) * a.HD);
  u32x4* dst = reinterpret_cast<u32x4*>(a.slabs.p[p] + (size_t)b * a.S_P * a.HD);
  const uint32_t base = piece * (kScatterThreads * kScatterUnroll) + threadIdx.x;
  u32x4 r[kScatterUnroll];
#pragma unroll
  for (int i = 0; i < kScatterUnroll; ++i) {
    const uint32_t c = base + i * kScatterThreads;
    if (c < a.seg_chunks) r[i] = src[c];
  }
#pragma unroll
  for (int i = 0; i < kScatterUnroll; ++i) {
    const uint32_t c = base + i * kScatterThreads;
    if (c < a.seg_chunks) dst[c] = r[i];
  }
}

int launch_scatter(const void* in, const SlabTable& slabs, int B, int S, int H, int D, int P, hipStream_t stream) {
  ScatterArgs a;
  a.in = static_cast<const uint16_t*>(in);
  a.slabs = slabs;
  a.S = (uint32_t)S;
  a.S_P = (uint32_t)(S / P);
  a.HD = (uint32_t)(H * D);
  a.seg_chunks = a.S_P * a.HD / 8;
  const uint32_t per_block = kScatterThreads * kScatterUnroll;
  a.blocks_per_seg = (a.seg_chunks + per_block - 1) / per_block;
  a.P = P;
  hipLaunchKernelGGL(a2a_scatter_kernel, dim3(a.blocks_per_seg * (uint32_t)B * (uint32_t)P), dim3(kScatterThreads), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
}

// ---------------------------------------------------------------------------------------
// Head-slice copy: the two all-to-alls of a Ulysses layer as separate steps.  Every row of
// the B x S sequence carries a slice of H_local * D elements at an offset within a row of
// src_w (resp. dst_w) elements; a side is either one contiguous tensor of S rows or P
// sequence shards of S/P rows each (row s in shard s / (S/P)).  Pre-attention: shards of all
// heads -> a contiguous local-head tensor; post-attention: the reverse into full-head
// receive buffers.  Each thread moves 4 chunks of 16 bytes.
struct SliceCopyArgs {
  const uint16_t* src[XSTAGE_MAX_P];
  uint16_t* dst[XSTAGE_MAX_P];
  int src_sharded, dst_sharded;
  uint32_t S, src_rows, dst_rows;
  uint32_t src_w, dst_w, src_off, dst_off;
  uint32_t row_chunks;
  uint32_t total_chunks;
};

__global__ __launch_bounds__(256) void slice_copy_kernel(const SliceCopyArgs a) {
  // B * S * H_local * D < 2^31 elements (checked on the host), so chunk and row indices fit
  // 32 bits.
  const uint32_t base = blockIdx.x * (kScatterThreads * kScatterUnroll) + threadIdx.x;
  u32x4 r[kScatterUnroll];
  u32x4* dp[kScatterUnroll];
#pragma unroll
  for (int i = 0; i < kScatterUnroll; ++i) {
    const uint32_t g = base + i * kScatterThreads;
    dp[i] = nullptr;
    if (g < a.total_chunks) {
      const uint32_t row = g / a.row_chunks;
      const uint32_t ch = g - row * a.row_chunks;
      const uint32_t b = row / a.S, s = row - b * a.S;
      const uint32_t ps = a.src_sharded ? s / a.src_rows : 0, rs = s - ps * a.src_rows;
      const uint32_t pd = a.dst_sharded ? s / a.dst_rows : 0, rd = s - pd * a.dst_rows;
      const uint16_t* src = a.src[ps] + ((size_t)b * a.src_rows + rs) * a.src_w + a.src_off + (size_t)ch * 8;
      dp[i] = reinterpret_cast<u32x4*>(a.dst[pd] + ((size_t)b * a.dst_rows + rd) * a.dst_w + a.dst_off + (size_t)ch * 8);
      r[i] = *reinterpret_cast<const u32x4*>(src);
    }
  }
#pragma unroll
  for (int i = 0; i < kScatterUnroll; ++i)
    if (dp[i]) *dp[i] = r[i];
}

int launch_slice_copy(const void* const* src, int src_sharded, int src_w, int src_off, void* const* dst,
                      int dst_sharded, int dst_w, int dst_off, int B, int S, int H_local, int D, int P,
                      hipStream_t stream) {
  SliceCopyArgs a = {};
  const int ns = src_sharded ? P : 1, nd = dst_sharded ? P : 1;
  for (int i = 0; i < ns; ++i) a.src[i] = static_cast<const uint16_t*>(src[i]);
  for (int i = 0; i < nd; ++i) a.dst[i] = static_cast<uint16_t*>(dst[i]);
  a.src_sharded = src_sharded;
  a.dst_sharded = dst_sharded;
  a.S = (uint32_t)S;
  a.src_rows = (uint32_t)(src_sharded ? S / P : S);
  a.dst_rows = (uint32_t)(dst_sharded ? S / P : S);
  a.src_w = (uint32_t)src_w;
  a.dst_w = (uint32_t)dst_w;
  a.src_off = (uint32_t)src_off;
  a.dst_off = (uint32_t)dst_off;
  a.row_chunks = (uint32_t)(H_local * D / 8);
  a.total_chunks = (uint32_t)((unsigned long long)B * S * a.row_chunks);
  const uint32_t per_block = kScatterThreads * kScatterUnroll;
  const uint32_t blocks = (a.total_chunks + per_block - 1) / per_block;
  if (blocks == 0) return XSTAGE_OK;
  hipLaunchKernelGGL(slice_copy_kernel, dim3(blocks), dim3(kScatterThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
}

// ---------------------------------------------------------------------------------------
// Burst-Gap producer: K workgroups of 4 waves.  Per round: barrier, stamp, issue the burst
// as 16-byte stores (nothing waits on them), barrier (every wave has issued), stamp, FMA
// gap, stamp.  The barriers carry no memory fence, so they order issue, not completion.
struct BGArgs {
  uint8_t* dst;
  unsigned long long* stamps;
  unsigned long long V;
  unsigned long long share;  // bytes per producer per round
  int rounds;
  int n_sets;
  unsigned gap;
  int K;
  uint32_t* sync;                  // per-round arrival counts (nullptr: no start barrier)
  unsigned long long sync_timeout;  // wall-clock ticks a producer waits at most per round
};

__device__ __forceinline__ unsigned long long wall_ticks() { return __builtin_amdgcn_s_memrealtime(); }

template <bool NT>
__global__ __launch_bounds__(256) void burst_gap_kernel(const BGArgs a) {
  const int wg = blockIdx.x, tid = threadIdx.x;
  const u32x4 val = {(uint32_t)tid, (uint32_t)wg, 0x5a5a5a5au, 0xa5a5a5a5u};
  float x = (float)tid * 1e-3f;
  for (int r = 0; r < a.rounds; ++r) {
    uint8_t* base = a.dst + (size_t)(r % a.n_sets) * a.V + (size_t)wg * a.share;
    if (a.sync != nullptr) {
      // Start barrier across producers: count this producer in, then wait until all K
      // are in or the timeout passes.  The count is an agent-scope atomic and the polls are
      // device-scope (sc1) vector loads; the wall clock always advances, so the wait ends.
      __builtin_amdgcn_s_barrier();
      if (tid == 0) {
        __hip_atomic_fetch_add(&a.sync[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(a.sync, (short)0, a.rounds * 4, 0x00020000);
        const unsigned long long t_end = wall_ticks() + a.sync_timeout;
        while (__builtin_amdgcn_raw_buffer_load_b32(rs, r * 4, 0, 16) < (uint32_t)a.K && wall_ticks() < t_end)
          __builtin_amdgcn_s_sleep(1);
      }
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t0 = wall_ticks();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 4
    for (unsigned long long off = (unsigned long long)tid * 16; off < a.share; off += 256 * 16) {
      if constexpr (NT)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(base + off));
      else
        *reinterpret_cast<u32x4*>(base + off) = val;
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t1 = wall_ticks();
    __builtin_amdgcn_sched_barrier(0);
    for (unsigned i = 0; i < a.gap; ++i) {
      x = __builtin_fmaf(x, 0.999f, 1e-3f);
      asm volatile("" : "+v"(x));
    }
    if (r == a.rounds - 1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t2 = wall_ticks();
    __builtin_amdgcn_sched_barrier(0);
    if (tid == 0) {
      unsigned long long* st = a.stamps + ((size_t)wg * a.rounds + r) * 3;
      st[0] = t0;
      st[1] = t1;
      st[2] = t2;
    }
  }
  asm volatile("" ::"v"(x));
}

int launch_burst_gap(const xstage_bg_params_t& p, hipStream_t stream) {
  BGArgs a;
  a.dst = static_cast<uint8_t*>(p.dst);
  a.stamps = p.stamps;
  a.V = p.V_bytes;
  a.share = p.V_bytes / (unsigned long long)p.K;
  a.rounds = p.rounds;
  a.n_sets = p.n_dst_sets;
  a.gap = p.gap_fma_iters;
  a.K = p.K;
  a.sync = p.sync;
  a.sync_timeout = p.sync_timeout_ticks;
  if (p.nontemporal)
    hipLaunchKernelGGL(burst_gap_kernel<true>, dim3(p.K), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(burst_gap_kernel<false>, dim3(p.K), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? XSTAGE_OK : XSTAGE_ERR_HIP;
}

}  // namespace xstage
