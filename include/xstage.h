/*
 * xstage.h - C ABI of libxstage.so: one GPU's share of Ulysses sequence-parallel attention
 * with the post-attention all-to-all fused into the attention epilogue, for MI355X (gfx950).
 *
 * Source of the method: the four-language gist.science explainer of arXiv 2607.23264,
 * "X-Stage: An Overlooked Pipeline Stage for Communication-Computation Overlap in DiT
 * Inference", technical summary.
 *   - "Contributions", FlashAttention-A2A (piggybacking) item: for Ulysses-style sequence
 *     parallel attention the post-attention all-to-all is fused into FlashAttention; the
 *     owner of each output tile issues its stores toward the destinations and immediately
 *     goes on with the next tile's query loop, with no dedicated communication wave.
 *   - "Results", FlashAttention-A2A: the fused kernel is compared with serial execution
 *     (attention, then a separate all-to-all).
 *   - "Methodology": the Burst-Gap model T_iss(G;K,V) = max(T0_iss(K,V), V/R - G) and the
 *     quantities T0_iss, R, Q; "Contributions", characterisation item: they are measured
 *     with parameterised store microbenchmarks.
 *
 * On one GPU the P destinations are P receive buffers ("slabs") in local HBM standing in
 * for the peers' receive buffers.
 *
 * Conventions for every entry point:
 *   - Tensors are bf16 bit patterns (uint16 storage), row-major, last index fastest, on the
 *     current HIP device.  Every tensor pointer must be 16-byte aligned.
 *   - q, k, v and the contiguous attention output are [B, S, H_local, D] ("BSHD").
 *   - Slab p (0 <= p < P) is [B, S/P, H_local, D] and receives sequence rows
 *     [p*S/P, (p+1)*S/P): slab[p][b][r][h][d] = O[b][p*S/P + r][h][d].
 *   - `out_slabs` is a HOST array of P device pointers; the pointers are copied by value
 *     into the kernel arguments, so the array may be freed as soon as the call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work and return;
 *     they never synchronize, never allocate and never free memory: the caller owns every
 *     buffer.  A call on a capturing stream is recorded as kernel nodes only (no memset
 *     nodes) and may be replayed from the graph.
 *   - Split workspace (attention entry points: split_ws, split_ws_bytes).  When a shape has
 *     few 128-row query tiles for the device (small B*H_local*S), the keys of each tile are
 *     split over several workgroups whose partial results meet in a caller-owned workspace:
 *     16 KiB of per-tile arrival counters, then the partials (the same layout for every
 *     shape).  xstage_attn_split_ws_size gives the bytes the fastest plan uses (0 when the
 *     shape is not split; at most 16 KiB + 128 MiB).  The split count is limited to what fits
 *     in split_ws_bytes: a smaller workspace gives the same result up to fp32 summation
 *     order, possibly more slowly, and split_ws = NULL runs without splits.  The workspace
 *     is plain device memory (any allocator), 16-byte aligned, disjoint from every other
 *     buffer of the call; it must hold zeros before its first use, and every call leaves
 *     the counters it used at zero once it completes, so one workspace serves any later
 *     call and shape.  Calls that may run concurrently (different streams) need separate
 *     workspaces.
 *   - Errors: every argument check runs before any HIP call; on an error nothing is
 *     launched and no output byte is touched.  Faults inside kernels surface at the
 *     caller's next synchronization.  XSTAGE_ERR_HIP reports the HIP launch status.
 *   - Attention: O = softmax(scale * Q K^T) V per (b, h), non-causal, products and sums in
 *     fp32, output rounded to bf16 (round to nearest, ties to even).  When a tile's keys are
 *     split over workgroups, each split's partial sums pass through an fp16 record (within
 *     2^-11 of themselves; scaled by a power of two where they would exceed fp16's range)
 *     before they are merged in fp32.  scale may be any finite value, including 0 and
 *     negative values.
 *   - Thread safety: the library keeps no device state; its host-side caches (CU count and
 *     per-shape schedule tables) are guarded by a mutex; entry points may be called
 *     concurrently.
 */
#ifndef XSTAGE_H_
#define XSTAGE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XSTAGE_MAX_P 64

typedef enum {
  XSTAGE_OK = 0,
  XSTAGE_ERR_INVALID = 1,     /* null pointer, size <= 0, S % P != 0, misaligned pointer,
                                 non-finite scale, overlapping buffers, bad parameters */
  XSTAGE_ERR_UNSUPPORTED = 2, /* D not in {64, 128}, P > XSTAGE_MAX_P, a tensor of
                                 2^31 elements or more */
  XSTAGE_ERR_HIP = 3          /* the HIP runtime refused the launch */
} xstage_status_t;

/* Fused attention + post-attention all-to-all scatter ("Contributions", FlashAttention-A2A
 * piggybacking item).  q, k, v: [B, S, H_local, D]; out_slabs: P device pointers, each to
 * [B, S/P, H_local, D].  Each output tile is written straight from the attention epilogue
 * into the slab that owns its rows; the issuing wave does not wait for the stores and
 * goes on with its next tile.  Slabs must not overlap each other or q, k, v. */
int xstage_attn_a2a_fwd(const void* q, const void* k, const void* v, void* const* out_slabs,
                        int B, int S, int H_local, int D, int P, float scale, void* split_ws,
                        unsigned long long split_ws_bytes, void* stream);

/* xstage_attn_a2a_fwd without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, hosts that forbid allocation):
 * the call never allocates.  Its split partials and arrival counters live in a 32 MiB
 * static device array of the library, one copy per GPU, held until the process ends; the
 * first call on a device looks up that copy's address and zeroes its counters with a fill
 * kernel on `stream`, and every call leaves them at zero.  The key-split count is the one
 * xstage_attn_a2a_fwd chooses with a 32 MiB workspace (the FLUX-1024 share's fastest plan
 * fits; longer shapes split less), so results equal that call's bit for bit; a plan that
 * would need more than the array holds returns XSTAGE_ERR_UNSUPPORTED.  All calls on one
 * GPU share its array: calls that may overlap on one GPU (different streams or threads)
 * race.  Arguments, requirements and result otherwise as for xstage_attn_a2a_fwd. */
int xstage_attn_a2a_fwd_noalloc(const void* q, const void* k, const void* v,
                                void* const* out_slabs, int B, int S, int H_local, int D, int P,
                                float scale, void* stream);

/* Bytes of split workspace the attention entry points use for this shape at full speed
 * (see the split workspace convention above); 0 when the shape is not split.  Host only. */
int xstage_attn_split_ws_size(int B, int S, int H_local, int D, unsigned long long* bytes);

/* Attention alone into a contiguous [B, S, H_local, D] output (the first half of the serial
 * baseline of "Results", FlashAttention-A2A).  `out` must not overlap q, k, v. */
int xstage_attn_fwd(const void* q, const void* k, const void* v, void* out,
                    int B, int S, int H_local, int D, float scale, void* split_ws,
                    unsigned long long split_ws_bytes, void* stream);

/* xstage_attn_a2a_fwd with full-head destination buffers ("Contributions",
 * FlashAttention-A2A item: each output tile is stored straight into its destination's
 * receive buffer).  In a Ulysses group over H_dst heads, destination p's receive buffer
 * holds its S/P sequence rows of every head: out_dst[p] is [B, S/P, H_dst, D], and this
 * call writes head columns [h_dst0, h_dst0 + H_local) only:
 *   out_dst[p][b][r][h_dst0 + h][d] = O[b][p*S/P + r][h][d];
 * every other element of out_dst is left untouched.  Requires H_dst >= H_local and
 * 0 <= h_dst0 <= H_dst - H_local (else XSTAGE_ERR_INVALID), B*S*H_dst*D < 2^31 (else
 * XSTAGE_ERR_UNSUPPORTED).  The P buffers (B*S*H_dst*D*2/P bytes each) must not overlap
 * each other or q, k, v.  With H_dst = H_local and h_dst0 = 0 this is xstage_attn_a2a_fwd. */
int xstage_attn_a2a_fwd_strided(const void* q, const void* k, const void* v, void* const* out_dst,
                                int B, int S, int H_local, int D, int P, int H_dst, int h_dst0,
                                float scale, void* split_ws, unsigned long long split_ws_bytes,
                                void* stream);

/* One rank's Ulysses attention layer with both all-to-alls fused into the attention kernel
 * (the post-attention one in the epilogue as in xstage_attn_a2a_fwd_strided, the
 * pre-attention one in the Q/K/V loads).  Before attention each of the P ranks holds one
 * contiguous sequence shard of every head; this rank computes the heads
 * [h0, h0 + H_local) over the whole sequence:
 *   q_src[p], k_src[p], v_src[p]: HOST arrays of P device pointers, shard p = [B, S/P, H, D]
 *       holding sequence rows [p*S/P, (p+1)*S/P) of all H heads (read only; shards may
 *       alias each other);
 *   out_dst[p]: HOST array of P device pointers, [B, S/P, H, D]; head columns
 *       [h0, h0 + H_local) are written, all other elements are left untouched:
 *       out_dst[p][b][r][h0 + h][d] = O[b][p*S/P + r][h][d], with
 *       O = attention of Q[b][s][h] = q_src[s / (S/P)][b][s % (S/P)][h0 + h] (same for K, V).
 * Requires 0 < H_local <= H, 0 <= h0 <= H - H_local (else XSTAGE_ERR_INVALID), P <= 32
 * and B*S*H*D < 2^31 (else XSTAGE_ERR_UNSUPPORTED).  The output buffers must not overlap
 * each other or any shard.  Same values as gathering the heads into contiguous q, k, v and
 * calling xstage_attn_a2a_fwd_strided with H_dst = H, h_dst0 = h0, bit for bit. */
int xstage_ulysses_attn_fwd(const void* const* q_src, const void* const* k_src,
                            const void* const* v_src, void* const* out_dst, int B, int S, int H,
                            int H_local, int h0, int D, int P, float scale, void* split_ws,
                            unsigned long long split_ws_bytes, void* stream);

/* The pre-attention all-to-all of a Ulysses layer as a separate step (serial layer): copies
 * heads [h0, h0 + H_local) of the P sequence shards src_shards[p] ([B, S/P, H, D], HOST
 * array of device pointers) into the contiguous out [B, S, H_local, D]:
 *   out[b][s][h][d] = src_shards[s / (S/P)][b][s % (S/P)][h0 + h][d].
 * Requires 0 < H_local <= H, 0 <= h0 <= H - H_local (else XSTAGE_ERR_INVALID); out must not
 * overlap any shard. */
int xstage_ulysses_gather(const void* const* src_shards, void* out, int B, int S, int H, int H_local,
                          int h0, int D, int P, void* stream);

/* The post-attention all-to-all into full-head receive buffers as a separate step: copies
 * the contiguous in [B, S, H_local, D] into head columns [h_dst0, h_dst0 + H_local) of
 * out_dst[p] ([B, S/P, H_dst, D]); every other element is left untouched.  Requirements as
 * for xstage_attn_a2a_fwd_strided (in in place of q, k, v). */
int xstage_a2a_scatter_strided(const void* in, void* const* out_dst, int B, int S, int H_local,
                               int D, int P, int H_dst, int h_dst0, void* stream);

/* Serial version of xstage_ulysses_attn_fwd: xstage_ulysses_gather of q, k and v into the
 * workspace, xstage_attn_fwd there, then xstage_a2a_scatter_strided into out_dst, all on
 * `stream`.  workspace: caller-owned, 4 * B * S * H_local * D * 2 bytes (gathered q, k, v
 * and the attention output), disjoint from every shard and output.  Same result as
 * xstage_ulysses_attn_fwd, bit for bit. */
int xstage_ulysses_attn_unfused(const void* const* q_src, const void* const* k_src,
                                const void* const* v_src, void* workspace, void* const* out_dst,
                                int B, int S, int H, int H_local, int h0, int D, int P, float scale,
                                void* split_ws, unsigned long long split_ws_bytes, void* stream);

/* Ulysses layer with K and V staged: xstage_ulysses_gather of k and v into the workspace,
 * then one attention launch that reads Q from the shards in place and writes its output
 * into out_dst as xstage_ulysses_attn_fwd does, all on `stream`.  Every query tile reads
 * all of K and V, so at long sequences the gathered copies keep those reads to one
 * contiguous buffer each, while Q (read once) and the output (written once) keep the
 * fused all-to-all.  Measured on MI355X (H_local = H/8, D = 128): about 3 % faster than
 * xstage_ulysses_attn_fwd when one tensor's shards span 335 MB (S * H * D * 2 bytes), level
 * at about 100 MB, and 24 % slower at 28 MB, where the two extra launches cost more than
 * the in-place reads lose.  workspace: caller-owned, 2 * B * S * H_local * D * 2 bytes (k,
 * then v), disjoint from every shard and output.  Requirements and result as for
 * xstage_ulysses_attn_fwd, bit for bit. */
int xstage_ulysses_attn_fwd_kv_staged(const void* const* q_src, const void* const* k_src,
                                      const void* const* v_src, void* workspace,
                                      void* const* out_dst, int B, int S, int H, int H_local,
                                      int h0, int D, int P, float scale, void* split_ws,
                                      unsigned long long split_ws_bytes, void* stream);

/* The separate all-to-all send step of the serial baseline ("Results", FlashAttention-A2A:
 * serial execution runs attention, then the all-to-all): copies a contiguous
 * [B, S, H_local, D] tensor into the P slabs.  Slabs must not overlap `in` or each other. */
int xstage_a2a_scatter(const void* in, void* const* out_slabs, int B, int S, int H_local,
                       int D, int P, void* stream);

/* Serial baseline ("Results", FlashAttention-A2A: the fused kernel is measured against
 * attention followed by a separate all-to-all): xstage_attn_fwd into `workspace`
 * ([B, S, H_local, D], caller-owned), then xstage_a2a_scatter into the slabs, both on
 * `stream`.  Same result as xstage_attn_a2a_fwd, bit for bit. */
int xstage_attn_a2a_unfused(const void* q, const void* k, const void* v, void* workspace,
                            void* const* out_slabs, int B, int S, int H_local, int D, int P,
                            float scale, void* split_ws, unsigned long long split_ws_bytes,
                            void* stream);

/* Work decomposition of the attention entry points for this shape on the current device,
 * given split_ws_bytes of split workspace (0: none): *n_workgroups workgroups (n_tiles x key
 * splits, n_tiles = B * H_local * ceil(S / rows), rows from xstage_attn_a2a_wg_rows), *n_split
 * key splits per tile (n_split may be NULL).  The split count is chosen per 128-row tile; a
 * launch of 256-row workgroups splits each of them the same way.  Host only; with
 * xstage_attn_a2a_wg_rows it sizes the stamps of xstage_attn_a2a_fwd_traced. */
int xstage_attn_a2a_plan(int B, int S, int H_local, int D, unsigned long long split_ws_bytes,
                         int* n_workgroups, int* n_split);

/* Query rows per workgroup of that launch (*rows): 128 (4 waves of 32 rows) or 256 (8 waves;
 * every K/V block staged in LDS then serves twice the rows).  256 is used when the launch with
 * 128 gives every CU two workgroups without placement-sized key ranges (no split and at least
 * two workgroups per CU, or more workgroups than fit at once), the most 128-row workgroups
 * any CU runs (ceil(workgroups / CUs)) is even, every key range spans at least 20 64-key
 * blocks, and every (b, h) has an even number of 128-row tiles; the key ranges and merge
 * order per query row are then the same, and so is the result, bit for bit.  Plumbing of this work decomposition (the pages fix no
 * tile shape; "Contributions", FlashAttention-A2A item, defines the fused call).  Host only. */
int xstage_attn_a2a_wg_rows(int B, int S, int H_local, int D, unsigned long long split_ws_bytes,
                            int* rows);

/* The work decomposition xstage_attn_a2a_fwd uses for this shape on the current device
 * (256 CUs assumed when no device is present), given split_ws_bytes of split workspace:
 * for each of the *n_workgroups workgroups,
 * the tile it computes (index over (b, h, m-tile of xstage_attn_a2a_wg_rows rows), m-tile
 * fastest), its split
 * index within the tile (the merge order) and its half-open range [j0, j1) of 64-key
 * blocks.  The ranges of a tile's splits partition [0, ceil(S / 64)) in split order.
 * Launches whose workgroups fit on the device at once (more than one per CU) use ranges
 * sized to each workgroup's CU placement; others use equal ranges.  Host only; the four
 * arrays hold at least `cap` ints (caller-owned); cap < *n_workgroups writes nothing and
 * returns XSTAGE_ERR_INVALID with *n_workgroups set. */
int xstage_attn_a2a_schedule(int B, int S, int H_local, int D, unsigned long long split_ws_bytes,
                             int cap, int* tile, int* split, int* j0, int* j1, int* n_workgroups);

/* Instrumented xstage_attn_a2a_fwd for the per-tile store-span study ("Results",
 * FlashAttention-A2A: the measured overhead against the completion-coupled counterfactual;
 * "Contributions", X-Stage item: neither a fully blocking nor an unbounded asynchronous
 * model describes the issuer).  Same arguments and the same slab contents as
 * xstage_attn_a2a_fwd, plus:
 *   mode 0: nothing else changes (the stores of a tile are not waited on);
 *   mode 1: completion-coupled counterfactual: each wave waits for its epilogue stores to
 *           complete before it ends;
 *   mode 2: unbounded-asynchronous bound: no output store is issued at all (the slabs are
 *           NOT written; everything else runs);
 *   mode 3: as mode 0, but stamp entries [2] and [3] hold the shader-clock counter
 *           (s_memtime) at start and at the end of the key loop, so that
 *           ([3] - [2]) / ([1] - [0]) * xstage_wallclock_hz is the core clock the loop ran at;
 *   stamps: device uint64 [n_workgroups][rows / 32 waves][4] (xstage_attn_a2a_plan and
 *           xstage_attn_a2a_wg_rows with the same split_ws_bytes, or 0 when split_ws is
 *           NULL), caller-owned,
 *           8-byte aligned, disjoint from every other argument; per wave, in wall-clock
 *           ticks (xstage_wallclock_hz): start, end of the key loop, last epilogue store
 *           issued (0 if the wave stores nothing: a split that does not merge, rows past S,
 *           mode 2), stores complete (mode 1 only, else 0); mode 3 as stated above.
 * Other modes are XSTAGE_ERR_INVALID. */
int xstage_attn_a2a_fwd_traced(const void* q, const void* k, const void* v, void* const* out_slabs,
                               int B, int S, int H_local, int D, int P, float scale, int mode,
                               unsigned long long* stamps, void* split_ws,
                               unsigned long long split_ws_bytes, void* stream);

/* Split-count override of the fused call, for tuning and for checking the split-count model
 * (plumbing of this work decomposition; the pages describe the fused call, "Contributions",
 * FlashAttention-A2A item, not its decomposition).  xstage_attn_a2a_fwd with the key range of
 * every 128-row tile split into exactly n_split ranges (1: no split) instead of the count the
 * library's model picks; the same decomposition otherwise (ranges sized to the workgroups'
 * CU placement when every workgroup fits on the device at once, equal ranges of 64-key
 * blocks otherwise, 256-row workgroups under the same rule as xstage_attn_a2a_wg_rows with
 * this split count), and the same result contract: with the model's own count the slabs
 * equal xstage_attn_a2a_fwd's bit for bit.
 *   n_split: 1..15, and ceil(S / 64) blocks must form exactly n_split non-empty equal
 *            ranges; shapes with more than 4096 tiles take n_split = 1 only;
 *   split_ws: at least xstage_attn_nsplit_ws_size bytes (NULL allowed for n_split = 1),
 *            16-byte aligned, zeroed before its first use, caller-owned, as for
 *            xstage_attn_a2a_fwd (every call leaves the counters at zero).
 * XSTAGE_ERR_INVALID for an unavailable n_split or a too small workspace, otherwise the
 * argument errors of xstage_attn_a2a_fwd.  Never synchronizes or allocates. */
int xstage_attn_a2a_fwd_nsplit(const void* q, const void* k, const void* v, void* const* out_slabs,
                               int B, int S, int H_local, int D, int P, float scale, int n_split,
                               void* split_ws, unsigned long long split_ws_bytes, void* stream);

/* Split workspace bytes xstage_attn_a2a_fwd_nsplit needs for this shape and n_split: 0 for
 * n_split = 1, else 16 KiB of counters plus n_tiles * n_split partial records of
 * 4 * (D / 16 + 1) * 1 KiB (at most 128 MiB of partials).  Host only; XSTAGE_ERR_INVALID when
 * n_split is unavailable for the shape (see above). */
int xstage_attn_nsplit_ws_size(int B, int S, int H_local, int D, int n_split, unsigned long long* bytes);

/* Paced fused attention + all-to-all: the burst-shaping use of the Burst-Gap model
 * ("Significance": the model as a way to shape the communication bursts and hide their
 * issuer-side cost; "Methodology": a burst of V followed by a gap G of compute) applied to
 * the epilogue of the fused kernel ("Contributions", FlashAttention-A2A item: the tile's
 * owner issues its stores and goes on with the next tile's query loop).  A persistent
 * launch: xstage_attn_a2a_paced_plan's n_workgroups workgroups (as many as fit on the
 * device at once) each compute tiles i, i + n_workgroups, ...; a finished tile's rows wait
 * in LDS and are issued in `chunks` equal chunks, one at the start of each of the next
 * tile's first key-loop iterations (128 keys each); chunks a short next tile has no
 * iteration for, and the last tile's rows, are issued after its loop.  chunks = 1 issues the
 * whole tile at once, at the next tile's first iteration.
 *   chunks: 1, 2, 4 or 8 for D = 128 (a wave's 32 rows are 8 16-byte stores per lane);
 *           1, 2 or 4 for D = 64; anything else is XSTAGE_ERR_INVALID.
 * Same arguments otherwise as xstage_attn_a2a_fwd, no key splits and no workspace: the slab
 * contents equal xstage_attn_a2a_fwd's with split_ws = NULL, bit for bit, for every
 * `chunks`.  Never synchronizes or allocates; argument errors as xstage_attn_a2a_fwd. */
int xstage_attn_a2a_fwd_paced(const void* q, const void* k, const void* v, void* const* out_slabs,
                              int B, int S, int H_local, int D, int P, float scale, int chunks,
                              void* stream);

/* Decomposition of xstage_attn_a2a_fwd_paced for this shape on the current device:
 * *n_tiles = B * H_local * ceil(S / 128) tiles over *n_workgroups persistent workgroups.
 * Host only (queries the device's occupancy once per D); XSTAGE_ERR_HIP if that query
 * fails. */
int xstage_attn_a2a_paced_plan(int B, int S, int H_local, int D, int* n_workgroups, int* n_tiles);

/* Expert-wave grouped GEMM with the combine all-to-all in the Linear-2 epilogue: the
 * stand-in for the interleaved scheduling of "Contributions", MegaMoE (reshaping) item, and
 * "Results", MegaMoE optimisation.  E experts on this GPU; expert e owns the token rows
 * [expert_offsets[e], expert_offsets[e+1]) of x and h (T = expert_offsets[E] tokens):
 *   Linear-1:  h[t, :] = bf16(x[t, :] . w1[e]^T)            (h: [T, d_ff], written)
 *   Linear-2:  y[t, :] = bf16(h[t, :] . w2[e]^T), stored to out[dst_slab[t]][dst_row[t], :]
 * with fp32 accumulation and round-to-nearest-even bf16 results; no activation between the
 * two products.  Experts are grouped into waves of experts_per_wave in index order.
 *   schedule 0 (expert waves): per wave, one launch of its Linear-1 tiles, then one of its
 *              Linear-2 tiles (the stores of a wave come in one concentrated phase);
 *   schedule 1 (interleaved): Linear-1 of wave 0, then for every wave w one launch mixing
 *              the Linear-2 tiles of wave w with the Linear-1 tiles of wave w+1 (the
 *              Linear-1 tiles are dispatched first; Linear-2 tiles run beside them).
 * Both schedules give the same result bit for bit.  Layouts (bf16, row-major):
 *   x [T, d_model], w1 [E, d_ff, d_model], w2 [E, d_model, d_ff] (weights as a linear
 *   layer stores them: output features by input features), h [T, d_ff] (caller-owned
 *   workspace), out[p] [out_rows[p], d_model]; dst_slab, dst_row: device int32 [T].
 * A token whose (dst_slab, dst_row) is outside [0, P) x [0, out_rows[p]) is not stored.
 *   stamps (optional, NULL for none): device uint64 [n_tiles][4 waves][4] (n_tiles from
 *   xstage_moe_waves_plan: all Linear-1 tiles in expert order, then all Linear-2 tiles) in
 *   wall-clock ticks: start, end of the k loop, last store issued, then the tile type (0, 1).
 * Requires 1 <= E <= 4096, d_model and d_ff multiples of 128 (<= 65536),
 * 1 <= experts_per_wave <= 32, schedule in {0, 1}, expert_offsets (HOST, E + 1 entries)
 * starting at 0 and nondecreasing, 1 <= P <= XSTAGE_MAX_P, out_rows[p] >= 0, 16-byte
 * aligned bf16 pointers, 4-byte aligned index arrays; h, every out[p] and stamps must not
 * overlap each other or any input.  Else XSTAGE_ERR_INVALID / XSTAGE_ERR_UNSUPPORTED. */
typedef struct {
  int E;
  int d_model;
  int d_ff;
  int experts_per_wave;
  int schedule;
  const int* expert_offsets;
  const void* x;
  const void* w1;
  const void* w2;
  void* h;
  const int* dst_slab;
  const int* dst_row;
  int P;
  void* const* out;
  const int* out_rows;
  unsigned long long* stamps;
} xstage_moe_params_t;

int xstage_moe_waves_run(const xstage_moe_params_t* p, void* stream);

/* The launches of a schedule, host only: for every expert e, l1_launch[e] and l2_launch[e]
 * are the indices of the launches holding its Linear-1 and Linear-2 tiles; *n_launches the
 * number of launches, *n_tiles the tiles of both kinds (sizes the stamps).  Arrays hold at
 * least E ints (caller-owned).  Same requirements on the shape as xstage_moe_waves_run. */
int xstage_moe_waves_plan(int E, const int* expert_offsets, int d_model, int d_ff,
                          int experts_per_wave, int schedule, int* l1_launch, int* l2_launch,
                          int* n_launches, int* n_tiles);

/* Burst-Gap store microbenchmark ("Methodology"; "Contributions", characterisation item).
 * K producer workgroups (256 threads each) run `rounds` rounds of: a burst that stores
 * V_bytes / K bytes as 16-byte stores into the producer's share of destination set
 * (round % n_dst_sets), then a dependent FMA loop of `gap_fma_iters` iterations (the gap G).
 * No wait for store completion inside a round; after the last round's gap the producer
 * waits for all its stores to complete.
 *   dst:    device buffer of at least n_dst_sets * V_bytes bytes (caller guarantees size).
 *   stamps: device uint64 [K][rounds][3] in wall-clock ticks (xstage_wallclock_hz):
 *           [0] burst start (all waves of the producer at the start barrier),
 *           [1] last store of the burst issued by every wave (no wait for completion),
 *           [2] end of the gap; in the last round, taken after the wait for completion.
 *   sync:   NULL, or device uint32 [rounds], zero-filled, 4-byte aligned, disjoint from dst
 *           and stamps: then every round starts with a start barrier across the K
 *           producers (each adds 1 to sync[round] and waits until all K have arrived or
 *           sync_timeout_ticks wall-clock ticks have passed, whichever comes first), so
 *           that the K bursts of a round start together and their union is one aggregate
 *           burst of V bytes; the wait always ends (the timeout bounds it).  Without sync
 *           the producers' rounds drift apart.  sync_timeout_ticks: 1 .. 10^9 when sync
 *           is set.
 *   V_bytes must be a multiple of K * 4096 (each producer stores whole 4 KiB rows of
 *   16-byte lanes); V_bytes = 0 runs the gap alone (calibration).  1 <= K <= 4096,
 *   1 <= rounds <= 65536, n_dst_sets >= 1, nontemporal in {0, 1}. */
typedef struct {
  int K;
  int rounds;
  int n_dst_sets;
  int nontemporal;
  unsigned long long V_bytes;
  unsigned int gap_fma_iters;
  void* dst;
  unsigned long long* stamps;
  unsigned int* sync;
  unsigned long long sync_timeout_ticks;
} xstage_bg_params_t;

int xstage_burst_gap_run(const xstage_bg_params_t* p, void* stream);

/* Frequency of the device wall clock used by the microbenchmark stamps, in Hz
 * (hipDeviceAttributeWallClockRate of the current device), which turns the Burst-Gap
 * stamps into the issue times of "Methodology".  The only entry point that queries the
 * device. */
int xstage_wallclock_hz(double* hz);

/* Burst-Gap issue time in seconds ("Methodology"): max(T0, V/R - G), with V in bytes and R
 * in bytes per second.  Returns a negative value for R <= 0 or non-finite inputs. */
double xstage_bg_t_iss(double G_s, double T0_s, double V_bytes, double R_bytes_per_s);

/* Pacing chunk count for an epilogue burst, host only: the Burst-Gap model ("Methodology")
 * applied to a tile of V_bytes that a producer issues before the G_s seconds of compute of
 * its next tile, with the capacity reading of the printed formula (pending capacity
 * Q_bytes drained at R; issue time without backpressure a_s + V / f1_Bps for a burst of V).
 * Issuing the tile as c chunks of V/c, each followed by G/c of the compute, lets every
 * chunk use the whole capacity, so the tile's issuer-visible time is
 *   T(c) = max(c * a + V / f1, V / R - min(G, c * Q / R)).
 * Returns the smallest c in [1, c_max] minimising T(c), and T(c) in *t_visible_s (may be
 * NULL); c = 1 is the unpaced burst.  Returns 0 for non-finite or negative inputs,
 * R <= 0, f1 <= 0 or c_max < 1. */
int xstage_bg_pacing_chunks(double V_bytes, double G_s, double a_s, double f1_Bps, double R_Bps, double Q_bytes,
                            int c_max, double* t_visible_s);

/* Static string naming a status code returned by any entry point above (plumbing of this
 * C ABI; the pages describe no API). */
const char* xstage_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* XSTAGE_H_ */
