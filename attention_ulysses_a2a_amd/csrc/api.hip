// extern "C" entry points of libxstage.so: argument checks, then launches.  Declarations
// and contracts: include/xstage.h.
#include <math.h>

#include <cmath>

#include <vector>

#include "attn_a2a.hpp"
#include "common.hpp"
#include "moe_waves.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace xstage {
int launch_scatter(const void* in, const SlabTable& slabs, int B, int S, int H, int D, int P, hipStream_t stream);
int launch_slice_copy(const void* const* src, int src_sharded, int src_w, int src_off, void* const* dst,
                      int dst_sharded, int dst_w, int dst_off, int B, int S, int H_local, int D, int P,
                      hipStream_t stream);
int launch_burst_gap(const xstage_bg_params_t& p, hipStream_t stream);

static SlabTable make_table(void* const* slabs, int P) {
  SlabTable t;
  for (int i = 0; i < XSTAGE_MAX_P; ++i) t.p[i] = i < P ? static_cast<uint16_t*>(slabs[i]) : nullptr;
  return t;
}

// The part of a caller's split workspace that a launch of this attention shape uses: its
// counters and partials (empty when the plan does not split or there is no workspace).
static Range split_ws_range(const void* ws, unsigned long long ws_bytes, int B, int S, int H, int D) {
  if (ws == nullptr) return Range{0, 0};
  const unsigned long long used = attn_ws_used(B, S, H, D, ws_bytes);
  return used ? range_of(ws, used) : Range{0, 0};
}

// Split workspace checks: 16-byte aligned, and the range the launch uses disjoint from every
// range in `others` (the call's inputs, outputs and other buffers).
static int check_split_ws(const void* ws, Range used, const Range* others, int n_others) {
  if (ws == nullptr) return XSTAGE_OK;
  if (!aligned16(ws)) return XSTAGE_ERR_INVALID;
  for (int o = 0; o < n_others; ++o)
    if (overlaps(used, others[o])) return XSTAGE_ERR_INVALID;
  return XSTAGE_OK;
}

static int check_attn_slabs(const void* q, const void* k, const void* v, void* const* slabs, int B, int S, int H,
                            int D, int P, float scale, const void* extra, unsigned long long extra_bytes,
                            const void* ws, unsigned long long ws_bytes) {
  int st = check_shape(B, S, H, D, P);
  if (st != XSTAGE_OK) return st;
  st = check_qkv(q, k, v, scale);
  if (st != XSTAGE_OK) return st;
  const unsigned long long tb = tensor_bytes(B, S, H, D);
  const Range wr = split_ws_range(ws, ws_bytes, B, S, H, D);
  Range others[5] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), range_of(extra, extra_bytes), wr};
  st = check_split_ws(ws, wr, others, 4);
  if (st != XSTAGE_OK) return st;
  return check_slabs(slabs, P, tb / (unsigned long long)P, others, 5);
}
}  // namespace xstage

using namespace xstage;

extern "C" {

int xstage_attn_split_ws_size(int B, int S, int H_local, int D, unsigned long long* bytes) {
  if (bytes == nullptr) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  *bytes = attn_ws_used(B, S, H_local, D, ~0ull);
  return XSTAGE_OK;
}

int xstage_attn_a2a_fwd(const void* q, const void* k, const void* v, void* const* out_slabs, int B, int S,
                        int H_local, int D, int P, float scale, void* split_ws, unsigned long long split_ws_bytes,
                        void* stream) {
  const int st = check_attn_slabs(q, k, v, out_slabs, B, S, H_local, D, P, scale, nullptr, 0, split_ws,
                                  split_ws_bytes);
  if (st != XSTAGE_OK) return st;
  return launch_attn_any(q, k, v, make_table(out_slabs, P), B, S, H_local, D, P, scale, split_ws, split_ws_bytes,
                         static_cast<hipStream_t>(stream));
}

int xstage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int S, int H_local, int D,
                    float scale, void* split_ws, unsigned long long split_ws_bytes, void* stream) {
  void* slabs[1] = {out};
  const int st = check_attn_slabs(q, k, v, out ? slabs : nullptr, B, S, H_local, D, 1, scale, nullptr, 0, split_ws,
                                  split_ws_bytes);
  if (st != XSTAGE_OK) return st;
  return launch_attn_any(q, k, v, make_table(slabs, 1), B, S, H_local, D, 1, scale, split_ws, split_ws_bytes,
                         static_cast<hipStream_t>(stream));
}

int xstage_a2a_scatter(const void* in, void* const* out_slabs, int B, int S, int H_local, int D, int P,
                       void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  if (in == nullptr || !aligned16(in)) return XSTAGE_ERR_INVALID;
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  const Range others[1] = {range_of(in, tb)};
  st = check_slabs(out_slabs, P, tb / (unsigned long long)P, others, 1);
  if (st != XSTAGE_OK) return st;
  return launch_scatter(in, make_table(out_slabs, P), B, S, H_local, D, P, static_cast<hipStream_t>(stream));
}

int xstage_attn_a2a_unfused(const void* q, const void* k, const void* v, void* workspace, void* const* out_slabs,
                            int B, int S, int H_local, int D, int P, float scale, void* split_ws,
                            unsigned long long split_ws_bytes, void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return XSTAGE_ERR_INVALID;
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  const Range ws = range_of(workspace, tb);
  if (q && (overlaps(ws, range_of(q, tb)) || overlaps(ws, range_of(k, tb)) || overlaps(ws, range_of(v, tb))))
    return XSTAGE_ERR_INVALID;
  st = check_attn_slabs(q, k, v, out_slabs, B, S, H_local, D, P, scale, workspace, tb, split_ws, split_ws_bytes);
  if (st != XSTAGE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* one[1] = {workspace};
  st = launch_attn_any(q, k, v, make_table(one, 1), B, S, H_local, D, 1, scale, split_ws, split_ws_bytes, s);
  if (st != XSTAGE_OK) return st;
  return launch_scatter(workspace, make_table(out_slabs, P), B, S, H_local, D, P, s);
}

int xstage_attn_a2a_fwd_strided(const void* q, const void* k, const void* v, void* const* out_dst, int B, int S,
                                int H_local, int D, int P, int H_dst, int h_dst0, float scale, void* split_ws,
                                unsigned long long split_ws_bytes, void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_dst < H_local || h_dst0 < 0 || h_dst0 > H_dst - H_local) return XSTAGE_ERR_INVALID;
  st = check_shape(B, S, H_dst, D, P);  // destination element offsets stay 32-bit
  if (st != XSTAGE_OK) return st;
  st = check_qkv(q, k, v, scale);
  if (st != XSTAGE_OK) return st;
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  const Range wr = split_ws_range(split_ws, split_ws_bytes, B, S, H_local, D);
  const Range others[4] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), wr};
  st = check_split_ws(split_ws, wr, others, 3);
  if (st != XSTAGE_OK) return st;
  st = check_slabs(out_dst, P, tensor_bytes(B, S, H_dst, D) / (unsigned long long)P, others, 4);
  if (st != XSTAGE_OK) return st;
  Layout lay;
  lay.dst_heads = H_dst;
  lay.dst_head0 = h_dst0;
  return launch_attn_any(q, k, v, make_table(out_dst, P), B, S, H_local, D, P, scale, split_ws, split_ws_bytes,
                         static_cast<hipStream_t>(stream), 0, nullptr, &lay);
}

int xstage_ulysses_attn_fwd(const void* const* q_src, const void* const* k_src, const void* const* v_src,
                            void* const* out_dst, int B, int S, int H, int H_local, int h0, int D, int P, float scale,
                            void* split_ws, unsigned long long split_ws_bytes, void* stream) {
  int st = check_shape(B, S, H, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_local <= 0 || H_local > H || h0 < 0 || h0 > H - H_local) return XSTAGE_ERR_INVALID;
  if (P > kMaxSrc) return XSTAGE_ERR_UNSUPPORTED;
  if (q_src == nullptr || k_src == nullptr || v_src == nullptr || !std::isfinite(scale)) return XSTAGE_ERR_INVALID;
  const unsigned long long shard = tensor_bytes(B, S, H, D) / (unsigned long long)P;
  Range src_ranges[3 * kMaxSrc + 1];
  SrcTable t = {};
  for (int p = 0; p < P; ++p) {
    const void* ptrs[3] = {q_src[p], k_src[p], v_src[p]};
    for (int j = 0; j < 3; ++j) {
      if (ptrs[j] == nullptr || !aligned16(ptrs[j])) return XSTAGE_ERR_INVALID;
      src_ranges[3 * p + j] = range_of(ptrs[j], shard);
    }
    t.q[p] = static_cast<const uint16_t*>(q_src[p]);
    t.k[p] = static_cast<const uint16_t*>(k_src[p]);
    t.v[p] = static_cast<const uint16_t*>(v_src[p]);
  }
  const Range wr = split_ws_range(split_ws, split_ws_bytes, B, S, H_local, D);
  st = check_split_ws(split_ws, wr, src_ranges, 3 * P);
  if (st != XSTAGE_OK) return st;
  src_ranges[3 * P] = wr;
  st = check_slabs(out_dst, P, shard, src_ranges, 3 * P + 1);
  if (st != XSTAGE_OK) return st;
  Layout lay;
  lay.src = &t;
  lay.src_heads = H;
  lay.src_head0 = h0;
  lay.dst_heads = H;
  lay.dst_head0 = h0;
  return launch_attn_any(q_src[0], k_src[0], v_src[0], make_table(out_dst, P), B, S, H_local, D, P, scale, split_ws,
                         split_ws_bytes, static_cast<hipStream_t>(stream), 0, nullptr, &lay);
}

// Shared checks of the Ulysses layouts: P shard pointers (non-null, aligned) of
// B*S*H*D*2/P bytes each, collected into `ranges`.
static int collect_shards(const void* const* shards, int P, unsigned long long bytes, std::vector<Range>* ranges) {
  if (shards == nullptr) return XSTAGE_ERR_INVALID;
  for (int p = 0; p < P; ++p) {
    if (shards[p] == nullptr || !aligned16(shards[p])) return XSTAGE_ERR_INVALID;
    ranges->push_back(range_of(shards[p], bytes));
  }
  return XSTAGE_OK;
}

static bool disjoint_from(Range r, const std::vector<Range>& others) {
  for (const Range& o : others)
    if (overlaps(r, o)) return false;
  return true;
}

int xstage_ulysses_gather(const void* const* src_shards, void* out, int B, int S, int H, int H_local, int h0, int D,
                          int P, void* stream) {
  int st = check_shape(B, S, H, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_local <= 0 || H_local > H || h0 < 0 || h0 > H - H_local) return XSTAGE_ERR_INVALID;
  if (out == nullptr || !aligned16(out)) return XSTAGE_ERR_INVALID;
  std::vector<Range> src;
  st = collect_shards(src_shards, P, tensor_bytes(B, S, H, D) / (unsigned long long)P, &src);
  if (st != XSTAGE_OK) return st;
  if (!disjoint_from(range_of(out, tensor_bytes(B, S, H_local, D)), src)) return XSTAGE_ERR_INVALID;
  void* dst[1] = {out};
  return launch_slice_copy(src_shards, 1, H * D, h0 * D, dst, 0, H_local * D, 0, B, S, H_local, D, P,
                           static_cast<hipStream_t>(stream));
}

int xstage_a2a_scatter_strided(const void* in, void* const* out_dst, int B, int S, int H_local, int D, int P, int H_dst,
                               int h_dst0, void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_dst < H_local || h_dst0 < 0 || h_dst0 > H_dst - H_local) return XSTAGE_ERR_INVALID;
  st = check_shape(B, S, H_dst, D, P);
  if (st != XSTAGE_OK) return st;
  if (in == nullptr || !aligned16(in)) return XSTAGE_ERR_INVALID;
  const Range others[1] = {range_of(in, tensor_bytes(B, S, H_local, D))};
  st = check_slabs(out_dst, P, tensor_bytes(B, S, H_dst, D) / (unsigned long long)P, others, 1);
  if (st != XSTAGE_OK) return st;
  const void* src[1] = {in};
  return launch_slice_copy(src, 0, H_local * D, 0, out_dst, 1, H_dst * D, h_dst0 * D, B, S, H_local, D, P,
                           static_cast<hipStream_t>(stream));
}

int xstage_ulysses_attn_unfused(const void* const* q_src, const void* const* k_src, const void* const* v_src,
                                void* workspace, void* const* out_dst, int B, int S, int H, int H_local, int h0,
                                int D, int P, float scale, void* split_ws, unsigned long long split_ws_bytes,
                                void* stream) {
  int st = check_shape(B, S, H, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_local <= 0 || H_local > H || h0 < 0 || h0 > H - H_local) return XSTAGE_ERR_INVALID;
  if (workspace == nullptr || !aligned16(workspace) || !std::isfinite(scale)) return XSTAGE_ERR_INVALID;
  const unsigned long long shard = tensor_bytes(B, S, H, D) / (unsigned long long)P;
  const unsigned long long tl = tensor_bytes(B, S, H_local, D);
  std::vector<Range> src;
  for (const void* const* t : {q_src, k_src, v_src}) {
    st = collect_shards(t, P, shard, &src);
    if (st != XSTAGE_OK) return st;
  }
  const Range ws = range_of(workspace, 4 * tl);
  if (!disjoint_from(ws, src)) return XSTAGE_ERR_INVALID;
  std::vector<Range> others = src;
  others.push_back(ws);
  const Range wr = split_ws_range(split_ws, split_ws_bytes, B, S, H_local, D);
  st = check_split_ws(split_ws, wr, others.data(), (int)others.size());
  if (st != XSTAGE_OK) return st;
  others.push_back(wr);
  st = check_slabs(out_dst, P, shard, others.data(), (int)others.size());
  if (st != XSTAGE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  void* qc[1] = {w};
  void* kc[1] = {w + tl};
  void* vc[1] = {w + 2 * tl};
  void* oc[1] = {w + 3 * tl};
  for (int i = 0; i < 3; ++i) {
    const void* const* srcs = i == 0 ? q_src : i == 1 ? k_src : v_src;
    void* const* dst = i == 0 ? qc : i == 1 ? kc : vc;
    st = launch_slice_copy(srcs, 1, H * D, h0 * D, dst, 0, H_local * D, 0, B, S, H_local, D, P, s);
    if (st != XSTAGE_OK) return st;
  }
  st = launch_attn_any(qc[0], kc[0], vc[0], make_table(oc, 1), B, S, H_local, D, 1, scale, split_ws, split_ws_bytes, s);
  if (st != XSTAGE_OK) return st;
  const void* osrc[1] = {oc[0]};
  return launch_slice_copy(osrc, 0, H_local * D, 0, out_dst, 1, H * D, h0 * D, B, S, H_local, D, P, s);
}

int xstage_ulysses_attn_fwd_kv_staged(const void* const* q_src, const void* const* k_src, const void* const* v_src,
                                      void* workspace, void* const* out_dst, int B, int S, int H, int H_local, int h0,
                                      int D, int P, float scale, void* split_ws, unsigned long long split_ws_bytes,
                                      void* stream) {
  int st = check_shape(B, S, H, D, P);
  if (st != XSTAGE_OK) return st;
  if (H_local <= 0 || H_local > H || h0 < 0 || h0 > H - H_local) return XSTAGE_ERR_INVALID;
  if (P > kMaxSrc) return XSTAGE_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) || !std::isfinite(scale)) return XSTAGE_ERR_INVALID;
  const unsigned long long shard = tensor_bytes(B, S, H, D) / (unsigned long long)P;
  const unsigned long long tl = tensor_bytes(B, S, H_local, D);
  std::vector<Range> src;
  for (const void* const* t : {q_src, k_src, v_src}) {
    st = collect_shards(t, P, shard, &src);
    if (st != XSTAGE_OK) return st;
  }
  const Range ws = range_of(workspace, 2 * tl);
  if (!disjoint_from(ws, src)) return XSTAGE_ERR_INVALID;
  std::vector<Range> others = src;
  others.push_back(ws);
  const Range wr = split_ws_range(split_ws, split_ws_bytes, B, S, H_local, D);
  st = check_split_ws(split_ws, wr, others.data(), (int)others.size());
  if (st != XSTAGE_OK) return st;
  others.push_back(wr);
  st = check_slabs(out_dst, P, shard, others.data(), (int)others.size());
  if (st != XSTAGE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  void* kc[1] = {w};
  void* vc[1] = {w + tl};
  st = launch_slice_copy(k_src, 1, H * D, h0 * D, kc, 0, H_local * D, 0, B, S, H_local, D, P, s);
  if (st != XSTAGE_OK) return st;
  st = launch_slice_copy(v_src, 1, H * D, h0 * D, vc, 0, H_local * D, 0, B, S, H_local, D, P, s);
  if (st != XSTAGE_OK) return st;
  SrcTable t = {};
  for (int p = 0; p < P; ++p) t.q[p] = static_cast<const uint16_t*>(q_src[p]);
  Layout lay;
  lay.src = &t;
  lay.kv_contiguous = 1;
  lay.src_heads = H;
  lay.src_head0 = h0;
  lay.dst_heads = H;
  lay.dst_head0 = h0;
  return launch_attn_any(q_src[0], kc[0], vc[0], make_table(out_dst, P), B, S, H_local, D, P, scale, split_ws,
                         split_ws_bytes, s, 0, nullptr, &lay);
}

int xstage_attn_a2a_plan(int B, int S, int H_local, int D, unsigned long long split_ws_bytes, int* n_workgroups,
                         int* n_split) {
  if (n_workgroups == nullptr) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  *n_workgroups = attn_workgroups(B, S, H_local, D, split_ws_bytes, n_split);
  return XSTAGE_OK;
}

int xstage_attn_a2a_wg_rows(int B, int S, int H_local, int D, unsigned long long split_ws_bytes, int* rows) {
  if (rows == nullptr) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  *rows = attn_wg_rows(B, S, H_local, D, split_ws_bytes);
  return XSTAGE_OK;
}

int xstage_attn_a2a_schedule(int B, int S, int H_local, int D, unsigned long long split_ws_bytes, int cap, int* tile,
                             int* split, int* j0, int* j1, int* n_workgroups) {
  if (n_workgroups == nullptr || cap < 0 || (cap > 0 && (!tile || !split || !j0 || !j1))) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  *n_workgroups = attn_schedule(B, S, H_local, D, split_ws_bytes, cap, tile, split, j0, j1);
  return *n_workgroups > cap ? XSTAGE_ERR_INVALID : XSTAGE_OK;
}

int xstage_attn_a2a_fwd_traced(const void* q, const void* k, const void* v, void* const* out_slabs, int B, int S,
                               int H_local, int D, int P, float scale, int mode, unsigned long long* stamps,
                               void* split_ws, unsigned long long split_ws_bytes, void* stream) {
  if (mode < 0 || mode > 3 || stamps == nullptr || (reinterpret_cast<uintptr_t>(stamps) & 7u) != 0)
    return XSTAGE_ERR_INVALID;
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  // [workgroup][wave][4] 64-bit stamps
  const unsigned long long wsb = split_ws ? split_ws_bytes : 0ull;
  const unsigned long long stamp_bytes = (unsigned long long)attn_workgroups(B, S, H_local, D, wsb, nullptr) *
                                         (unsigned long long)(attn_wg_rows(B, S, H_local, D, wsb) / 32) * 4ull * 8ull;
  const Range sr = range_of(stamps, stamp_bytes);
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  if (q && (overlaps(sr, range_of(q, tb)) || overlaps(sr, range_of(k, tb)) || overlaps(sr, range_of(v, tb))))
    return XSTAGE_ERR_INVALID;
  st = check_attn_slabs(q, k, v, out_slabs, B, S, H_local, D, P, scale, stamps, stamp_bytes, split_ws,
                        split_ws_bytes);
  if (st != XSTAGE_OK) return st;
  return launch_attn_any(q, k, v, make_table(out_slabs, P), B, S, H_local, D, P, scale, split_ws, split_ws_bytes,
                         static_cast<hipStream_t>(stream), 1 + mode, stamps);
}

int xstage_attn_nsplit_ws_size(int B, int S, int H_local, int D, int n_split, unsigned long long* bytes) {
  if (bytes == nullptr) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  bool ok = false;
  const unsigned long long need = attn_ws_forced(B, S, H_local, D, n_split, &ok);
  if (!ok) return XSTAGE_ERR_INVALID;
  *bytes = need;
  return XSTAGE_OK;
}

int xstage_attn_a2a_fwd_nsplit(const void* q, const void* k, const void* v, void* const* out_slabs, int B, int S,
                               int H_local, int D, int P, float scale, int n_split, void* split_ws,
                               unsigned long long split_ws_bytes, void* stream) {
  int st = check_shape(B, S, H_local, D, P);
  if (st != XSTAGE_OK) return st;
  bool ok = false;
  const unsigned long long need = attn_ws_forced(B, S, H_local, D, n_split, &ok);
  if (!ok || (need > 0 && (split_ws == nullptr || split_ws_bytes < need))) return XSTAGE_ERR_INVALID;
  // checked like the product call's workspace, over the bytes this split count uses
  st = check_qkv(q, k, v, scale);
  if (st != XSTAGE_OK) return st;
  const unsigned long long tb = tensor_bytes(B, S, H_local, D);
  const Range wr = need ? range_of(split_ws, need) : Range{0, 0};
  Range others[4] = {range_of(q, tb), range_of(k, tb), range_of(v, tb), wr};
  st = check_split_ws(need ? split_ws : nullptr, wr, others, 3);
  if (st != XSTAGE_OK) return st;
  st = check_slabs(out_slabs, P, tb / (unsigned long long)P, others, 4);
  if (st != XSTAGE_OK) return st;
  return launch_attn_any(q, k, v, make_table(out_slabs, P), B, S, H_local, D, P, scale, need ? split_ws : nullptr,
                         need, static_cast<hipStream_t>(stream), 0, nullptr, nullptr, 0, n_split);
}

int xstage_attn_a2a_fwd_paced(const void* q, const void* k, const void* v, void* const* out_slabs, int B, int S,
                              int H_local, int D, int P, float scale, int chunks, void* stream) {
  const int st = check_attn_slabs(q, k, v, out_slabs, B, S, H_local, D, P, scale, nullptr, 0, nullptr, 0);
  if (st != XSTAGE_OK) return st;
  const int stores_per_lane = 32 * (D / 8) / 64;  // a wave's 32 rows in 16-byte stores: 8 (D=128), 4 (D=64)
  if (chunks < 1 || chunks > stores_per_lane || stores_per_lane % chunks != 0) return XSTAGE_ERR_INVALID;
  return launch_attn_any(q, k, v, make_table(out_slabs, P), B, S, H_local, D, P, scale, nullptr, 0,
                         static_cast<hipStream_t>(stream), kAttnModePaced, nullptr, nullptr, chunks);
}

int xstage_attn_a2a_paced_plan(int B, int S, int H_local, int D, int* n_workgroups, int* n_tiles) {
  if (n_workgroups == nullptr || n_tiles == nullptr) return XSTAGE_ERR_INVALID;
  const int st = check_shape(B, S, H_local, D, 1);
  if (st != XSTAGE_OK) return st;
  int wg = 0;
  const int tiles = attn_paced_workgroups(B, S, H_local, D, &wg);
  if (wg < 1) return XSTAGE_ERR_HIP;
  *n_workgroups = wg;
  *n_tiles = tiles;
  return XSTAGE_OK;
}

static int check_moe_shape(int E, const int* offsets, int d_model, int d_ff, int epw, int schedule,
                           std::vector<int>* rows) {
  if (E < 1 || offsets == nullptr || epw < 1 || (schedule != 0 && schedule != 1)) return XSTAGE_ERR_INVALID;
  if (E > 4096 || epw > kMoeMaxWaveExperts) return XSTAGE_ERR_UNSUPPORTED;
  if (d_model <= 0 || d_ff <= 0 || d_model % 128 != 0 || d_ff % 128 != 0) return XSTAGE_ERR_INVALID;
  if (d_model > 65536 || d_ff > 65536) return XSTAGE_ERR_UNSUPPORTED;
  if (offsets[0] != 0) return XSTAGE_ERR_INVALID;
  rows->resize(E);
  for (int e = 0; e < E; ++e) {
    if (offsets[e + 1] < offsets[e]) return XSTAGE_ERR_INVALID;
    (*rows)[e] = offsets[e + 1] - offsets[e];
  }
  return XSTAGE_OK;
}

static int moe_total_tiles(int E, const std::vector<int>& rows, int d_model, int d_ff) {
  long long n = 0;
  for (int e = 0; e < E; ++e) n += moe_tiles(rows[e], d_ff) + moe_tiles(rows[e], d_model);
  return n > (1 << 30) ? -1 : (int)n;
}

int xstage_moe_waves_plan(int E, const int* expert_offsets, int d_model, int d_ff, int experts_per_wave, int schedule,
                          int* l1_launch, int* l2_launch, int* n_launches, int* n_tiles) {
  std::vector<int> rows;
  const int st = check_moe_shape(E, expert_offsets, d_model, d_ff, experts_per_wave, schedule, &rows);
  if (st != XSTAGE_OK) return st;
  if (!l1_launch || !l2_launch || !n_launches || !n_tiles) return XSTAGE_ERR_INVALID;
  const int nt = moe_total_tiles(E, rows, d_model, d_ff);
  if (nt < 0) return XSTAGE_ERR_UNSUPPORTED;
  MoeShape sh = {E, d_model, d_ff, experts_per_wave, expert_offsets, rows.data()};
  std::vector<MoeLaunch> plan;
  *n_launches = moe_plan(sh, schedule, &plan);
  for (int i = 0; i < (int)plan.size(); ++i) {
    for (int e = plan[i].l1_begin; e < plan[i].l1_end; ++e) l1_launch[e] = i;
    for (int e = plan[i].l2_begin; e < plan[i].l2_end; ++e) l2_launch[e] = i;
  }
  *n_tiles = nt;
  return XSTAGE_OK;
}

int xstage_moe_waves_run(const xstage_moe_params_t* p, void* stream) {
  if (p == nullptr) return XSTAGE_ERR_INVALID;
  std::vector<int> rows;
  int st = check_moe_shape(p->E, p->expert_offsets, p->d_model, p->d_ff, p->experts_per_wave, p->schedule, &rows);
  if (st != XSTAGE_OK) return st;
  if (p->P < 1) return XSTAGE_ERR_INVALID;
  if (p->P > XSTAGE_MAX_P) return XSTAGE_ERR_UNSUPPORTED;
  const void* bf[4] = {p->x, p->w1, p->w2, p->h};
  for (const void* q : bf)
    if (q == nullptr || !aligned16(q)) return XSTAGE_ERR_INVALID;
  if (!p->dst_slab || !p->dst_row || (reinterpret_cast<uintptr_t>(p->dst_slab) & 3u) ||
      (reinterpret_cast<uintptr_t>(p->dst_row) & 3u) || !p->out || !p->out_rows)
    return XSTAGE_ERR_INVALID;
  if (p->stamps && (reinterpret_cast<uintptr_t>(p->stamps) & 7u)) return XSTAGE_ERR_INVALID;
  const int nt = moe_total_tiles(p->E, rows, p->d_model, p->d_ff);
  if (nt < 0) return XSTAGE_ERR_UNSUPPORTED;
  const unsigned long long T = (unsigned long long)p->expert_offsets[p->E];
  const unsigned long long E = (unsigned long long)p->E, dm = p->d_model, df = p->d_ff;
  // Everything read, then everything written: each written range must be disjoint from all.
  std::vector<Range> reads = {range_of(p->x, T * dm * 2), range_of(p->w1, E * df * dm * 2),
                              range_of(p->w2, E * dm * df * 2), range_of(p->dst_slab, T * 4),
                              range_of(p->dst_row, T * 4)};
  std::vector<Range> writes = {range_of(p->h, T * df * 2)};
  for (int q = 0; q < p->P; ++q) {
    if (p->out[q] == nullptr || !aligned16(p->out[q]) || p->out_rows[q] < 0) return XSTAGE_ERR_INVALID;
    writes.push_back(range_of(p->out[q], (unsigned long long)p->out_rows[q] * dm * 2));
  }
  if (p->stamps) writes.push_back(range_of(p->stamps, (unsigned long long)nt * 16 * 8));
  for (size_t a = 0; a < writes.size(); ++a) {
    for (const Range& r : reads)
      if (overlaps(writes[a], r)) return XSTAGE_ERR_INVALID;
    for (size_t b = 0; b < a; ++b)
      if (overlaps(writes[a], writes[b])) return XSTAGE_ERR_INVALID;
  }
  if (T == 0) return XSTAGE_OK;
  MoeShape sh = {p->E, p->d_model, p->d_ff, p->experts_per_wave, p->expert_offsets, rows.data()};
  MoeBuffers buf = {};
  buf.x = static_cast<const uint16_t*>(p->x);
  buf.w1 = static_cast<const uint16_t*>(p->w1);
  buf.w2 = static_cast<const uint16_t*>(p->w2);
  buf.h = static_cast<uint16_t*>(p->h);
  buf.dst_slab = p->dst_slab;
  buf.dst_row = p->dst_row;
  buf.P = p->P;
  for (int q = 0; q < p->P; ++q) {
    buf.out[q] = static_cast<uint16_t*>(p->out[q]);
    buf.out_rows[q] = p->out_rows[q];
  }
  buf.stamps = p->stamps;
  return launch_moe(sh, buf, p->schedule, static_cast<hipStream_t>(stream));
}

int xstage_burst_gap_run(const xstage_bg_params_t* p, void* stream) {
  if (p == nullptr) return XSTAGE_ERR_INVALID;
  if (p->K < 1 || p->K > 4096 || p->rounds < 1 || p->rounds > 65536 || p->n_dst_sets < 1) return XSTAGE_ERR_INVALID;
  if (p->nontemporal != 0 && p->nontemporal != 1) return XSTAGE_ERR_INVALID;
  if (p->stamps == nullptr || (reinterpret_cast<uintptr_t>(p->stamps) & 7u) != 0) return XSTAGE_ERR_INVALID;
  if (p->V_bytes % (4096ull * (unsigned long long)p->K) != 0) return XSTAGE_ERR_INVALID;
  if (p->V_bytes > 0 && (p->dst == nullptr || !aligned16(p->dst))) return XSTAGE_ERR_INVALID;
  if (p->sync != nullptr) {
    if ((reinterpret_cast<uintptr_t>(p->sync) & 3u) != 0) return XSTAGE_ERR_INVALID;
    if (p->sync_timeout_ticks < 1 || p->sync_timeout_ticks > 1000000000ull) return XSTAGE_ERR_INVALID;
    const Range sr = range_of(p->sync, (unsigned long long)p->rounds * 4ull);
    if (overlaps(sr, range_of(p->stamps, (unsigned long long)p->K * p->rounds * 24ull))) return XSTAGE_ERR_INVALID;
    if (p->V_bytes > 0 && overlaps(sr, range_of(p->dst, (unsigned long long)p->n_dst_sets * p->V_bytes)))
      return XSTAGE_ERR_INVALID;
  }
  return launch_burst_gap(*p, static_cast<hipStream_t>(stream));
}

int xstage_wallclock_hz(double* hz) {
  if (hz == nullptr) return XSTAGE_ERR_INVALID;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return XSTAGE_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return XSTAGE_ERR_HIP;
  *hz = (double)khz * 1e3;
  return XSTAGE_OK;
}

double xstage_bg_t_iss(double G_s, double T0_s, double V_bytes, double R_bytes_per_s) {
  if (!(R_bytes_per_s > 0) || !isfinite(G_s) || !isfinite(T0_s) || !isfinite(V_bytes) || !isfinite(R_bytes_per_s))
    return -1.0;
  const double drain = V_bytes / R_bytes_per_s - G_s;
  return drain > T0_s ? drain : T0_s;
}

int xstage_bg_pacing_chunks(double V_bytes, double G_s, double a_s, double f1_Bps, double R_Bps, double Q_bytes,
                            int c_max, double* t_visible_s) {
  const double in[6] = {V_bytes, G_s, a_s, f1_Bps, R_Bps, Q_bytes};
  for (double x : in)
    if (!isfinite(x) || x < 0) return 0;
  if (!(R_Bps > 0) || !(f1_Bps > 0) || c_max < 1) return 0;
  int best = 1;
  double best_t = 0.0;
  for (int c = 1; c <= c_max; ++c) {
    const double issue = c * a_s + V_bytes / f1_Bps;
    const double hidden = G_s < c * Q_bytes / R_Bps ? G_s : c * Q_bytes / R_Bps;
    const double drain = V_bytes / R_Bps - hidden;
    const double t = issue > drain ? issue : drain;
    if (c == 1 || t < best_t) {
      best = c;
      best_t = t;
    }
  }
  if (t_visible_s) *t_visible_s = best_t;
  return best;
}

const char* xstage_status_str(int status) {
  switch (status) {
    case XSTAGE_OK: return "XSTAGE_OK";
    case XSTAGE_ERR_INVALID: return "XSTAGE_ERR_INVALID";
    case XSTAGE_ERR_UNSUPPORTED: return "XSTAGE_ERR_UNSUPPORTED";
    case XSTAGE_ERR_HIP: return "XSTAGE_ERR_HIP";
    default: return "XSTAGE_UNKNOWN_STATUS";
  }
}

}  // extern "C"
