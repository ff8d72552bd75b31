// Host-side argument checks of the C ABI.  Pure C++ (no HIP calls): every check runs before
// anything is launched, so a rejected call touches no device memory.
#pragma once

#include <stdint.h>

#include <cmath>

#include "xstage.h"

namespace xstage {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline Range range_of(const void* p, unsigned long long bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

// Shape checks shared by every attention / scatter entry point.
inline int check_shape(int B, int S, int H, int D, int P) {
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || P <= 0) return XSTAGE_ERR_INVALID;
  if (D != 64 && D != 128) return XSTAGE_ERR_UNSUPPORTED;
  if (P > XSTAGE_MAX_P) return XSTAGE_ERR_UNSUPPORTED;
  if (S % P != 0) return XSTAGE_ERR_INVALID;
  // Kernels index one tensor with 32-bit element offsets: keep B*S*H*D below 2^31.
  const unsigned long long elems = static_cast<unsigned long long>(B) * static_cast<unsigned long long>(S) *
                                   static_cast<unsigned long long>(H) * static_cast<unsigned long long>(D);
  if (elems >= (1ull << 31)) return XSTAGE_ERR_UNSUPPORTED;
  return XSTAGE_OK;
}

inline unsigned long long tensor_bytes(int B, int S, int H, int D) {
  return static_cast<unsigned long long>(B) * S * H * D * 2ull;
}

// Checks the P slab pointers: non-null, aligned, pairwise disjoint and disjoint from every
// range in `others` (n_others entries).
inline int check_slabs(void* const* slabs, int P, unsigned long long slab_bytes, const Range* others, int n_others) {
  if (slabs == nullptr) return XSTAGE_ERR_INVALID;
  for (int p = 0; p < P; ++p) {
    if (slabs[p] == nullptr || !aligned16(slabs[p])) return XSTAGE_ERR_INVALID;
    const Range rp = range_of(slabs[p], slab_bytes);
    for (int o = 0; o < n_others; ++o)
      if (overlaps(rp, others[o])) return XSTAGE_ERR_INVALID;
    for (int r = 0; r < p; ++r)
      if (overlaps(rp, range_of(slabs[r], slab_bytes))) return XSTAGE_ERR_INVALID;
  }
  return XSTAGE_OK;
}

inline int check_qkv(const void* q, const void* k, const void* v, float scale) {
  if (q == nullptr || k == nullptr || v == nullptr) return XSTAGE_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return XSTAGE_ERR_INVALID;
  if (!std::isfinite(scale)) return XSTAGE_ERR_INVALID;
  return XSTAGE_OK;
}

}  // namespace xstage
