// Device-side building blocks shared by the libxstage kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xstage.h"

namespace xstage {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;  // global-memory 16-byte chunk

// Destination table of the post-attention all-to-all: P receive buffers, passed by value in
// the kernel arguments (no device-side table, nothing allocated).
struct SlabTable {
  uint16_t* p[XSTAGE_MAX_P];
};

// Sequence shards of q, k and v, read in place (the pre-attention all-to-all): shard p holds
// rows [p * S/P, (p + 1) * S/P) of every head.  Passed by value in kernel arguments.
constexpr int kMaxSrc = 32;
struct SrcTable {
  const uint16_t* q[kMaxSrc];
  const uint16_t* k[kMaxSrc];
  const uint16_t* v[kMaxSrc];
};

// Where a launch reads its inputs and writes its outputs, beyond the plain layouts
// (q, k, v contiguous [B, S, H, D]; slabs [B, S/P, H, D]).
struct Layout {
  const SrcTable* src = nullptr;  // non-null: inputs are P shards [B, S/P, src_heads, D]
  int src_heads = 0, src_head0 = 0;  // shard row width (heads) and this call's first head
  int dst_heads = 0, dst_head0 = 0;  // slab row width (heads) and this call's first column
  int kv_contiguous = 0;  // with src: only Q from the shards, K and V from contiguous
                          // [B, S, H_local, D] tensors (the k, v arguments)
};

constexpr float kLog2e = 1.4426950408889634f;

// 32-lane halves of a wave64 swap: returns, in every lane, max(x[lane], x[lane ^ 32]).
__device__ __forceinline__ float max_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two fp32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

}  // namespace xstage
