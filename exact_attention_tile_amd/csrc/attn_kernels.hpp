// Device-side building blocks shared by the bf16 and fp8 attention kernels
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

// Launch parameters common to both entry points.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* dq;   // fp8 only: per-(b,h) descales, device
  const float* dk;
  const float* dv;
  int B, H, N;
  int n_qtiles;      // ceil(N / rows per workgroup)
  int remap;         // 1: XCD-aware block order (grid size divisible by 8)
  float c;           // |scale| * log2(e): scores are kept in log2 units
  unsigned qsign;    // sign-flip mask applied to Q when scale < 0
};

// Maps the launch index to (batch*head, query tile).  Work-groups are handed
// to the 8 XCDs round-robin (block i -> XCD i % 8), so when the grid is a
// multiple of 8 the index is first regrouped so that consecutive logical
// blocks -- the query tiles of one head, which share its K/V -- land on one
// XCD and share its L2.  Within a head, tiles go longest-first (for causal
// attention the last query tile sees the most keys).
__device__ __forceinline__ void block_to_work(const FwdParams& p, int& bh, int& qt) {
  int total = gridDim.x;
  int L = blockIdx.x;
  if (p.remap) {
    int per = total >> 3;
    L = (L & 7) * per + (L >> 3);
  }
  bh = L / p.n_qtiles;
  qt = p.n_qtiles - 1 - (L - bh * p.n_qtiles);
}

// The two lane halves of a wave hold the same query column; these combine
// a per-lane value with the one held by lane ^ 32.  permlane32_swap returns
// {own, partner} in some order in every lane, so max/sum of the pair need no
// lane test.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16x2 (round to nearest even), one v_cvt_pk_bf16_f32;
// a in the low half
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
}

}  // namespace attn
