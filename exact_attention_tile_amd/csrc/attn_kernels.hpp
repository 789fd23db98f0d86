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
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  int B, H, N;       // N: sequence length (fixed-length calls)
  int Hkv;           // K/V heads; query head h reads K/V head h / group
  int group;         // H / Hkv
  const int* cu;     // variable-length calls: device [B+1] token offsets, else null
  int total;         // variable-length calls: tokens in the packed tensors
  int maxlen;        // longest sequence (N for fixed-length calls)
  int n_qtiles;      // ceil(maxlen / rows per workgroup)
  int remap;         // XCD-aware block order (items divisible by 8): 1 head-major, 2 tile-major
  int items;         // work items: (batch*head, query tile) pairs of the block order
  int persist;       // 1: gridDim.x work-groups (a multiple of 8) loop over the items
  float c;           // |scale| * log2(e): scores are kept in log2 units
  unsigned qsign;    // sign-flip mask applied to Q when scale < 0
};

// The sequence one work-group works on: its length and the element offsets
// of its first token in Q/O ([tokens][H][d]) and K/V ([tokens][Hkv][d]) and
// of its first row in the log-sum-exp ([B][H][N], or [H][total] for
// variable-length calls).
struct SeqView {
  int N;
  int hk;            // K/V head
  long long q_base, kv_base, lse_base;
};

// Fills `v` for (batch b, query head h) and returns false when the
// work-group has nothing to do: its first query row q0 lies past the end of
// the sequence, or the sequence's offsets are malformed (negative, not
// increasing, past `total`, or longer than `maxlen`) -- such a sequence is
// skipped and nothing outside the tensors is ever touched.
__device__ __forceinline__ bool seq_view(const FwdParams& p, int D, int b, int h, int q0, SeqView& v) {
  long long seq0;
  int n;
  if (p.cu) {
    const int s0 = p.cu[b];
    const int s1 = p.cu[b + 1];
    if (s0 < 0 || s1 < s0 || s1 > p.total || s1 - s0 > p.maxlen) return false;
    seq0 = s0;
    n = s1 - s0;
  } else {
    seq0 = (long long)b * p.N;
    n = p.N;
  }
  if (q0 >= n) return false;
  v.N = n;
  v.hk = h / p.group;
  v.q_base = (seq0 * p.H + h) * D;
  v.kv_base = (seq0 * p.Hkv + v.hk) * D;
  v.lse_base = p.cu ? (long long)h * p.total + seq0 : ((long long)b * p.H + h) * n;
  return true;
}

// Maps the launch index to (batch*head, query tile).  Work-groups are handed
// to the 8 XCDs round-robin (block i -> XCD i % 8), so when the grid is a
// multiple of 8 the index is first regrouped so that consecutive logical
// blocks -- the query tiles of one head, which share its K/V -- land on one
// XCD and share its L2.  Within a head, tiles go longest-first (for causal
// attention the last query tile sees the most keys).  Causal calls with few
// query tiles per head (remap == 2, chosen by the host) keep each XCD's share
// of heads but run the longest tile of every head first, then the next
// longest: the tile lengths then pair up over the XCD's CUs.
//
// Variable-length calls order the work differently: sequence lengths vary,
// so a contiguous run of heads per XCD would give one XCD all of a long
// sequence.  Instead every XCD gets the same share of every sequence: with H
// a multiple of 8, XCD x takes heads x, x+8, ... of each sequence.  It runs
// them sequence by sequence, longest sequence first (ranked on the device
// from the offsets), a sequence's heads one after the other and a head's
// query tiles last (longest) first.  So the XCD's CUs share one or two heads'
// K/V in L2 at a time, and the last work-groups are the short ones.  Other
// shapes send unit bh to XCD bh % 8 and run query-tile-major.  Work-groups
// past the end of a short sequence exit at once.
//
// The sequence of rank r (by length, longest first, ties by index) of a
// batch of B <= 128 sequences; each lane ranks up to two candidates.
__device__ __forceinline__ int seq_by_rank(const int* cu, int B, int r) {
  const int lane = threadIdx.x & 63;
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int b = c0 + lane;
    int rank = -1;
    if (b < B) {
      const int len = cu[b + 1] - cu[b];
      rank = 0;
      for (int i = 0; i < B; ++i) {
        const int li = cu[i + 1] - cu[i];
        rank += (li > len) || (li == len && i < b);
      }
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(rank == r);
    if (hit) return c0 + __builtin_ctzll(hit);
  }
  return 0;   // unreachable: the ranks are a permutation of 0 .. B-1
}

__device__ __forceinline__ void block_to_work(const FwdParams& p, int L, int& bh, int& qt) {
  const int total = p.items;
  if (p.cu) {
    const int BH = p.B * p.H;
    if ((p.H & 7) == 0 && p.B <= 128) {
      const int hx = p.H >> 3;                     // heads per XCD per sequence
      const int k = L >> 3;
      const int j = k / p.n_qtiles;
      qt = p.n_qtiles - 1 - (k - j * p.n_qtiles);
      const int r = j / hx;
      const int b = seq_by_rank(p.cu, p.B, r);
      bh = b * p.H + (L & 7) + 8 * (j - r * hx);
    } else if ((BH & 7) == 0) {
      const int per = BH >> 3;
      const int k = L >> 3;
      const int t = k / per;
      qt = p.n_qtiles - 1 - t;
      bh = (L & 7) + 8 * (k - t * per);
    } else {
      const int t = L / BH;
      qt = p.n_qtiles - 1 - t;
      bh = L - t * BH;
    }
    return;
  }
  if (p.remap == 2) {
    // XCD x takes heads x*hx .. x*hx+hx-1 (B*H = 8*hx), the longest query
    // tile of each of them first, then the next longest, ...
    const int hx = (p.B * p.H) >> 3;
    const int k = L >> 3;
    const int t = k / hx;
    bh = (L & 7) * hx + (k - t * hx);
    qt = p.n_qtiles - 1 - t;
    return;
  }
  if (p.remap) {
    int per = total >> 3;
    L = (L & 7) * per + (L >> 3);
  }
  bh = L / p.n_qtiles;
  qt = p.n_qtiles - 1 - (L - bh * p.n_qtiles);
}

// Work item L of this work-group's step s.  One work-group per item
// (persist 0): the work-group's own index, step 0 only.  Persistent launch
// (gridDim.x work-groups, a multiple of 8, one per compute unit): item L
// belongs to XCD L % 8 in the block order, and work-group g runs on XCD
// g % 8, so each XCD's W = gridDim.x / 8 work-groups take that XCD's items
// (local index k = L / 8, longest first) in rounds of W.  The order within
// a round is serpentine: work-group j takes the j-th item in even rounds
// and the (W-1-j)-th in odd ones, which pairs long causal tiles with short
// ones.  Returns false once the XCD's items are used up.
__device__ __forceinline__ bool item_of_n(int items, int persist, int s, int& L) {
  if (!persist) {
    L = blockIdx.x;
    return s == 0;
  }
  const int g = blockIdx.x;
  const int j = g >> 3, W = gridDim.x >> 3;
  const int k = s * W + ((s & 1) ? W - 1 - j : j);
  if (k >= (items >> 3)) return false;
  L = (g & 7) + 8 * k;
  return true;
}
__device__ __forceinline__ bool item_of(const FwdParams& p, int s, int& L) {
  return item_of_n(p.items, p.persist, s, L);
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

// ---- LDS-DMA tile loads (global_load_lds_dwordx4) ---------------------------
// One instruction moves 1 KiB: lane l reads 16 bytes at its global address
// and writes them to LDS bytes [M0 + imm + 16 l, +16).  The immediate offset
// imm is added to both the global and the LDS address, so up to four loads
// (imm = 0, 1024, 2048, 3072) share one M0 value, provided each lane's
// global offset for load i is stored less 1024 i.  An SALU write of M0
// needs one wait state before an LDS-DMA instruction reads it (the s_nop).
// The loads are inline asm so that the compiler does not order them against
// LDS reads of other buffers; the caller waits for them (vmcnt).
//
// lds_dma_s<C>: C loads from the SGPR base plus the lanes' 32-bit offsets
// go[0..C-1] (go[i] = byte offset - 1024 i), into LDS from m0.
template <int C>
__device__ __forceinline__ void lds_dma_s(unsigned m0, const unsigned* go, const void* base) {
  static_assert(C >= 1 && C <= 4, "one M0 value covers four loads");
  if constexpr (C == 1) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(m0), "v"(go[0]), "s"(base) : "memory");
  } else if constexpr (C == 2) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %3\n\t"
                 "global_load_lds_dwordx4 %2, %3 offset:1024"
                 ::"s"(m0), "v"(go[0]), "v"(go[1]), "s"(base) : "memory");
  } else if constexpr (C == 3) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %4\n\t"
                 "global_load_lds_dwordx4 %2, %4 offset:1024\n\t"
                 "global_load_lds_dwordx4 %3, %4 offset:2048"
                 ::"s"(m0), "v"(go[0]), "v"(go[1]), "v"(go[2]), "s"(base) : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %5\n\t"
                 "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
                 "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
                 "global_load_lds_dwordx4 %4, %5 offset:3072"
                 ::"s"(m0), "v"(go[0]), "v"(go[1]), "v"(go[2]), "v"(go[3]), "s"(base) : "memory");
  }
}
// lds_dma_v<C>: the same from per-lane 64-bit addresses g[i] (each 1024 i
// bytes below the data it loads).
template <int C>
__device__ __forceinline__ void lds_dma_v(unsigned m0, const void* const* g) {
  static_assert(C >= 1 && C <= 4, "one M0 value covers four loads");
  if constexpr (C == 1) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(m0), "v"(g[0]) : "memory");
  } else if constexpr (C == 2) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "global_load_lds_dwordx4 %2, off offset:1024"
                 ::"s"(m0), "v"(g[0]), "v"(g[1]) : "memory");
  } else if constexpr (C == 3) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "global_load_lds_dwordx4 %2, off offset:1024\n\t"
                 "global_load_lds_dwordx4 %3, off offset:2048"
                 ::"s"(m0), "v"(g[0]), "v"(g[1]), "v"(g[2]) : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "global_load_lds_dwordx4 %2, off offset:1024\n\t"
                 "global_load_lds_dwordx4 %3, off offset:2048\n\t"
                 "global_load_lds_dwordx4 %4, off offset:3072"
                 ::"s"(m0), "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]) : "memory");
  }
}
// N loads of one wave (LDS bytes m0 + 1024 i for load i): groups of four,
// one M0 write per group.
template <int N, int G = 0>
__device__ __forceinline__ void lds_dma_tile_s(unsigned m0, const unsigned* go, const void* base) {
  if constexpr (G < N) {
    lds_dma_s<(N - G < 4 ? N - G : 4)>(m0 + G * 1024, go + G, base);
    lds_dma_tile_s<N, G + 4>(m0, go, base);
  }
}
template <int N, int G = 0>
__device__ __forceinline__ void lds_dma_tile_v(unsigned m0, const void* const* gp) {
  if constexpr (G < N) {
    lds_dma_v<(N - G < 4 ? N - G : 4)>(m0 + G * 1024, gp + G);
    lds_dma_tile_v<N, G + 4>(m0, gp);
  }
}

// Host side: enqueues `kernel` on `stream` and returns the status of that
// launch alone (hipGetLastError would also report an earlier, unrelated
// failure on the calling thread).  The arguments are taken by value with
// the kernel's own parameter types.
template <typename T> struct same_type { using type = T; };

template <typename... KArgs>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block,
                                hipStream_t stream, typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}

}  // namespace attn
