// E4M3 quantisation of attention inputs for the fp8 entry points, with the
// optional random Hadamard rotation ("FlashAttention-3: Pipeline Assíncrono
// com Warp Specialization, WGMMA e FP8 no Hopper e Blackwell", section
// "Estabilidade em FP8: Algoritmo de 2 Passos e Incoherent Processing":
// multiplying by a random orthogonal Hadamard matrix spreads outliers over
// all dimensions).  Applied to the rows of Q and K with the same signs,
// M = diag(s) H_d / sqrt(d) leaves Q K^T unchanged.
//
// Four launches on the caller's stream:
//   amax    y = x diag(s) H_d for every row (sign flips, then the fast
//           Walsh-Hadamard butterfly in binary32, strides 1, 2, ..., d/2,
//           (a, b) -> (a + b, a - b)); each work-group (128 rows of one
//           (batch, head)) stores its max |y| as a partial, in the codes
//           buffer, which is free until the codes launch;
//   reduce  descale[bh] = max of the head's partials (plain loads and
//           stores: same-address atomics from every work-group serialise
//           at the memory side and cost more than this launch);
//   codes   y again, v = y / (amax / 448) correctly rounded in binary32,
//           clamped to +-448, rounded to nearest even onto E4M3
//           (v_cvt_pk_fp8_f32);
//   final   descale[bh] = amax / 448, times 1/sqrt(d) (rounded once to
//           binary32) with the rotation, so that code * descale
//           approximates x M.
// Every rounding decision is taken in binary32 in a fixed order, so the
// codes are reproducible bit for bit.
//
// A row of d values is spread over d/32 lanes holding 32 consecutive values
// each (four 16-byte loads, two 16-byte stores): butterfly strides 1 to 16
// stay inside a lane, strides 32 and 64 pair lane l with lane l ^ 1 and
// l ^ 2 of the same row through data-parallel-primitive moves.  Each thread
// loads all of its rows before transforming any.  Inputs are expected
// finite.
#include <cmath>

#include "attn_kernels.hpp"

namespace attn {

struct QuantParams {
  const void* x;
  void* codes;
  float* descale;          // [B][H]: the maximum between reduce and final
  const unsigned* signs;   // d/32 words, bit i = sign of column i; null: no rotation
  int N, H, nchunks;
};

constexpr int kQuantThreads = 256;
constexpr int kQuantRows = 128;   // rows of one (batch, head) per work-group

// The value of lane l ^ M (M = 1 or 2: the partner inside a row of 2 or 4
// lanes), by a quad permutation.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(M == 1 || M == 2, "lane_xor: 1 or 2");
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;          // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

template <int D>
struct QuantRow {
  static constexpr int L = D / 32;                  // lanes per row
  static constexpr int R = kQuantThreads / L;       // rows per pass
  static constexpr int T = kQuantRows / R;          // rows per thread
  using Raw = u32x4[4];
  float y[32];

  // bf16 -> binary32 (exact), then with the rotation: sign flips (exact) and
  // the butterfly.  Across lanes (a, b) -> (a + b, a - b) is one fused
  // multiply-add per value, fma(+-1, mine, partner): the lower lane gets
  // mine + partner, the upper partner - mine, each rounded once as the
  // plain sum or difference is.
  __device__ __forceinline__ void decode(const Raw& w, unsigned sb, bool rot) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * c + 2 * e] = __uint_as_float(w[c][e] << 16);
        y[8 * c + 2 * e + 1] = __uint_as_float(w[c][e] & 0xFFFF0000u);
      }
    }
    if (!rot) return;
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = __uint_as_float(__float_as_uint(y[j]) ^ (((sb >> j) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 32; h *= 2) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if ((j & h) == 0) {
          const float a = y[j];
          const float b = y[j + h];
          y[j] = a + b;
          y[j + h] = a - b;
        }
      }
    }
    const int l = threadIdx.x % L;
    cross<1>(l);
    if constexpr (L == 4) cross<2>(l);
  }

  template <int M>
  __device__ __forceinline__ void cross(int l) {
    const float sgn = (l & M) ? -1.f : 1.f;
    float o[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = lane_xor<M>(y[j]);
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = __builtin_fmaf(sgn, y[j], o[j]);
  }
};

// The rows of one thread, loaded before any is transformed; rows past the
// chunk's end are not loaded (they decode to zeros).
template <int D>
__device__ __forceinline__ void load_rows(const __bf16* xg, long long tok, int n, int n1,
                                          typename QuantRow<D>::Raw (&w)[QuantRow<D>::T]) {
#pragma unroll
  for (int t = 0; t < QuantRow<D>::T; ++t) {
    const int r = n + t * QuantRow<D>::R;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      w[t][c] = r < n1 ? *(const u32x4*)(xg + r * tok + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }
}

struct QuantGeom {
  int bh, chunk, l, n, n1;
  long long tok, off;
};

template <int D>
__device__ __forceinline__ QuantGeom quant_geom(const QuantParams& p) {
  QuantGeom g;
  g.bh = blockIdx.x / p.nchunks;
  g.chunk = blockIdx.x - g.bh * p.nchunks;
  g.l = threadIdx.x % QuantRow<D>::L;
  g.tok = (long long)p.H * D;
  const int b = g.bh / p.H;
  g.off = ((long long)b * p.N * p.H + (g.bh - b * p.H)) * D + 32 * g.l;
  g.n = g.chunk * kQuantRows + threadIdx.x / QuantRow<D>::L;
  g.n1 = min(p.N, (g.chunk + 1) * kQuantRows);
  return g;
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void attn_quant_amax_kernel(QuantParams p) {
  using Row = QuantRow<D>;
  __shared__ float red[kQuantThreads / 64];
  const QuantGeom g = quant_geom<D>(p);
  const bool rot = p.signs != nullptr;
  const unsigned sb = rot ? p.signs[g.l] : 0u;
  typename Row::Raw w[Row::T];
  load_rows<D>((const __bf16*)p.x + g.off, g.tok, g.n, g.n1, w);
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < Row::T; ++t) {
    Row r;
    r.decode(w[t], sb, rot);
#pragma unroll
    for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(r.y[j]));
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kQuantThreads / 64; ++i) m = fmaxf(m, red[i]);
    ((float*)p.codes)[blockIdx.x] = m;
  }
}

// One wave per (batch, head): the maximum of its work-groups' partials.
__global__ __launch_bounds__(256) void attn_quant_reduce_kernel(QuantParams p, int bh_count) {
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= bh_count) return;
  const float* part = (const float*)p.codes + (long long)bh * p.nchunks;
  float m = 0.f;
  for (int i = threadIdx.x & 63; i < p.nchunks; i += 64) m = fmaxf(m, part[i]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((threadIdx.x & 63) == 0) p.descale[bh] = m;
}

// y / div correctly rounded.  FAST: q0 = y * rcp with rcp = RN(1/div), the
// remainder y - q0 div (exact by fma), one correction step (Markstein's
// theorem: with the reciprocal correctly rounded and q0 within an ulp,
// RN(q0 + rem * rcp) is the correctly rounded quotient), and the sign of y
// put back so that -0 stays -0.  The remainder must not underflow, which
// holds for every quotient that can reach a nonzero code once div >= 2^-60;
// below that the plain division runs.
template <bool FAST>
__device__ __forceinline__ float quotient(float y, float div, float rcp) {
  if constexpr (FAST) {
    const float q0 = y * rcp;
    const float rem = __builtin_fmaf(-q0, div, y);
    return __builtin_copysignf(__builtin_fmaf(rem, rcp, q0), y);
  } else {
    return y / div;
  }
}

template <int D, bool FAST>
__device__ __forceinline__ void quant_rows(const QuantParams& p, const QuantGeom& g, unsigned sb,
                                           bool rot, const typename QuantRow<D>::Raw (&w)[QuantRow<D>::T],
                                           float div, float rcp) {
  using Row = QuantRow<D>;
  unsigned char* cg = (unsigned char*)p.codes + g.off;
#pragma unroll
  for (int t = 0; t < Row::T; ++t) {
    const int rr = g.n + t * Row::R;
    Row r;
    r.decode(w[t], sb, rot);
    if (rr >= g.n1) continue;
    unsigned out[8];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = __builtin_amdgcn_fmed3f(quotient<FAST>(r.y[j + e], div, rcp), -448.f, 448.f);
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], c, true);
      out[j / 4] = (unsigned)c;
    }
    u32x4* dst = (u32x4*)(cg + rr * g.tok);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  }
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void attn_quant_codes_kernel(QuantParams p) {
  using Row = QuantRow<D>;
  const QuantGeom g = quant_geom<D>(p);
  const bool rot = p.signs != nullptr;
  const unsigned sb = rot ? p.signs[g.l] : 0u;
  typename Row::Raw w[Row::T];
  load_rows<D>((const __bf16*)p.x + g.off, g.tok, g.n, g.n1, w);
  const float ds = p.descale[g.bh] / 448.f;
  const float div = ds > 0.f ? ds : 1.f;
  if (div >= 0x1p-60f)
    quant_rows<D, true>(p, g, sb, rot, w, div, 1.f / div);
  else
    quant_rows<D, false>(p, g, sb, rot, w, div, 0.f);
}

__global__ __launch_bounds__(256) void attn_quant_final_kernel(float* descale, int n, float post) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float ds = descale[i] / 448.f;
    descale[i] = post > 0.f ? ds * post : ds;
  }
}

hipError_t launch_quant(const void* x, void* codes, float* descale, const unsigned* signs, int B,
                        int N, int H, int d, hipStream_t stream) {
  const int bh = B * H;
  const int nchunks = (N + kQuantRows - 1) / kQuantRows;
  QuantParams prm = {x, codes, descale, signs, N, H, nchunks};
  const dim3 grid((unsigned)(bh * nchunks));
  // stop at the first launch that fails: the later kernels read what the
  // earlier ones write
  hipError_t e = d == 128
      ? launch_kernel(attn_quant_amax_kernel<128>, grid, dim3(kQuantThreads), stream, prm)
      : launch_kernel(attn_quant_amax_kernel<64>, grid, dim3(kQuantThreads), stream, prm);
  if (e != hipSuccess) return e;
  e = launch_kernel(attn_quant_reduce_kernel, dim3((bh + 3) / 4), dim3(256), stream, prm, bh);
  if (e != hipSuccess) return e;
  e = d == 128 ? launch_kernel(attn_quant_codes_kernel<128>, grid, dim3(kQuantThreads), stream, prm)
               : launch_kernel(attn_quant_codes_kernel<64>, grid, dim3(kQuantThreads), stream, prm);
  if (e != hipSuccess) return e;
  // 1/sqrt(d) rounded once to binary32 (exact for d = 64)
  const float post = signs ? (float)(1.0 / std::sqrt((double)d)) : 0.f;
  const int small = (bh + 255) / 256 < 1024 ? (bh + 255) / 256 : 1024;
  return launch_kernel(attn_quant_final_kernel, dim3(small), dim3(256), stream, descale, bh, post);
}

}  // namespace attn
