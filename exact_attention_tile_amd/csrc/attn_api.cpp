// C ABI of the tiled exact attention forward, its backward pass and the fp8
// quantiser (declared in include/attn.h).
//
// Every argument is validated on the host before any HIP call; on error
// nothing is launched.  On success the entry point's kernels are enqueued on
// the caller's stream in order: one for a single-pass forward, two for the
// two-pass fp8 forward, three for the backward pass, four for the
// quantiser.  The library allocates, frees and synchronises nothing; the
// backward pass's workspace is the caller's.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>
#include <stdint.h>

#include "attn_kernels.hpp"

namespace attn {
int bf16_rows_per_block(int d);
hipError_t launch_bf16(const FwdParams& prm, int d, int causal, int grid, hipStream_t stream);
int fp8_rows_per_block(int d);
hipError_t launch_fp8(const FwdParams& prm, int d, int causal, int grid, bool two_pass,
                      hipStream_t stream);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int B, int H, int N, int d, int causal, float scale,
                           int cus, hipStream_t stream);
hipError_t launch_quant(const void* x, void* codes, float* descale, const unsigned* signs, int B,
                        int N, int H, int d, hipStream_t stream);
}  // namespace attn

namespace {

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Checks common to every entry point: the tensor pointers, the scalar
// arguments and the sizes.  `tokens` is the number of token rows in each
// tensor (B*N, or the packed total), H/Hkv the query and K/V heads.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int64_t tokens, int H, int Hkv, int d, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (tokens <= 0 || H <= 0 || Hkv <= 0) return ATTN_ERR_INVALID_ARG;
  if (H % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  // element count tokens*H*d must fit in int64 (and the per-head row
  // offsets the kernels form from it)
  const int64_t lim = INT64_MAX / 4;
  int64_t n = tokens;
  if (n > lim / H) return ATTN_ERR_INVALID_ARG;
  n *= H;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (n > lim / d) return ATTN_ERR_INVALID_ARG;
  // the kernels form the byte offset of a K/V row within one tile (up to 128
  // rows of H*d elements) in 32 bits
  if ((int64_t)H * d > (1 << 24)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)lse & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int validate_fixed(int B, int N, int64_t* tokens) {
  if (B <= 0 || N <= 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B > (INT64_MAX / 4) / N) return ATTN_ERR_INVALID_ARG;
  *tokens = (int64_t)B * N;
  return ATTN_OK;
}

// Compute units of the current device, read once per device (0 when it
// cannot be read: then every launch has one work-group per item).
int device_compute_units() {
  static std::atomic<int> known[64];   // 0: not read yet, -1: unavailable
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = known[dev].load(std::memory_order_relaxed);
    if (v != 0) return v > 0 ? v : 0;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = -1;
  if (dev < 64) known[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? n : 0;
}

int validate_descales(const float* dq, const float* dk, const float* dv) {
  if (!dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)dq & 3u) || ((uintptr_t)dk & 3u) || ((uintptr_t)dv & 3u)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Work-group count and block order for one call.  The grid has one
// work-group per (batch, head, query tile of the longest sequence); it must
// fit the 32-bit grid.  Block order (fixed-length calls, the kernels'
// block_to_work): with the grid a multiple of 8 each XCD takes a contiguous
// share of the heads.  It runs them head by head (a head's K/V in its L2),
// except for causal calls with fewer than 32 query tiles per head and a
// head count divisible by 8: those run their heads' longest tiles first.
// With few tiles per head the causal tile lengths do not pair up across the
// XCD's 32 CUs, and head by head would leave the longest tiles of the last
// heads to a few CUs at the end (1.5x the balanced time for B=4, H=16,
// N=2048, in-order dispatch to 32 CUs).
//
// Fixed-length calls with that order and more items than the device has
// compute units launch one work-group per compute unit instead, each
// looping over its XCD's items (item_of, attn_kernels.hpp).  The hardware
// starts a new work-group on a compute unit several microseconds after the
// last one ends, and a causal call's items differ in length, so with one
// work-group per item these gaps took 2-6% of each compute unit's time.
int plan(attn::FwdParams& prm, int rows_per_block, int causal, int* grid_out) {
  const int64_t tiles = ((int64_t)prm.maxlen + rows_per_block - 1) / rows_per_block;
  int64_t grid = (int64_t)prm.B * prm.H * tiles;
  if (grid > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  prm.n_qtiles = (int)tiles;
  prm.remap = (grid % 8 == 0) ? 1 : 0;
  if (prm.remap && causal && !prm.cu && tiles < 32 && ((int64_t)prm.B * prm.H) % 8 == 0) prm.remap = 2;
  prm.items = (int)grid;
  prm.persist = 0;
  if (prm.remap && !prm.cu) {
    const int cus = device_compute_units();
    if (cus >= 8 && cus % 8 == 0 && grid > cus) {
      prm.persist = 1;
      grid = cus;
    }
  }
  *grid_out = (int)grid;
  return ATTN_OK;
}

void set_scale(attn::FwdParams& prm, float scale, unsigned neg_mask) {
  // kernels mask scores with -inf before the fma(s, c, -m): c must be > 0.
  // For |scale| this small every s*c rounds to 0 either way.
  prm.c = fmaxf(fabsf(scale) * 1.4426950408889634f, 1e-30f);
  prm.qsign = scale < 0.f ? neg_mask : 0u;
}

void set_common(attn::FwdParams& prm, const void* q, const void* k, const void* v, void* o,
                float* lse, int B, int H, int Hkv) {
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.B = B;
  prm.H = H;
  prm.Hkv = Hkv;
  prm.group = H / Hkv;
}

int run_bf16(attn::FwdParams& prm, int d, int causal, float scale, hipStream_t stream) {
  set_scale(prm, scale, 0x80008000u);
  int grid = 0;
  const int st = plan(prm, attn::bf16_rows_per_block(d), causal, &grid);
  if (st != ATTN_OK) return st;
  return attn::launch_bf16(prm, d, causal, grid, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int run_fp8(attn::FwdParams& prm, int d, int causal, float scale, hipStream_t stream,
            bool two_pass = false) {
  set_scale(prm, scale, 0x80808080u);
  int grid = 0;
  const int st = plan(prm, attn::fp8_rows_per_block(d), causal, &grid);
  if (st != ATTN_OK) return st;
  return attn::launch_fp8(prm, d, causal, grid, two_pass, stream) == hipSuccess ? ATTN_OK
                                                                                : ATTN_ERR_HIP;
}

// Fixed-length call with Hkv K/V heads.
int fixed_params(attn::FwdParams& prm, const void* q, const void* k, const void* v, void* o,
                 float* lse, int B, int H, int Hkv, int N, int d, int causal, float scale) {
  int64_t tokens = 0;
  int st = validate_fixed(B, N, &tokens);
  if (st != ATTN_OK) return st;
  st = validate(q, k, v, o, lse, tokens, H, Hkv, d, causal, scale);
  if (st != ATTN_OK) return st;
  set_common(prm, q, k, v, o, lse, B, H, Hkv);
  prm.N = N;
  prm.maxlen = N;
  return ATTN_OK;
}

// Variable-length call.  Returns ATTN_OK with *empty = true when there is
// nothing to compute (total == 0).
int varlen_params(attn::FwdParams& prm, const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens, int B, int total, int max_seqlen, int H,
                  int Hkv, int d, int causal, float scale, bool* empty) {
  *empty = false;
  if (B <= 0 || total < 0 || max_seqlen <= 0 || !cu_seqlens) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)cu_seqlens & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  if (total == 0) {
    // still check the scalar arguments
    if (H <= 0 || Hkv <= 0 || H % Hkv != 0 || (causal != 0 && causal != 1) || !isfinite(scale))
      return ATTN_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    *empty = true;
    return ATTN_OK;
  }
  if (max_seqlen > total) return ATTN_ERR_INVALID_ARG;
  const int st = validate(q, k, v, o, lse, total, H, Hkv, d, causal, scale);
  if (st != ATTN_OK) return st;
  set_common(prm, q, k, v, o, lse, B, H, Hkv);
  prm.cu = cu_seqlens;
  prm.total = total;
  prm.maxlen = max_seqlen;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, int causal, float scale, hipStream_t stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream);
}

extern "C" int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, int causal, float scale,
                            hipStream_t stream) {
  attn::FwdParams prm = {};
  const int st = fixed_params(prm, q, k, v, o, lse, B, H, H_kv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  return run_bf16(prm, d, causal, scale, stream);
}

extern "C" int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int* cu_seqlens, int B, int total, int max_seqlen, int H,
                               int H_kv, int d, int causal, float scale, hipStream_t stream) {
  attn::FwdParams prm = {};
  bool empty = false;
  const int st = varlen_params(prm, q, k, v, o, lse, cu_seqlens, B, total, max_seqlen, H, H_kv, d,
                               causal, scale, &empty);
  if (st != ATTN_OK || empty) return st;
  return run_bf16(prm, d, causal, scale, stream);
}

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                            const float* descale_q, const float* descale_k,
                            const float* descale_v, int B, int H, int N, int d, int causal,
                            float scale, hipStream_t stream) {
  return attn_fwd_fp8_gqa(q, k, v, o, lse, descale_q, descale_k, descale_v, B, H, H, N, d, causal,
                          scale, stream);
}

extern "C" int attn_fwd_fp8_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                                const float* descale_q, const float* descale_k,
                                const float* descale_v, int B, int H, int H_kv, int N, int d,
                                int causal, float scale, hipStream_t stream) {
  attn::FwdParams prm = {};
  int st = fixed_params(prm, q, k, v, o, lse, B, H, H_kv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  st = validate_descales(descale_q, descale_k, descale_v);
  if (st != ATTN_OK) return st;
  prm.dq = descale_q;
  prm.dk = descale_k;
  prm.dv = descale_v;
  return run_fp8(prm, d, causal, scale, stream);
}

extern "C" int attn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const float* descale_q, const float* descale_k,
                                   const float* descale_v, const int* cu_seqlens, int B,
                                   int total, int max_seqlen, int H, int H_kv, int d, int causal,
                                   float scale, hipStream_t stream) {
  attn::FwdParams prm = {};
  bool empty = false;
  int st = varlen_params(prm, q, k, v, o, lse, cu_seqlens, B, total, max_seqlen, H, H_kv, d,
                         causal, scale, &empty);
  if (st != ATTN_OK) return st;
  st = validate_descales(descale_q, descale_k, descale_v);
  if (st != ATTN_OK || empty) return st;
  prm.dq = descale_q;
  prm.dk = descale_k;
  prm.dv = descale_v;
  return run_fp8(prm, d, causal, scale, stream);
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta, int B, int H, int N, int d, int causal, float scale,
                        hipStream_t stream) {
  int64_t tokens = 0;
  int st = validate_fixed(B, N, &tokens);
  if (st != ATTN_OK) return st;
  st = validate(q, k, v, o, lse, tokens, H, H, d, causal, scale);
  if (st != ATTN_OK) return st;
  if (!dout || !dq || !dk || !dv || !delta) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)delta & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  const int64_t grid = (int64_t)B * H * ((N + 127) / 128);   // the larger of the kernels' grids
  if (grid > INT32_MAX || (tokens * H + 15) / 16 > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  const hipError_t e = attn::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N,
                                             d, causal, scale, device_compute_units(), stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8_2pass(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const float* descale_q, const float* descale_k,
                                  const float* descale_v, int B, int H, int H_kv, int N, int d,
                                  int causal, float scale, hipStream_t stream) {
  attn::FwdParams prm = {};
  int st = fixed_params(prm, q, k, v, o, lse, B, H, H_kv, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  st = validate_descales(descale_q, descale_k, descale_v);
  if (st != ATTN_OK) return st;
  prm.dq = descale_q;
  prm.dk = descale_k;
  prm.dv = descale_v;
  return run_fp8(prm, d, causal, scale, stream, true);
}

extern "C" int attn_fp8_quantize(const void* x, void* codes, float* descale,
                                 const unsigned* sign_bits, int B, int N, int H, int d,
                                 hipStream_t stream) {
  if (!x || !codes || !descale) return ATTN_ERR_INVALID_ARG;
  int64_t tokens = 0;
  int st = validate_fixed(B, N, &tokens);
  if (st != ATTN_OK) return st;
  if (H <= 0) return ATTN_ERR_INVALID_ARG;
  if (tokens > (INT64_MAX / 4) / H || tokens * H > (INT64_MAX / 4) / 128) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(codes)) return ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)descale & 3u) || ((uintptr_t)sign_bits & 3u)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)B * H * ((N + 127) / 128) > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  const hipError_t e = attn::launch_quant(x, codes, descale, sign_bits, B, N, H, d, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

extern "C" const char* attn_version(void) { return "exact_attention_tile_amd 0.1 (gfx950)"; }
