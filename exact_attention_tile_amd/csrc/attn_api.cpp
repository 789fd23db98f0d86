// C ABI of the tiled exact attention forward (see include/attn.h).
//
// Every argument is validated on the host before any HIP call; on error
// nothing is launched.  On success exactly one kernel is enqueued on the
// caller's stream; the library allocates, frees and synchronises nothing.
#include "attn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_kernels.hpp"

namespace attn {
int bf16_rows_per_block(int d);
hipError_t launch_bf16(const FwdParams& prm, int d, int causal, int grid, hipStream_t stream);
int fp8_rows_per_block(int d);
hipError_t launch_fp8(const FwdParams& prm, int d, int causal, int grid, hipStream_t stream);
}  // namespace attn

namespace {

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Shared validation.  Returns ATTN_OK or the first error found.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
             int H, int N, int d, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  // element count B*N*H*d must fit in int64 (and the per-head row offsets
  // the kernels form from it)
  const int64_t lim = INT64_MAX / 4;
  int64_t n = B;
  if (n > lim / N) return ATTN_ERR_INVALID_ARG;
  n *= N;
  if (n > lim / H) return ATTN_ERR_INVALID_ARG;
  n *= H;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (n > lim / d) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)lse & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Work-group count and block order for one call.  The grid has one
// work-group per (batch, head, query tile); it must fit the 32-bit grid.
int plan(attn::FwdParams& prm, int rows_per_block, int* grid_out) {
  const int64_t tiles = ((int64_t)prm.N + rows_per_block - 1) / rows_per_block;
  const int64_t grid = (int64_t)prm.B * prm.H * tiles;
  if (grid > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  prm.n_qtiles = (int)tiles;
  prm.remap = (grid % 8 == 0) ? 1 : 0;
  *grid_out = (int)grid;
  return ATTN_OK;
}

void set_scale(attn::FwdParams& prm, float scale, unsigned neg_mask) {
  // kernels mask scores with -inf before the fma(s, c, -m): c must be > 0.
  // For |scale| this small every s*c rounds to 0 either way.
  prm.c = fmaxf(fabsf(scale) * 1.4426950408889634f, 1e-30f);
  prm.qsign = scale < 0.f ? neg_mask : 0u;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int N, int d, int causal, float scale, hipStream_t stream) {
  int st = validate(q, k, v, o, lse, B, H, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  attn::FwdParams prm = {};
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.B = B;
  prm.H = H;
  prm.N = N;
  set_scale(prm, scale, 0x80008000u);
  int grid = 0;
  st = plan(prm, attn::bf16_rows_per_block(d), &grid);
  if (st != ATTN_OK) return st;
  hipError_t e = attn::launch_bf16(prm, d, causal, grid, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                            const float* descale_q, const float* descale_k,
                            const float* descale_v, int B, int H, int N, int d, int causal,
                            float scale, hipStream_t stream) {
  int st = validate(q, k, v, o, lse, B, H, N, d, causal, scale);
  if (st != ATTN_OK) return st;
  if (!descale_q || !descale_k || !descale_v) return ATTN_ERR_INVALID_ARG;
  if (((uintptr_t)descale_q & 3u) || ((uintptr_t)descale_k & 3u) || ((uintptr_t)descale_v & 3u))
    return ATTN_ERR_UNSUPPORTED;
  attn::FwdParams prm = {};
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.dq = descale_q;
  prm.dk = descale_k;
  prm.dv = descale_v;
  prm.B = B;
  prm.H = H;
  prm.N = N;
  set_scale(prm, scale, 0x80808080u);
  int grid = 0;
  st = plan(prm, attn::fp8_rows_per_block(d), &grid);
  if (st != ATTN_OK) return st;
  hipError_t e = attn::launch_fp8(prm, d, causal, grid, stream);
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
