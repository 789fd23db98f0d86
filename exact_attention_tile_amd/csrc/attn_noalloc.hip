// attn_bwd_noalloc: attn_bwd with its D workspace in a static device array,
// for callers that cannot allocate device memory (see include/attn.h).
//
// The workspace of the backward pass (D_i = sum_c dO_ic O_ic, one fp32 per
// row of B*H*N) lives in `scratch`, a file-scope device array that each GPU
// the library runs on holds from the module's load to the end of the
// process.  In host code `scratch` names a host-side stand-in, not a device
// address: the device address is looked up once per device with
// hipGetSymbolAddress (the device current at that moment) and kept in
// g_scratch[device]; only that pointer is ever passed to a kernel.
//
// Every call on a GPU shares that GPU's array.  The D kernel writes every
// row a call reads before the dQ and dK/dV kernels read it (in stream
// order), so nothing has to start at zero; calls that overlap on one GPU
// (on different streams or threads) race on the array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"

namespace {

static __device__ __align__(256) float scratch[ATTN_BWD_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` runs on, which
// must be the current device.  Looked up on the first call per device.
int scratch_for(hipStream_t stream, float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ATTN_ERR_HIP;
    if (sdev != dev) return ATTN_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return ATTN_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int B, int H, int N, int d, int causal, float scale,
                                hipStream_t stream) {
  // checks that need no HIP call come first; attn_bwd repeats them and
  // checks the rest before it launches anything
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H * N > (int64_t)ATTN_BWD_NOALLOC_MAX_ROWS) return ATTN_ERR_UNSUPPORTED;
  float* ws = nullptr;
  const int st = scratch_for(stream, &ws);
  if (st != ATTN_OK) return st;
  return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, d, causal, scale, stream);
}
