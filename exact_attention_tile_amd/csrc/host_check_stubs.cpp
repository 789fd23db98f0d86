// Stand-ins for the kernel launchers, linked only into the host-check build
// of the C ABI (libattn_hostcheck.so: attn_api.cpp compiled with the host
// address and undefined-behaviour sanitizers, no kernels).  That build runs
// the argument-validation tests on the CPU; those calls are all rejected
// before a launch, so every stand-in reports a HIP error if reached.
#include <hip/hip_runtime.h>

#include "attn_kernels.hpp"

namespace attn {
int bf16_rows_per_block(int) { return 256; }
int fp8_rows_per_block(int) { return 256; }
hipError_t launch_bf16(const FwdParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fp8(const FwdParams&, int, int, int, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const float*,
                           const void*, void*, void*, void*, float*, int, int, int, int, int, float,
                           int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quant(const void*, void*, float*, const unsigned*, int, int, int, int,
                        hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace attn
