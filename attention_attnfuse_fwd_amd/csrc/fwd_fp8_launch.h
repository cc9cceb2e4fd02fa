// Launcher of the fp8 prefill instances (Q, K, V in OCP E4M3; eight waves).
#pragma once

#include "fwd_bf16_kernel.h"
#include "launch.h"

namespace attnfuse {

template <int D>
hipError_t launch_fwd_fp8(const AttnParams& p, bool scoremod, bool sparse, unsigned grid,
                          hipStream_t stream) {
#define ATTNFUSE_FP8_CASE(S, SP)                                                                  \
  if (scoremod == S && sparse == SP) {                                                            \
    hipLaunchKernelGGL((fwd_bf16_kernel<D, 8, false, S, SP, false, true>), dim3(grid), dim3(512), \
                       0, stream, p);                                                             \
    return hipGetLastError();                                                                     \
  }
  ATTNFUSE_FP8_CASE(false, false)
  ATTNFUSE_FP8_CASE(false, true)
  ATTNFUSE_FP8_CASE(true, false)
  ATTNFUSE_FP8_CASE(true, true)
#undef ATTNFUSE_FP8_CASE
  return hipErrorInvalidValue;
}

}  // namespace attnfuse
