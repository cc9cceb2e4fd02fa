// Explicit instantiation helper for the bf16 prefill kernel variants.
#pragma once

#include "fwd_bf16_kernel.h"
#include "launch.h"

namespace attnfuse {

template <int D, int NW>
hipError_t launch_fwd_bf16(const AttnParams& p, bool rope, bool scoremod, bool sparse,
                           unsigned grid, hipStream_t stream) {
  // An additive bias selects the instances that read it; ALiBi alone does not.
  const bool bias = scoremod && p.bias != nullptr;
#define ATTNFUSE_CASE(R, S, SP, B)                                                            \
  if (rope == R && scoremod == S && sparse == SP && bias == B) {                              \
    if constexpr (fwd_bf16_supported(D, NW, R, S, SP)) {                                      \
      hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, R, S, SP, B>), dim3(grid), dim3(NW * 64), 0, \
                         stream, p);                                                          \
      return hipGetLastError();                                                               \
    }                                                                                         \
    return hipErrorInvalidValue;                                                              \
  }
  ATTNFUSE_CASE(false, false, false, false)
  ATTNFUSE_CASE(false, false, true, false)
  ATTNFUSE_CASE(false, true, false, false)
  ATTNFUSE_CASE(false, true, true, false)
  ATTNFUSE_CASE(false, true, false, true)
  ATTNFUSE_CASE(false, true, true, true)
  ATTNFUSE_CASE(true, false, false, false)
  ATTNFUSE_CASE(true, false, true, false)
  ATTNFUSE_CASE(true, true, false, false)
  ATTNFUSE_CASE(true, true, true, false)
  ATTNFUSE_CASE(true, true, false, true)
  ATTNFUSE_CASE(true, true, true, true)
#undef ATTNFUSE_CASE
  return hipErrorInvalidValue;
}

}  // namespace attnfuse
