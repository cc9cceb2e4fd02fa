// Attention backward, head dim 128 (kernels in bwd_kernels.h), and the
// dispatch over the head dims.
#include "bwd_kernels.h"

namespace attnfuse {

hipError_t launch_bwd_d64(const AttnParams& p, const BwdParams& g, hipStream_t stream);

hipError_t launch_bwd(const AttnParams& p, const BwdParams& g, int D, hipStream_t stream) {
  if (D == 64) return launch_bwd_d64(p, g, stream);
  if (D == 128) return launch_bwd_d<128>(p, g, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnfuse
