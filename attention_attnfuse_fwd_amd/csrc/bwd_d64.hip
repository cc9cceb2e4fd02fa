// Attention backward, head dim 64 (kernels in bwd_kernels.h).
#include "bwd_kernels.h"

namespace attnfuse {

hipError_t launch_bwd_d64(const AttnParams& p, const BwdParams& g, hipStream_t stream) {
  return launch_bwd_d<64>(p, g, stream);
}

}  // namespace attnfuse
