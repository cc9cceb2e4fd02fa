// bf16 prefill kernel variants for head dim 64, 8 waves per workgroup.
#include "fwd_bf16_launch.h"

namespace attnfuse {
template hipError_t launch_fwd_bf16<64, 8>(const AttnParams&, bool, bool, bool, unsigned,
                                             hipStream_t);
}  // namespace attnfuse
