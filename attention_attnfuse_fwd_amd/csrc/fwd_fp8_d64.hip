// fp8 prefill kernel variants for head dim 64.
#include "fwd_fp8_launch.h"

namespace attnfuse {
template hipError_t launch_fwd_fp8<64>(const AttnParams&, bool, bool, unsigned, hipStream_t);
}  // namespace attnfuse
