// Internal launchers (C++ linkage, not part of the C ABI).  Each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace attnfuse {

// bf16 MFMA prefill kernel for head dim D with NW waves per workgroup.
template <int D, int NW>
hipError_t launch_fwd_bf16(const AttnParams& p, bool rope, bool scoremod, bool sparse,
                           unsigned grid, hipStream_t stream);

// fp8 prefill (Q, K, V OCP E4M3 codes, bf16 out; eight waves, no RoPE / bias).
template <int D>
hipError_t launch_fwd_fp8(const AttnParams& p, bool scoremod, bool sparse, unsigned grid,
                          hipStream_t stream);

// fp32 prefill kernel (64 query rows per workgroup).
hipError_t launch_fwd_fp32(const AttnParams& p, int D, unsigned grid, hipStream_t stream);

// Split-KV decode phase 1 (partials into p.ws) and phase 2 (LSE merge).
// Head dim 128 with score mods and either RoPE or a block mask does not fit
// two waves per SIMD without spilling; the dispatcher runs it with 4 waves.
constexpr bool fwd_bf16_supported(int D, int NW, bool rope, bool scoremod, bool sparse) {
  return !(D == 128 && NW == 8 && scoremod && (rope || sparse));
}

hipError_t launch_decode_split(const AttnParams& p, int D, bool rope, bool kv8, unsigned grid,
                               hipStream_t stream);
hipError_t launch_decode_combine(const AttnParams& p, int D, hipStream_t stream);

// Backward: delta, dK / dV and dQ passes on one stream.
hipError_t launch_bwd(const AttnParams& p, const BwdParams& g, int D, hipStream_t stream);

// RoPE cos / sin tables and the stand-alone pre-rotation pass.
hipError_t launch_rope_table(double theta, int D, long long len, float* cos_out, float* sin_out,
                             uint32_t* cs_out, uint32_t* csb_out, hipStream_t stream);
hipError_t launch_prerotate(const void* x, void* x_rot, bool bf16, bool vec_ok, int D, int B,
                            int H, int N, long long sb, long long sh, long long sn, int pos0,
                            const float* rcos, const float* rsin, hipStream_t stream);

}  // namespace attnfuse
