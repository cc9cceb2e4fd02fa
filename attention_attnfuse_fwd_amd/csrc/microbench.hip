// Machine-peak probes for the rooflines of the attention kernels: a
// matrix-core loop (the bf16 MFMA shape the prefill kernels use, back to
// back with independent accumulators) and a streaming read of a device
// buffer (the access pattern bound of the decode).  Both time themselves with
// the shader-clock counter (s_memtime) against the constant 100 MHz counter
// (s_memrealtime) in the first wave of the first workgroup, so the caller
// also learns the shader clock while the probe ran.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <chrono>

#include "../../include/attnfuse.h"
#include "../../include/attnfuse_microbench.h"
#include "common.h"

namespace attnfuse {
namespace {

// Each wave keeps four independent 32x32 accumulators so that consecutive
// MFMAs never wait on each other's results.
__global__ __launch_bounds__(256) void mb_mfma_bf16_kernel(int iters, float* sink,
                                                           unsigned long long* stamps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((lane + i) & 7);
    b[i] = (__bf16)(float)((lane * 3 + i) & 7);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool stamp = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (stamp) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (stamp) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    stamps[0] = t1 - t0;
    stamps[1] = r1 - r0;
  }
}

// Same loop with operands read once from `ops` (four bf16x8 per lane: a0,
// b0, a1, b1) and alternated between consecutive MFMAs, so the matrix core's
// inputs change every instruction as they do in a real product (the loop
// above feeds it the same small integers throughout).
__global__ __launch_bounds__(256) void mb_mfma_bf16_ops_kernel(int iters, const uint4* __restrict__ ops,
                                                               float* sink, unsigned long long* stamps) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const bf16x8 a0 = __builtin_bit_cast(bf16x8, ops[4 * t + 0]);
  const bf16x8 b0 = __builtin_bit_cast(bf16x8, ops[4 * t + 1]);
  const bf16x8 a1 = __builtin_bit_cast(bf16x8, ops[4 * t + 2]);
  const bf16x8 b1 = __builtin_bit_cast(bf16x8, ops[4 * t + 3]);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool stamp = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (stamp) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a0, b0, c0);
    c1 = mfma32(a1, b1, c1);
    c2 = mfma32(a0, b1, c2);
    c3 = mfma32(a1, b0, c3);
  }
  float s = 0.f;
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[t] = s;
  if (stamp) {
    stamps[0] = __builtin_amdgcn_s_memtime() - t0;
    stamps[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

// Grid-stride read of n16 16-byte words, four streaming (non-temporal) loads
// in flight per thread, the load the decode uses for its KV cache; the XOR of
// everything read goes to sink so that no load can be dropped.
__global__ __launch_bounds__(256) void mb_read_kernel(const uint4* __restrict__ src,
                                                      unsigned long long n16, float* sink,
                                                      unsigned long long* stamps) {
  const bool stamp = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (stamp) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long stride = (unsigned long long)gridDim.x * 256;
  unsigned long long i = (unsigned long long)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = ld16_stream(src + i);
    const uint4 v1 = ld16_stream(src + i + stride);
    const uint4 v2 = ld16_stream(src + i + 2 * stride);
    const uint4 v3 = ld16_stream(src + i + 3 * stride);
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld16_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[blockIdx.x * 256 + threadIdx.x] = __uint_as_float(acc);
  if (stamp) {
    stamps[0] = __builtin_amdgcn_s_memtime() - t0;
    stamps[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__global__ void mb_empty_kernel(AttnParams p) {
  if (p.B < 0 && threadIdx.x == 0) p.lse[0] = 0.f;  // never taken: keeps the argument live
}

}  // namespace
}  // namespace attnfuse

extern "C" {

int attnfuse_mb_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, unsigned long long* stamps,
                          void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || !sink || !stamps)
    return ATTNFUSE_MB_ERR_INVALID;
  hipLaunchKernelGGL(attnfuse::mb_mfma_bf16_kernel, dim3(workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, sink, stamps);
  return hipGetLastError() == hipSuccess ? ATTNFUSE_MB_OK : ATTNFUSE_MB_ERR_HIP;
}

int attnfuse_mb_mfma_bf16_ops(int32_t workgroups, int32_t iters, const void* operands, float* sink,
                              unsigned long long* stamps, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || !operands ||
      !attnfuse::aligned16(operands) || !sink || !stamps)
    return ATTNFUSE_MB_ERR_INVALID;
  hipLaunchKernelGGL(attnfuse::mb_mfma_bf16_ops_kernel, dim3(workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, reinterpret_cast<const uint4*>(operands),
                     sink, stamps);
  return hipGetLastError() == hipSuccess ? ATTNFUSE_MB_OK : ATTNFUSE_MB_ERR_HIP;
}

int attnfuse_mb_hbm_read(const void* src, size_t bytes, int32_t workgroups, float* sink,
                         unsigned long long* stamps, void* stream) {
  if (!src || !sink || !stamps || bytes < 16 || bytes % 16 || !attnfuse::aligned16(src) ||
      workgroups < 1 || workgroups > (1 << 20))
    return ATTNFUSE_MB_ERR_INVALID;
  hipLaunchKernelGGL(attnfuse::mb_read_kernel, dim3(workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(src),
                     (unsigned long long)(bytes / 16), sink, stamps);
  return hipGetLastError() == hipSuccess ? ATTNFUSE_MB_OK : ATTNFUSE_MB_ERR_HIP;
}

int attnfuse_mb_host_cost(int32_t which, const void* q, const void* k, const void* v, void* out,
                          const attnfuse_variant_desc* desc, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, int32_t calls, double* ns_per_call, void* stream) {
  if (which < 0 || which > 3 || calls < 1 || calls > (1 << 20) || !ns_per_call)
    return ATTNFUSE_MB_ERR_INVALID;
  if (which != 2 && !desc) return ATTNFUSE_MB_ERR_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  attnfuse::AttnParams p{};
  p.B = 1;
  attnfuse_variant_desc dz{};
  if (which == 3) {  // no queries: attnfuse_fwd validates everything, then returns
    dz = *desc;
    dz.Nq = 0;
  }
  const auto t0 = std::chrono::steady_clock::now();
  int st = ATTNFUSE_OK;
  for (int i = 0; i < calls && st == ATTNFUSE_OK; ++i) {
    if (which == 0) {
      st = attnfuse_fwd(q, k, v, out, desc, stream);
    } else if (which == 1) {
      st = attnfuse_decode(q, k, v, out, desc, num_splits, workspace, workspace_bytes, stream);
    } else if (which == 3) {
      st = attnfuse_fwd(q, k, v, out, &dz, stream);
    } else {
      hipLaunchKernelGGL(attnfuse::mb_empty_kernel, dim3(1), dim3(64), 0, s, p);
      st = hipGetLastError() == hipSuccess ? ATTNFUSE_OK : ATTNFUSE_ERR_HIP;
    }
  }
  const auto t1 = std::chrono::steady_clock::now();
  *ns_per_call = std::chrono::duration<double, std::nano>(t1 - t0).count() / calls;
  return st == ATTNFUSE_OK ? ATTNFUSE_MB_OK : st;
}

}  // extern "C"
