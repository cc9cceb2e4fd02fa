// RoPE support kernels ("4.1 Fused RoPE": the rotation reads a precomputed
// cos / sin table; NeoX half-split pairs (r, r + D/2)).
//
//  * rope_table: cos / sin of p * theta^(-2r/D), angle formed in fp64 (an fp32
//    angle at p ~ 3e4 would carry ~2e-3 rad of error), rounded to fp32 (fp32
//    prefill, pre-rotation pass), packed as fp16 (cos, sin) pairs (the bf16
//    prefill's Q and K rotations and the decode's K rotation, fp32 arithmetic
//    with the fp16 factors) and, on request, as bf16 pairs (no kernel of this
//    library reads those).
//  * prerotate: the separate rotation pass that the fused kernel replaces
//    ("1 Introduction": the pre-rotation workaround costs two extra memory
//    round trips; "5.3 The Rotation Calculus" weighs the two).  Rotates a
//    Q- or K-shaped tensor into a new buffer with the same strides.
#include "common.h"
#include "launch.h"

namespace attnfuse {

__global__ void rope_table_kernel(double theta, int D, long long len, float* cos_out,
                                  float* sin_out, uint32_t* cs_out, uint32_t* csb_out) {
  const int h2 = D / 2;
  const long long n = len * h2;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long pos = idx / h2;
    const int r = (int)(idx % h2);
    const double w = pow(theta, -2.0 * r / D);
    const double a = (double)pos * w;
    const double c = cos(a), s = sin(a);
    if (cos_out) cos_out[idx] = (float)c;
    if (sin_out) sin_out[idx] = (float)s;
    if (cs_out) {
      const f16x2 h = {(_Float16)c, (_Float16)s};
      cs_out[idx] = __builtin_bit_cast(uint32_t, h);
    }
    if (csb_out) csb_out[idx] = pack_bf16x2((float)c, (float)s);
  }
}

template <bool BF16>
__global__ void prerotate_kernel(const void* x, void* y, int D, int B, int H, int N, long long sb,
                                 long long sh, long long sn, int pos0, const float* rcos,
                                 const float* rsin) {
  const int h2 = D / 2;
  const long long n = (long long)B * H * N * h2;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int r = (int)(idx % h2);
    long long rest = idx / h2;
    const int row = (int)(rest % N);
    rest /= N;
    const int hh = (int)(rest % H);
    const int bb = (int)(rest / H);
    const long long off = bb * sb + hh * sh + row * sn + r;
    const long long t = (long long)(pos0 + row) * h2 + r;
    const float c = rcos[t], s = rsin[t];
    if (BF16) {
      const __bf16* xs = reinterpret_cast<const __bf16*>(x);
      __bf16* ys = reinterpret_cast<__bf16*>(y);
      const float lo = (float)xs[off], hi = (float)xs[off + h2];
      ys[off] = (__bf16)(lo * c - hi * s);
      ys[off + h2] = (__bf16)(hi * c + lo * s);
    } else {
      const float* xs = reinterpret_cast<const float*>(x);
      float* ys = reinterpret_cast<float*>(y);
      const float lo = xs[off], hi = xs[off + h2];
      ys[off] = lo * c - hi * s;
      ys[off + h2] = hi * c + lo * s;
    }
  }
}

// Vectorised bf16 pre-rotation for contiguous rows (16-byte chunks, fp32
// math, one bf16 rounding per element).
__global__ void prerotate_bf16x8_kernel(const __bf16* x, __bf16* y, int D, int B, int H, int N,
                                        long long sb, long long sh, long long sn, int pos0,
                                        const float* rcos, const float* rsin) {
  const int chunks = D / 16;  // chunk pairs per row
  const long long n = (long long)B * H * N * chunks;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(idx % chunks);
    long long rest = idx / chunks;
    const int row = (int)(rest % N);
    rest /= N;
    const int hh = (int)(rest % H);
    const int bb = (int)(rest / H);
    const long long off = bb * sb + hh * sh + row * sn + 8 * c;
    uint4 lo = ld16(x + off), hi = ld16(x + off + D / 2);
    const long long t = (long long)(pos0 + row) * (D / 2) + 8 * c;
    rope_rotate_bf16x8(lo, hi, ld_f8(rcos + t), ld_f8(rsin + t));
    st16(y + off, lo);
    st16(y + off + D / 2, hi);
  }
}

hipError_t launch_rope_table(double theta, int D, long long len, float* cos_out, float* sin_out,
                             uint32_t* cs_out, uint32_t* csb_out, hipStream_t stream) {
  const long long n = len * (D / 2);
  const long long blocks = min((n + 255) / 256, 65536LL);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, theta, D,
                     len, cos_out, sin_out, cs_out, csb_out);
  return hipGetLastError();
}

hipError_t launch_prerotate(const void* x, void* x_rot, bool bf16, bool vec_ok, int D, int B,
                            int H, int N, long long sb, long long sh, long long sn, int pos0,
                            const float* rcos, const float* rsin, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  if (bf16 && vec_ok && D % 16 == 0 && sb % 8 == 0 && sh % 8 == 0 && sn % 8 == 0) {
    const long long n = rows * (D / 16);
    const long long blocks = min((n + 255) / 256, 1LL << 20);
    hipLaunchKernelGGL(prerotate_bf16x8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const __bf16*>(x), reinterpret_cast<__bf16*>(x_rot), D, B,
                       H, N, sb, sh, sn, pos0, rcos, rsin);
    return hipGetLastError();
  }
  const long long n = rows * (D / 2);
  const long long blocks = min((n + 255) / 256, 1LL << 20);
  if (bf16)
    hipLaunchKernelGGL(prerotate_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       x_rot, D, B, H, N, sb, sh, sn, pos0, rcos, rsin);
  else
    hipLaunchKernelGGL(prerotate_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       x_rot, D, B, H, N, sb, sh, sn, pos0, rcos, rsin);
  return hipGetLastError();
}

}  // namespace attnfuse
