// Fused attention forward in fp32 throughout (no bf16 rounding anywhere).
//
// The same exact computation as the bf16 MFMA kernel ("2 Background /
// FlashAttention and online softmax"; RoPE per "4.1 Fused RoPE"), on the
// vector ALU: one workgroup = one wave = 64 query rows of one q-head, one
// query per lane.  32-key tiles of K (rotated once per workgroup in fp32) and
// V are staged in LDS and read as broadcasts; each lane keeps its rotated
// query, its output accumulator and the online-softmax state in registers.
#include "common.h"
#include "launch.h"

namespace attnfuse {

template <int D>
__global__ void __launch_bounds__(64) fwd_fp32_kernel(const AttnParams p) {
  constexpr int TK = 32;
  constexpr int H2 = D / 2;
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];

  const int tid = threadIdx.x;
  const int n_qblk = p.n_qblk;
  const int bh = blockIdx.x % (p.B * p.Hq);
  const int qrank = blockIdx.x / (p.B * p.Hq);
  const int qblk = p.longest_first ? (n_qblk - 1 - qrank) : qrank;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int kvh = h / p.G;
  const int r0 = qblk * 64;
  const int i = r0 + tid;
  const int iq = min(i, p.Nq - 1);
  const int last = min(r0 + 63, p.Nq - 1);

  const float* qrow = reinterpret_cast<const float*>(p.q) + b * p.qsb + h * p.qsh + (long long)iq * p.qsn;
  const float* kb = reinterpret_cast<const float*>(p.k) + b * p.ksb + kvh * p.ksh;
  const float* vb = reinterpret_cast<const float*>(p.v) + b * p.vsb + kvh * p.vsh;

  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = qrow[d];
  if (p.rcos) {
    const float* c = p.rcos + (long long)(p.q_pos0 + iq) * H2;
    const float* s = p.rsin + (long long)(p.q_pos0 + iq) * H2;
#pragma unroll
    for (int r = 0; r < H2; ++r) {
      const float lo = q[r], hi = q[r + H2];
      q[r] = lo * c[r] - hi * s[r];
      q[r + H2] = hi * c[r] + lo * s[r];
    }
  }

  // Key tiles to visit.
  int n_tiles, t_begin = 0, s_begin = 0, tpb = 1;
  if (p.row_ptr) {
    const int* rp = p.row_ptr + (p.bs_head_stride ? (long long)h * p.bs_head_stride : 0);
    const int qbs = r0 / p.bm;
    const long long a = min(max((long long)rp[qbs], 0LL), p.bs_nnz);
    const long long e = min(max((long long)rp[qbs + 1], a), p.bs_nnz);
    s_begin = (int)a;
    tpb = p.bn / TK;
    n_tiles = (int)(e - a) * tpb;
  } else {
    int j_lo = 0, j_hi = p.Nk - 1;
    if (p.has_band) {
      j_lo = max(j_lo, r0 + p.band_lo);
      j_hi = min(j_hi, (int)min((long long)last + p.band_hi, (long long)kBandInf));
    }
    t_begin = j_lo / TK;
    n_tiles = (j_hi >= j_lo) ? (j_hi / TK - t_begin + 1) : 0;
  }

  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float slope2 = p.alibi ? p.alibi[h] * kLog2e : 0.f;
  const int dpos = p.k_pos0 - p.q_pos0;
  const float* brow = p.bias ? p.bias + b * p.bsb + h * p.bsh + (long long)iq * p.bsi : nullptr;

  for (int t = 0; t < n_tiles; ++t) {
    // Sparse columns are clamped into [0, nkb]; column nkb lies past the keys.
    const int nkb = p.row_ptr ? (p.Nk + p.bn - 1) / p.bn : 0;
    const int k0 = p.row_ptr ? min(max(p.col_idx[s_begin + t / tpb], 0), nkb) * p.bn + (t % tpb) * TK
                             : (t_begin + t) * TK;
    // Stage the tile: unit = (key, 4-wide chunk of the low half); rotate in fp32.
    for (int u = tid; u < TK * (H2 / 4); u += 64) {
      const int j = u / (H2 / 4), c = 4 * (u % (H2 / 4));
      const int kj = min(k0 + j, p.Nk - 1);
      const float4 lo = *reinterpret_cast<const float4*>(kb + (long long)kj * p.ksn + c);
      const float4 hi = *reinterpret_cast<const float4*>(kb + (long long)kj * p.ksn + c + H2);
      float l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
      if (p.rcos) {
        const float* cc = p.rcos + (long long)(p.k_pos0 + kj) * H2 + c;
        const float* ss = p.rsin + (long long)(p.k_pos0 + kj) * H2 + c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = l4[e], bb = h4[e];
          l4[e] = a * cc[e] - bb * ss[e];
          h4[e] = bb * cc[e] + a * ss[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ks[j][c + e] = l4[e];
        ks[j][c + H2 + e] = h4[e];
      }
      const float4 v0 = *reinterpret_cast<const float4*>(vb + (long long)kj * p.vsn + c);
      const float4 v1 = *reinterpret_cast<const float4*>(vb + (long long)kj * p.vsn + c + H2);
      vs[j][c + 0] = v0.x; vs[j][c + 1] = v0.y; vs[j][c + 2] = v0.z; vs[j][c + 3] = v0.w;
      vs[j][c + H2 + 0] = v1.x; vs[j][c + H2 + 1] = v1.y;
      vs[j][c + H2 + 2] = v1.z; vs[j][c + H2 + 3] = v1.w;
    }
    __syncthreads();

    float x[TK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], ks[j][d], acc);
      const int kj = k0 + j;
      float xv = acc * p.scale_log2;
      if (p.alibi) xv = __builtin_fmaf(slope2, (float)(kj - i + dpos), xv);
      if (brow) xv = __builtin_fmaf(brow[(long long)min(kj, p.Nk - 1) * p.bsj], kLog2e, xv);
      bool ok = kj < p.Nk;
      if (p.has_band) ok = ok && (kj - i >= p.band_lo) && (kj - i <= p.band_hi);
      x[j] = ok ? xv : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pj = fast_exp2(x[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pj, vs[j][d], o[d]);
    }
    __syncthreads();
  }

  if (i < p.Nq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = reinterpret_cast<float*>(p.o) + b * p.osb + h * p.osh + (long long)i * p.osn;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<float4*>(orow + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
    if (p.lse)
      p.lse[((long long)b * p.Hq + h) * p.Nq + i] =
          l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_fwd_fp32(const AttnParams& p, int D, unsigned grid, hipStream_t stream) {
  if (D == 64) {
    hipLaunchKernelGGL(fwd_fp32_kernel<64>, dim3(grid), dim3(64), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(fwd_fp32_kernel<128>, dim3(grid), dim3(64), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attnfuse
