// Split-KV single-query decode ("4.2 Flash Decoding"): phase 1 computes one
// online-softmax partial (m, l, acc) per key chunk, phase 2 merges the
// partials by log-sum-exp.
//
// Phase 1: one workgroup (4 waves) per (b, kv-head, group of up to 32 q-heads,
// chunk).  The q-heads of a kv-head's group are the 32 MFMA columns (GQA:
// K and V are read once for the whole group; unused columns are padding).
// The chunk is streamed in 128-key tiles through a double-buffered LDS ring
// (K rotated once per workgroup on register fragments); wave w takes keys
// 32w .. 32w+31 of every tile with its own running (m, l, O^T), and the four
// waves are merged in LDS before the partial is written.  Workgroups are
// ordered so that the kv-heads of one chunk run on the same XCD, sharing the
// chunk's RoPE table rows in that XCD's L2.
//
// Partial layout in the workspace (fp32): for (b, h, chunk), D + 2 floats:
// acc[0..D-1] (un-normalised), then m (exp2 domain, scaled), then l.
#include "common.h"
#include "launch.h"
#include "tile_stage.h"

namespace attnfuse {

namespace {
constexpr int kDecTile = 128;  // keys per LDS tile
constexpr int kDecNT = 256;    // 4 waves
}

template <int D, bool ROPE>
__global__ void __launch_bounds__(kDecNT) decode_split_kernel(const AttnParams p) {
  using S = TileStage<D, kDecTile, kDecNT, ROPE>;
  constexpr int KBUF = S::KBUF;
  constexpr int VSTR = S::VSTR;
  constexpr int BUF = KBUF + D * VSTR;
  constexpr int NKK = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;

  // workgroup -> (chunk, unit); chunk s of every unit lands on XCD s % 8.
  const int U = p.B * p.Hkv * p.n_hgrp;
  const int slot = blockIdx.x / 8;
  const int split = (blockIdx.x % 8) + 8 * (slot / U);
  if (split >= p.splits) return;  // whole workgroup leaves together, before any barrier
  const int u = slot % U;
  const int hgrp = u % p.n_hgrp;
  const int kvh = (u / p.n_hgrp) % p.Hkv;
  const int b = u / (p.n_hgrp * p.Hkv);
  const int g = hgrp * 32 + lq;          // head within the kv group for this column
  const bool col_valid = g < p.G;
  const int h = kvh * p.G + min(g, p.G - 1);

  const int c0 = split * p.chunk;
  const int c1 = min(p.Nk, c0 + p.chunk);
  const int n_tiles = c1 > c0 ? (c1 - c0 + kDecTile - 1) / kDecTile : 0;

  const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ksb + kvh * p.ksh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;

  // Query fragments (one query position; one q-head per column).
  bf16x8 qf[NKK];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + b * p.qsb + h * p.qsh;
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      const int d0 = 16 * kk + 8 * lh;
      uint4 lo = ld16(qrow + d0);
      uint4 hi = ld16(qrow + d0 + D / 2);
      if (ROPE) {
        const long long row = (long long)p.q_pos0 * (D / 2) + d0;
        rope_rotate_bf16x8(lo, hi, ld_f8(p.rcos + row), ld_f8(p.rsin + row));
      }
      qf[kk] = __builtin_bit_cast(bf16x8, lo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, hi);
    }
  }

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float slope2 = p.alibi ? p.alibi[h] * kLog2e : 0.f;
  const int dpos = p.k_pos0 - p.q_pos0;

  S stage;
  if (n_tiles > 0) {
    stage.load(p, kb, vb, c0, c1, tid);
    stage.store(smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = c0 + t * kDecTile;
    const bool more = t + 1 < n_tiles;
    if (more) stage.load(p, kb, vb, k0 + kDecTile, c1, tid);

    const int kw = k0 + 32 * wave;  // this wave's first key
    bool skip = kw >= c1;
    bool need_mask = kw + 32 > c1;
    if (p.has_band) {  // query row index is 0
      skip |= (kw + 31 < p.band_lo) || (kw > p.band_hi);
      need_mask |= (kw < p.band_lo) || (kw + 31 > p.band_hi);
    }
    if (!skip) {
      const __bf16* ks = smem + (t & 1) * BUF;
      const __bf16* vs = ks + KBUF;
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (32 * wave + lq) * S::KSTR + 16 * kk + 8 * lh);
        s = mfma32(a, qf[kk], s);
      }
      const int jb = kw + 4 * lh;  // key index at register offset 0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jb + 8 * (r / 4) + (r % 4);
        float x = s[r] * p.scale_log2;
        if (p.alibi) x = __builtin_fmaf(slope2, (float)(j + dpos), x);
        if (need_mask) {
          bool ok = j < c1;
          if (p.has_band) ok = ok && j >= p.band_lo && j <= p.band_hi;
          x = ok ? x : -INFINITY;
        }
        s[r] = x;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, partner32(mx));
      const float m_new = fmaxf(m_run, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f)) {
        const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(s[r] - m_use);
        lsum += s[r];
      }
      l_run += lsum;
      bf16x8 pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 w;
        w.x = pack_bf16x2(s[8 * c + 0], s[8 * c + 1]);
        w.y = pack_bf16x2(s[8 * c + 2], s[8 * c + 3]);
        w.z = pack_bf16x2(s[8 * c + 4], s[8 * c + 5]);
        w.w = pack_bf16x2(s[8 * c + 6], s[8 * c + 7]);
        pf[c] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (32 * dt + lq) * VSTR + 32 * wave + 16 * c + 8 * lh);
          o[dt] = mfma32(a, pf[c], o[dt]);
        }
    }
    if (more) stage.store(smem + ((t + 1) & 1) * BUF, tid);
    __syncthreads();
  }

  // Merge the four waves' partials in LDS (the tile ring is free now).
  float* red = reinterpret_cast<float*>(smem);
  float* mw = red;                 // [4][32]
  float* lw = red + 4 * 32;        // [4][32]
  float* ow = red + 8 * 32;        // [4][D][32]
  const float l_tot = l_run + partner32(l_run);
  if (lh == 0) {
    mw[wave * 32 + lq] = m_run;
    lw[wave * 32 + lq] = l_tot;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * dt + 8 * (r / 4) + 4 * lh + (r % 4);
      ow[(wave * D + d) * 32 + lq] = o[dt][r];
    }
  __syncthreads();
  for (int idx = tid; idx < 32 * D; idx += kDecNT) {
    const int col = idx / D, d = idx % D;
    const int gg = hgrp * 32 + col;
    if (gg >= p.G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mw[w * 32 + col]);
    float acc = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mwv = mw[w * 32 + col];
        const float a = (mwv == -INFINITY) ? 0.f : fast_exp2(mwv - M);
        acc += a * ow[(w * D + d) * 32 + col];
        L += a * lw[w * 32 + col];
      }
    }
    const int hh = kvh * p.G + gg;
    float* dst = p.ws + (((long long)b * p.Hq + hh) * p.splits + split) * (D + 2);
    dst[d] = acc;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = L;
    }
  }
  (void)col_valid;
}

// Phase 2: one workgroup of D threads per (b, q-head); thread d merges column d.
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(const AttnParams p) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* base = p.ws + (long long)bh * p.splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, base[s * (D + 2) + D]);
  float acc = 0.f, L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const float* part = base + s * (D + 2);
      const float ms = part[D];
      if (ms == -INFINITY) continue;
      const float a = fast_exp2(ms - M);
      acc += a * part[d];
      L += a * part[D + 1];
    }
  }
  const int b = bh / p.Hq, h = bh % p.Hq;
  const float val = L > 0.f ? acc / L : 0.f;
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh;
  orow[d] = (__bf16)val;
  if (p.lse && d == 0) p.lse[bh] = L > 0.f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
}

hipError_t launch_decode_split(const AttnParams& p, int D, bool rope, unsigned grid,
                               hipStream_t stream) {
#define ATTNFUSE_DEC(DD, R)                                                                  \
  if (D == DD && rope == R) {                                                                \
    hipLaunchKernelGGL((decode_split_kernel<DD, R>), dim3(grid), dim3(kDecNT), 0, stream, p); \
    return hipGetLastError();                                                                \
  }
  ATTNFUSE_DEC(64, false)
  ATTNFUSE_DEC(64, true)
  ATTNFUSE_DEC(128, false)
  ATTNFUSE_DEC(128, true)
#undef ATTNFUSE_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const AttnParams& p, int D, hipStream_t stream) {
  const unsigned grid = (unsigned)(p.B * p.Hq);
  if (D == 64) {
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(grid), dim3(64), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(grid), dim3(128), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attnfuse
