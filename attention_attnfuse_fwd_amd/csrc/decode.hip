// Split-KV single-query decode ("4.2 Flash Decoding"): phase 1 computes one
// online-softmax partial (m, l, acc) per key chunk, phase 2 merges the
// partials by log-sum-exp.
//
// Phase 1 is bound by HBM bandwidth, so it is built to keep many bytes in
// flight.  One workgroup (4 waves, two workgroups per CU) per (b, kv-head,
// group of up to 32 q-heads, chunk); the q-heads of the group are the 32 MFMA
// columns, so K and V are read once for the whole group (GQA).  Each wave
// streams its own 32-key subtiles of the chunk (subtiles w, w + 4, ...):
//   global -> registers -> RoPE on the K fragments -> the wave's private LDS
//   region (K row-major, V transposed) -> MFMA,
// with the loads of the next subtile in flight while the current one is
// multiplied, and no workgroup barrier until the four waves' (m, l, O^T) are
// merged in LDS at the end.  Workgroups are ordered so that the kv-heads of
// one chunk run on the same XCD and share the chunk's RoPE table rows in L2.
//
// Partial layout in the workspace (fp32): for (b, h, chunk), D + 2 floats:
// acc[0..D-1] (un-normalised), then m (exp2 domain, scaled), then l.
#include "common.h"
#include "launch.h"
#include "tile_stage.h"

namespace attnfuse {

namespace {
constexpr int kDecNT = 256;  // 4 waves
constexpr int kDecSK = 32;   // keys per wave step
}

template <int D, bool ROPE, bool KV8>
__global__ void __launch_bounds__(kDecNT, 2) decode_split_kernel(const AttnParams p) {
  using KS = KStage<D, kDecSK, 64, ROPE, KV8>;
  using VS = VStage<D, kDecSK, 64, KV8>;
  using T = typename KS::T;
  constexpr int KSTR = KS::KSTR;
  constexpr int VSTR = VS::VSTR;
  constexpr int WBUF = kDecSK * KSTR + D * VSTR;  // one wave's LDS region (elements)
  constexpr int NKK = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[4 * WBUF];

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
  const int g = hgrp * 32 + lq;  // head within the kv group for this column
  const int h = kvh * p.G + min(g, p.G - 1);

  const int c0 = split * p.chunk;
  const int c1 = min(p.Nk, c0 + p.chunk);
  const int n_steps = c1 > c0 ? (c1 - c0 + kDecSK - 1) / kDecSK : 0;

  const T* kb = reinterpret_cast<const T*>(p.k) + b * p.ksb + kvh * p.ksh;
  const T* vb = reinterpret_cast<const T*>(p.v) + b * p.vsb + kvh * p.vsh;
  __bf16* const ks = smem + wave * WBUF;
  __bf16* const vs = ks + kDecSK * KSTR;

  // Wave w takes steps w, w + 4, ... of the chunk, visited from a rotated
  // starting point: chunk bases are 2^k bytes apart, so without the rotation
  // every workgroup would address the same HBM channels at the same moment.
  // (The online softmax does not depend on the key order.)
  const int rot = n_steps > 0 ? (int)((7u * split + 13u * kvh + 5u * b) % (unsigned)n_steps) : 0;
  auto step_k0 = [&](int step) {
    const int s2 = step + rot;
    return c0 + (s2 >= n_steps ? s2 - n_steps : s2) * kDecSK;
  };

  // Start streaming before touching the query.
  KS kst;
  VS vst;
  int st = wave;  // this wave's current step
  if (st < n_steps) {
    kst.load(p, kb, step_k0(st), c1, lane);
    kst.load_tables(p, lane);
    vst.load(p, vb, step_k0(st), c1, lane);
  }

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
        const uint32_t* row = p.rcs + (long long)p.q_pos0 * (D / 2) + d0;
        rope_rotate_bf16x8_h(lo, hi, ld16(row), ld16(row + 4));
      }
      qf[kk] = __builtin_bit_cast(bf16x8, lo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, hi);
    }
  }

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_part[2] = {0.f, 0.f};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float slope2 = p.alibi ? p.alibi[h] * kLog2e : 0.f;
  const int dpos = p.k_pos0 - p.q_pos0;

  for (; st < n_steps; st += 4) {
    const int k0 = step_k0(st);
    // Stage this step into the wave's region, then put the next step in flight.
    kst.store(ks, lane);
    vst.store(vs, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (st + 4 < n_steps) {
      const int kn = step_k0(st + 4);
      kst.load(p, kb, kn, c1, lane);
      kst.load_tables(p, lane);
      vst.load(p, vb, kn, c1, lane);
    }

    bool skip = false, need_mask = k0 + kDecSK > c1;
    if (p.has_band) {  // the query row index is 0
      skip = (k0 + kDecSK - 1 < p.band_lo) || (k0 > p.band_hi);
      need_mask |= (k0 < p.band_lo) || (k0 + kDecSK - 1 > p.band_hi);
    }
    if (!skip) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + lq * KSTR + 16 * kk + 8 * lh);
        s = mfma32(a, qf[kk], s);
      }
      const int jb = k0 + 4 * lh;  // key index at register offset 0
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
      float t8[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) t8[r] = fmaxf(s[r], s[r + 8]);
#pragma unroll
      for (int w = 4; w >= 1; w /= 2)
#pragma unroll
        for (int r = 0; r < w; ++r) t8[r] = fmaxf(t8[r], t8[r + w]);
      const float mx = fmaxf(t8[0], partner32(t8[0]));
      const float m_new = fmaxf(m_run, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f)) {
        const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_part[0] *= alpha;
        l_part[1] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r] - m_use);
      bf16x8 pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = pack_bf16x2(s[8 * c + 2 * q], s[8 * c + 2 * q + 1]);
          l_part[q & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[q]), ones,
                                                          l_part[q & 1], false);
        }
        pf[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (32 * dt + lq) * VSTR + 16 * c + 8 * lh);
          o[dt] = mfma32(a, pf[c], o[dt]);
        }
    }
    // The next store overwrites this wave's region: every lane is done reading it.
    __builtin_amdgcn_wave_barrier();
  }

  // Merge the four waves' partials in LDS.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  float* mw = red;           // [4][32]
  float* lw = red + 4 * 32;  // [4][32]
  float* ow = red + 8 * 32;  // [4][D][32]
  const float l_run = l_part[0] + l_part[1];
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
}

// Phase 2: one workgroup of 256 threads per (b, q-head), one memory round
// trip.  Thread (c, g) owns chunks c, c + NC, ... and the 8-wide d slice g
// (D / 8 slices); it loads all of its (m, l, acc-slice) records at once, then
// the log-sum-exp merge runs from registers: M = max m_c (LDS max over the
// chunk lanes), weights 2^(m_c - M), LDS sums of the weighted acc and l.
template <int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(const AttnParams p) {
  constexpr int NG = D / 8;          // 8-wide d slices
  constexpr int NC = 256 / NG;       // chunk lanes (16 for D = 128, 32 for D = 64)
  constexpr int MAXR = 8;            // records per thread held at once (splits <= NC * MAXR)
  __shared__ float s_m[256];
  __shared__ float s_l[NC];
  __shared__ float s_acc[NC][D + 4];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid / NG, g = tid % NG;
  const float* base = p.ws + (long long)bh * p.splits * (D + 2);

  float M = -INFINITY, L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += NC * MAXR) {
    // Load a batch of records (independent loads, one round trip).
    float mr[MAXR], lr[MAXR];
    float2 vr[MAXR][4];
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const int s = s0 + c + NC * k;
      mr[k] = -INFINITY;
      lr[k] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) vr[k][e] = make_float2(0.f, 0.f);
      if (s < p.splits) {
        const float* part = base + (long long)s * (D + 2);
        mr[k] = part[D];
        lr[k] = part[D + 1];
        // part is 8-byte aligned (D + 2 floats per record).
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[k][e] = *reinterpret_cast<const float2*>(part + 8 * g + 2 * e);
      }
    }
    // Maximum over this batch and everything before it (all chunk lanes).
    float mloc = M;
#pragma unroll
    for (int k = 0; k < MAXR; ++k) mloc = fmaxf(mloc, mr[k]);
    s_m[tid] = mloc;
    __syncthreads();
    float Mn = -INFINITY;
    for (int cc = 0; cc < NC; ++cc) Mn = fmaxf(Mn, s_m[cc * NG + g]);
    __syncthreads();
    // Rescale what was accumulated against the old maximum, then add the batch.
    const float a0 = (M == -INFINITY || Mn == -INFINITY) ? 0.f : fast_exp2(M - Mn);
    L *= a0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a0;
    M = Mn;
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const float w = (mr[k] == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(mr[k] - M);
      L = __builtin_fmaf(w, lr[k], L);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = __builtin_fmaf(w, vr[k][e].x, acc[2 * e]);
        acc[2 * e + 1] = __builtin_fmaf(w, vr[k][e].y, acc[2 * e + 1]);
      }
    }
  }
  // Sum over the NC chunk lanes (every lane holds the same M).
#pragma unroll
  for (int e = 0; e < 8; ++e) s_acc[c][8 * g + e] = acc[e];
  if (g == 0) s_l[c] = L;
  __syncthreads();
  for (int w = NC / 2; w >= 1; w /= 2) {
    if (c < w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[c][8 * g + e] += s_acc[c + w][8 * g + e];
      if (g == 0) s_l[c] += s_l[c + w];
    }
    __syncthreads();
  }
  const float Lt = s_l[0];
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  const int b = bh / p.Hq, h = bh % p.Hq;
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh;
  const float oscale = inv * p.v_scale;  // v_scale: fp8 V cache dequantisation (else 1)
  for (int d = tid; d < D; d += 256) orow[d] = (__bf16)(s_acc[0][d] * oscale);
  if (p.lse && tid == 0) p.lse[bh] = Lt > 0.f ? (M + __builtin_log2f(Lt)) * kLn2 : -INFINITY;
}

hipError_t launch_decode_split(const AttnParams& p, int D, bool rope, bool kv8, unsigned grid,
                               hipStream_t stream) {
#define ATTNFUSE_DEC(DD, R, K8)                                                                   \
  if (D == DD && rope == R && kv8 == K8) {                                                        \
    hipLaunchKernelGGL((decode_split_kernel<DD, R, K8>), dim3(grid), dim3(kDecNT), 0, stream, p); \
    return hipGetLastError();                                                                     \
  }
  ATTNFUSE_DEC(64, false, false)
  ATTNFUSE_DEC(64, true, false)
  ATTNFUSE_DEC(128, false, false)
  ATTNFUSE_DEC(128, true, false)
  ATTNFUSE_DEC(64, false, true)
  ATTNFUSE_DEC(64, true, true)
  ATTNFUSE_DEC(128, false, true)
  ATTNFUSE_DEC(128, true, true)
#undef ATTNFUSE_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const AttnParams& p, int D, hipStream_t stream) {
  const unsigned grid = (unsigned)(p.B * p.Hq);
  if (D == 64) {
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attnfuse
