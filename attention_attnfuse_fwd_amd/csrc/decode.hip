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
// Partial layout in the workspace (fp32), two arrays: acc [B][Hq][splits][D]
// (un-normalised output rows, 16-byte aligned), then ml [B][Hq][splits][2]
// holding m (running maximum, exp2 domain, scaled) and l (the sum of the
// exponentials) of each chunk.
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
  kst.init(p, lane);
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
    const long long rec = ((long long)b * p.Hq + kvh * p.G + gg) * p.splits + split;
    p.ws[rec * D + d] = acc;
    if (d == 0) {
      float* ml = p.ws + (long long)p.B * p.Hq * p.splits * D + 2 * rec;
      ml[0] = M;
      ml[1] = L;
    }
  }
}

// Phase 2: one wave per (b, q-head, 32-wide slice of d), one memory round
// trip for up to 64 chunks.  Lane s holds chunk s's (m, l) and its 32 acc
// values; lanes merge their own chunks first (more than 64 chunks: online, in
// steps of 64), then the wave takes M = max m, rescales every lane's (l, acc)
// by 2^(m - M), and sums l with lane shuffles and the 32 acc columns through
// LDS.
template <int D>
__global__ void __launch_bounds__(64) decode_combine_kernel(const AttnParams p) {
  constexpr int NC = D / 32;  // d slices per head
  __shared__ float red[64][33];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
  const long long n_rec = (long long)p.B * p.Hq * p.splits;
  const float* accb = p.ws + (long long)bh * p.splits * D + 32 * c;
  const float* mlb = p.ws + n_rec * D + (long long)bh * p.splits * 2;

  float M = -INFINITY, L = 0.f;
  float a[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) a[e] = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += 64) {
    const int s = s0 + lane;
    float m = -INFINITY, l = 0.f;
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < p.splits) {
      const float2 ml = *reinterpret_cast<const float2*>(mlb + 2 * s);
      m = ml.x;
      l = ml.y;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const float4*>(accb + (long long)s * D + 4 * k);
    }
    const float Mn = fmaxf(M, m);
    const float wa = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
    const float wb = (m == -INFINITY) ? 0.f : fast_exp2(m - Mn);
    M = Mn;
    L = L * wa + l * wb;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[4 * k + 0] = a[4 * k + 0] * wa + v[k].x * wb;
      a[4 * k + 1] = a[4 * k + 1] * wa + v[k].y * wb;
      a[4 * k + 2] = a[4 * k + 2] * wa + v[k].z * wb;
      a[4 * k + 3] = a[4 * k + 3] * wa + v[k].w * wb;
    }
  }
  float Mg = M;
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) Mg = fmaxf(Mg, __shfl_xor(Mg, off));
  const float w = (M == -INFINITY) ? 0.f : fast_exp2(M - Mg);
  float Lg = L * w;
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) Lg += __shfl_xor(Lg, off);
#pragma unroll
  for (int e = 0; e < 32; ++e) red[lane][e] = a[e] * w;
  __syncthreads();
  // lane t sums column t % 32 over rows 32 * (t / 32) .. + 31; the halves meet by a swap
  const int col = lane & 31, r0 = 32 * (lane >> 5);
  float acc = 0.f;
#pragma unroll 8
  for (int r = 0; r < 32; ++r) acc += red[r0 + r][col];
  acc += partner32(acc);
  const float inv = Lg > 0.f ? 1.f / Lg : 0.f;
  const int b = bh / p.Hq, h = bh % p.Hq;
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh;
  if (lane < 32) orow[32 * c + lane] = (__bf16)(acc * inv * p.v_scale);  // v_scale: fp8 V cache
  if (p.lse && c == 0 && lane == 0) p.lse[bh] = Lg > 0.f ? (Mg + __builtin_log2f(Lg)) * kLn2 : -INFINITY;
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
  const unsigned grid = (unsigned)(p.B * p.Hq * (D / 32));
  if (D == 64) {
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(grid), dim3(64), 0, stream, p);
  } else if (D == 128) {
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(grid), dim3(64), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attnfuse
