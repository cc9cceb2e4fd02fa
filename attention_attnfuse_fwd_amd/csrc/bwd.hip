// Attention backward ("4.4 Backward Pass"), the FlashAttention-2 split into
// three passes, none of which needs atomics:
//   1. delta[b, h, i] = sum_d dO[i, d] O[i, d]            (row reduction)
//   2. per (b, kv-head, block of 128 keys): dK and dV, looping over the
//      q-heads of the group and the query tiles the masks allow
//   3. per (b, q-head, block of 128 query rows): dQ, looping over key tiles
// Probabilities are re-derived tile by tile from the forward's saved
// L = m + ln l:  P = exp(S - L),  dS = P (dP - delta),  dQ' = scale dS K',
// dK' = scale dS^T Q',  dV = P^T dO; the RoPE gradients rotate dQ' and dK'
// back by the negative angle (the rotation is orthogonal).
//
// All products run on bf16 MFMA (32x32x16, fp32 accumulate) with the
// operands the forward uses: rotated Q and K rounded once to bf16, P and dS
// rounded to bf16.  Tiles are staged through padded row-major LDS; the
// transposed operands (dO^T, Q'^T, K'^T) are read with ds_read_b64_tr_b16.
// This first version loads each tile synchronously (no prefetch).
#include "common.h"
#include "launch.h"

namespace attnfuse {

namespace {

constexpr int kBwdThreads = 256;  // 4 waves

// Transposed A operand (32 rows of the result x 16 contraction steps) from a
// row-major bf16 tile T[row][RS] in LDS, for MFMA k index 8*kb + e  <->  tile
// row row0 + 8*(e/4) + 4*kb + e%4 (the order in which a 32x32 accumulator
// holds its rows), result row = column col0 + lane % 32.
template <int RS>
__device__ __forceinline__ bf16x8 tr_frag(uint32_t tile, int row0, int col0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  const int kb = g >> 1, c16 = 16 * (g & 1);
  const int a = i >> 2, bq = i & 3;
  const uint32_t r1 = tile + (uint32_t)(((row0 + 4 * kb + a) * RS + col0 + c16 + 4 * bq) * 2);
  const uint32_t r2 = r1 + (uint32_t)(8 * RS * 2);
  const i16x4 x = lds_read_tr4(r1), y = lds_read_tr4(r2);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Row-major A / B operand: 8 consecutive elements of row `row`, columns
// 16*kk + 8*kb .. +7.
template <int RS>
__device__ __forceinline__ bf16x8 row_frag(const __bf16* tile, int row, int kk) {
  const int kb = (threadIdx.x & 63) >> 5;
  return *reinterpret_cast<const bf16x8*>(tile + row * RS + 16 * kk + 8 * kb);
}

// 8 bf16 values of row `row` (global, element stride sn), columns c .. c+7.
__device__ __forceinline__ uint4 ld_row8(const __bf16* base, long long sn, int row, int c) {
  return ld16(base + (long long)row * sn + c);
}

// Rows [r0, r0 + R) of a [N, D] bf16 matrix (rows clamped to N - 1), staged
// in two steps so the next tile's loads can be in flight while the current
// one is multiplied: load() reads this thread's share into registers (with
// the RoPE angles when rope), store() rotates it and writes a padded LDS tile.
template <int D, int R, int RS>
struct RowStage {
  static constexpr int CH = D / 16;                         // chunk pairs per row
  static constexpr int U = (R * CH + kBwdThreads - 1) / kBwdThreads;
  uint4 lo[U], hi[U];
  F8 c[U], s[U];
  __device__ __forceinline__ void load(const __bf16* src, long long sn, int r0, int N, bool rope,
                                       const AttnParams& p, int pos0) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = threadIdx.x + kBwdThreads * k;
      if ((R * CH) % kBwdThreads == 0 || u < R * CH) {
        const int row = u / CH, ch = u % CH;
        const int rs = min(r0 + row, N - 1);
        lo[k] = ld_row8(src, sn, rs, 8 * ch);
        hi[k] = ld_row8(src, sn, rs, D / 2 + 8 * ch);
        if (rope) {
          const int pos = min(pos0 + rs, p.rope_len - 1);
          c[k] = ld_f8(p.rcos + (long long)pos * (D / 2) + 8 * ch);
          s[k] = ld_f8(p.rsin + (long long)pos * (D / 2) + 8 * ch);
        }
      }
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, bool rope) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = threadIdx.x + kBwdThreads * k;
      if ((R * CH) % kBwdThreads == 0 || u < R * CH) {
        const int row = u / CH, ch = u % CH;
        uint4 l = lo[k], h = hi[k];
        if (rope) rope_rotate_bf16x8(l, h, c[k], s[k]);
        st16(tile + row * RS + 8 * ch, l);
        st16(tile + row * RS + D / 2 + 8 * ch, h);
      }
    }
  }
};

// Register fragments of one row (lane's row) as a B operand over the head
// dim: f[kk] = row[16 kk + 8 kb .. +7]; rotated when rope (the low and high
// halves of the row sit in f[kk] and f[kk + D/32]).
template <int D>
__device__ __forceinline__ void row_frags(bf16x8 (&f)[D / 16], const __bf16* src, long long sn,
                                          int row, bool rope, const AttnParams& p, int pos) {
  const int kb = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const int d0 = 16 * kk + 8 * kb;
    uint4 lo = ld_row8(src, sn, row, d0);
    uint4 hi = ld_row8(src, sn, row, D / 2 + d0);
    if (rope) {
      const int ps = min(pos, p.rope_len - 1);
      rope_rotate_bf16x8(lo, hi, ld_f8(p.rcos + (long long)ps * (D / 2) + d0),
                         ld_f8(p.rsin + (long long)ps * (D / 2) + d0));
    }
    f[kk] = __builtin_bit_cast(bf16x8, lo);
    f[kk + D / 32] = __builtin_bit_cast(bf16x8, hi);
  }
}

// Un-rotate (rotate by the negative angle) an accumulator held as
// acc[dt][r] = value at d = 32 dt + 8 (r/4) + 4 kb + r%4 of the lane's row,
// scale it, and store it as bf16 to dst (row pointer).
template <int D>
__device__ __forceinline__ void store_grad_row(__bf16* dst, const f32x16 (&acc)[D / 32], float scale,
                                               bool rope, const AttnParams& p, int pos) {
  constexpr int NDT = D / 32;
  const int kb = (threadIdx.x & 63) >> 5;
  float v[NDT][16];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[dt][r] = acc[dt][r] * scale;
  if (rope) {
    const int ps = min(pos, p.rope_len - 1);
#pragma unroll
    for (int dt = 0; dt < NDT / 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r / 4) + 4 * kb + r % 4;  // < D/2: the pair index
        const float c = p.rcos[(long long)ps * (D / 2) + d], s = p.rsin[(long long)ps * (D / 2) + d];
        const float lo = v[dt][r], hi = v[dt + NDT / 2][r];
        v[dt][r] = lo * c + hi * s;
        v[dt + NDT / 2][r] = hi * c - lo * s;
      }
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * kb;
      uint2 w;
      w.x = pack_bf16x2(v[dt][4 * g], v[dt][4 * g + 1]);
      w.y = pack_bf16x2(v[dt][4 * g + 2], v[dt][4 * g + 3]);
      *reinterpret_cast<uint2*>(dst + d) = w;
    }
}

}  // namespace

// ---- pass 1: delta = rowsum(dO * O) ----
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const AttnParams p, const BwdParams g) {
  constexpr int CPR = D / 8;         // chunks per row
  constexpr int RPB = 256 / CPR;     // rows per block
  const long long rows = (long long)p.B * p.Hq * p.Nq;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < rows) {
    const int i = (int)(row % p.Nq);
    const long long bh = row / p.Nq;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + b * p.osb + h * p.osh + (long long)i * p.osn;
    const __bf16* d = g.dout + b * p.osb + h * p.osh + (long long)i * p.osn;
    const uint4 ov = ld16(o + 8 * c), dv = ld16(d + 8 * c);
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov);
    const uint32_t* dw = reinterpret_cast<const uint32_t*>(&dv);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += bf16lo(ow[w]) * bf16lo(dw[w]) + bf16hi(ow[w]) * bf16hi(dw[w]);
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, CPR);
  if (row < rows && c == 0) g.delta[row] = acc;
}

// ---- pass 3: dQ.  4 waves x 32 query rows of one q-head; key tiles of 64. ----
template <int D>
__global__ void __launch_bounds__(kBwdThreads, 1) bwd_dq_kernel(const AttnParams p, const BwdParams g) {
  constexpr int NKK = D / 16, NDT = D / 32, RS = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 ks[64 * RS];
  __shared__ __attribute__((aligned(16))) __bf16 vs[64 * RS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 31, lh = lane >> 5;
  const int nqb = (p.Nq + 127) / 128;
  const int qblk = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.G;
  const int r0 = qblk * 128;
  const int i = r0 + 32 * wave + lq;
  const int iq = min(i, p.Nq - 1);
  const bool rope = p.rcos != nullptr;

  const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qsb + h * p.qsh;
  const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ksb + kvh * p.ksh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;
  const __bf16* dob = g.dout + b * p.osb + h * p.osh;

  // The lane's query row: Q' and dO as B operands over the head dim.
  bf16x8 qf[NKK], df[NKK];
  row_frags<D>(qf, qb, p.qsn, iq, rope, p, p.q_pos0 + iq);
  row_frags<D>(df, dob, p.osn, iq, false, p, 0);
  const long long row_id = ((long long)b * p.Hq + h) * p.Nq + iq;
  const float lse = p.lse[row_id];
  const float lse2 = lse * kLog2e;
  const float delta = g.delta[row_id];
  const bool row_ok = i < p.Nq && lse != -INFINITY;
  const float slope2 = p.alibi ? p.alibi[h] * kLog2e : 0.f;
  const int dpos = p.k_pos0 - p.q_pos0;

  // Key tiles any row of the block may see (the band is j - i in index space).
  const int wg_last = min(r0 + 127, p.Nq - 1);
  int j_lo = 0, j_hi = p.Nk - 1;
  if (p.has_band) {
    j_lo = max(j_lo, (int)max((long long)r0 + p.band_lo, 0LL));
    j_hi = min(j_hi, (int)min((long long)wg_last + p.band_hi, (long long)p.Nk - 1));
  }
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  const uint32_t ks_lds = lds_addr(ks);
  RowStage<D, 64, RS> kst, vst;
  const int kt0 = (j_lo / 64) * 64;
  if (j_hi >= j_lo) {
    kst.load(kb, p.ksn, kt0, p.Nk, rope, p, p.k_pos0);
    vst.load(vb, p.vsn, kt0, p.Nk, false, p, 0);
  }
  for (int k0 = kt0; j_hi >= j_lo && k0 <= j_hi; k0 += 64) {
    __syncthreads();
    kst.store(ks, rope);
    vst.store(vs, false);
    __syncthreads();
    if (k0 + 64 <= j_hi) {  // the next tile's loads overlap this tile's products
      kst.load(kb, p.ksn, k0 + 64, p.Nk, rope, p, p.k_pos0);
      vst.load(vb, p.vsn, k0 + 64, p.Nk, false, p, 0);
    }
    // S^T and dP^T for two 32-key subtiles (lane = query column).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
      dp[st] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s[st] = mfma32(row_frag<RS>(ks, 32 * st + lq, kk), qf[kk], s[st]);
        dp[st] = mfma32(row_frag<RS>(vs, 32 * st + lq, kk), df[kk], dp[st]);
      }
    }
    // dS^T = P^T (dP^T - delta), packed to bf16 in 16-key chunks.
    bf16x8 dsf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        float x2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int st = c / 2, r = 8 * (c % 2) + 2 * q2 + e;
          const int j = k0 + 32 * st + 8 * (r / 4) + 4 * lh + r % 4;
          bool ok = row_ok && j < p.Nk;
          if (p.has_band) ok = ok && (j - i >= p.band_lo) && (j - i <= p.band_hi);
          float x = s[st][r] * p.scale_log2 - lse2;
          if (p.alibi) x = __builtin_fmaf(slope2, (float)(j - i + dpos), x);
          const float pr = ok ? fast_exp2(x) : 0.f;
          x2[e] = pr * (dp[st][r] - delta);
        }
        w[q2] = pack_bf16x2(x2[0], x2[1]);
      }
      dsf[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    // dQ'^T += K'^T dS^T.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[dt] = mfma32(tr_frag<RS>(ks_lds, 16 * c, 32 * dt), dsf[c], acc[dt]);
  }
  if (i < p.Nq) {
    __bf16* dst = g.dq + b * p.qsb + h * p.qsh + (long long)i * p.qsn;
    store_grad_row<D>(dst, acc, p.scale_log2 / kLog2e, rope, p, p.q_pos0 + i);
  }
}

// ---- pass 2: dK, dV.  4 waves x 32 keys of one kv-head; query tiles of 32. ----
template <int D>
__global__ void __launch_bounds__(kBwdThreads, 1) bwd_dkdv_kernel(const AttnParams p, const BwdParams g) {
  constexpr int NKK = D / 16, NDT = D / 32, RS = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 qs[32 * RS];
  __shared__ __attribute__((aligned(16))) __bf16 dos[32 * RS];
  __shared__ float lse_s[32], delta_s[32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 31, lh = lane >> 5;
  const int nkb = (p.Nk + 127) / 128;
  const int kblk = blockIdx.x % nkb;
  const int bk = blockIdx.x / nkb;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int k0 = kblk * 128;
  const int j = k0 + 32 * wave + lq;  // the lane's key (result column)
  const int jc = min(j, p.Nk - 1);
  const bool rope = p.rcos != nullptr;

  const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ksb + kvh * p.ksh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;
  bf16x8 kf[NKK], vf[NKK];
  row_frags<D>(kf, kb, p.ksn, jc, rope, p, p.k_pos0 + jc);
  row_frags<D>(vf, vb, p.vsn, jc, false, p, 0);
  const int dpos = p.k_pos0 - p.q_pos0;

  // Query rows that may see a key of the block: band_lo <= j - i <= band_hi.
  const int k_last = min(k0 + 127, p.Nk - 1);
  int i_lo = 0, i_hi = p.Nq - 1;
  if (p.has_band) {
    i_lo = max(i_lo, (int)max((long long)k0 - p.band_hi, 0LL));
    i_hi = min(i_hi, (int)min((long long)k_last - p.band_lo, (long long)p.Nq - 1));
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = f32x16{};
  const uint32_t qs_lds = lds_addr(qs), dos_lds = lds_addr(dos);
  // (head, query tile) steps: the group's q-heads one after the other, each
  // over the query tiles the band allows; the next step's loads are issued
  // before this step's products.
  const int qt0 = (i_lo / 32) * 32;
  const int ntq = i_hi >= i_lo ? (i_hi - qt0) / 32 + 1 : 0;
  const int nsteps = ntq * p.G;
  RowStage<D, 32, RS> qst, dst;
  float lse_r = 0.f, delta_r = 0.f;
  auto load_step = [&](int t) {
    const int h = kvh * p.G + t / ntq, q0 = qt0 + 32 * (t % ntq);
    qst.load(reinterpret_cast<const __bf16*>(p.q) + b * p.qsb + h * p.qsh, p.qsn, q0, p.Nq, rope, p,
             p.q_pos0);
    dst.load(g.dout + b * p.osb + h * p.osh, p.osn, q0, p.Nq, false, p, 0);
    if (threadIdx.x < 32) {
      const long long rr = ((long long)b * p.Hq + h) * p.Nq + min(q0 + (int)threadIdx.x, p.Nq - 1);
      lse_r = p.lse[rr];
      delta_r = g.delta[rr];
    }
  };
  if (nsteps > 0) load_step(0);
  for (int t = 0; t < nsteps; ++t) {
    const int h = kvh * p.G + t / ntq, q0 = qt0 + 32 * (t % ntq);
    const float slope2 = p.alibi ? p.alibi[h] * kLog2e : 0.f;
    __syncthreads();
    qst.store(qs, rope);
    dst.store(dos, false);
    if (threadIdx.x < 32) {
      lse_s[threadIdx.x] = lse_r;
      delta_s[threadIdx.x] = delta_r;
    }
    __syncthreads();
    if (t + 1 < nsteps) load_step(t + 1);
    // S and dP (32 query rows x the wave's 32 keys; lane = key column).
    f32x16 s = f32x16{}, dpv = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s = mfma32(row_frag<RS>(qs, lq, kk), kf[kk], s);
      dpv = mfma32(row_frag<RS>(dos, lq, kk), vf[kk], dpv);
    }
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t wp[4], wd[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        float pv[2], dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 8 * c + 2 * q2 + e;
          const int m = 8 * (r / 4) + 4 * lh + r % 4;  // query row within the tile
          const int ii = q0 + m;
          const float lse = lse_s[m];
          bool ok = ii < p.Nq && j < p.Nk && lse != -INFINITY;
          if (p.has_band) ok = ok && (j - ii >= p.band_lo) && (j - ii <= p.band_hi);
          float x = s[r] * p.scale_log2 - lse * kLog2e;
          if (p.alibi) x = __builtin_fmaf(slope2, (float)(j - ii + dpos), x);
          pv[e] = ok ? fast_exp2(x) : 0.f;
          dsv[e] = pv[e] * (dpv[r] - delta_s[m]);
        }
        wp[q2] = pack_bf16x2(pv[0], pv[1]);
        wd[q2] = pack_bf16x2(dsv[0], dsv[1]);
      }
      pf[c] = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
      dsf[c] = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
    }
    // dV^T += dO^T P,  dK'^T += Q'^T dS.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dv[dt] = mfma32(tr_frag<RS>(dos_lds, 16 * c, 32 * dt), pf[c], dv[dt]);
        dk[dt] = mfma32(tr_frag<RS>(qs_lds, 16 * c, 32 * dt), dsf[c], dk[dt]);
      }
  }
  if (j < p.Nk) {
    __bf16* dkd = g.dk + b * p.ksb + kvh * p.ksh + (long long)j * p.ksn;
    __bf16* dvd = g.dv + b * p.vsb + kvh * p.vsh + (long long)j * p.vsn;
    store_grad_row<D>(dkd, dk, p.scale_log2 / kLog2e, rope, p, p.k_pos0 + j);
    store_grad_row<D>(dvd, dv, 1.f, false, p, 0);
  }
}

hipError_t launch_bwd(const AttnParams& p, const BwdParams& g, int D, hipStream_t stream) {
  const long long rows = (long long)p.B * p.Hq * p.Nq;
  const unsigned grid_q = (unsigned)((long long)p.B * p.Hq * ((p.Nq + 127) / 128));
  const unsigned grid_k = (unsigned)((long long)p.B * p.Hkv * ((p.Nk + 127) / 128));
#define ATTNFUSE_BWD(DD)                                                                           \
  if (D == DD) {                                                                                   \
    constexpr int rpb = 256 / (DD / 8);                                                            \
    if (rows > 0)                                                                                  \
      hipLaunchKernelGGL(bwd_delta_kernel<DD>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), \
                         0, stream, p, g);                                                         \
    if (grid_k > 0)                                                                                \
      hipLaunchKernelGGL(bwd_dkdv_kernel<DD>, dim3(grid_k), dim3(kBwdThreads), 0, stream, p, g);    \
    if (grid_q > 0)                                                                                \
      hipLaunchKernelGGL(bwd_dq_kernel<DD>, dim3(grid_q), dim3(kBwdThreads), 0, stream, p, g);      \
    return hipGetLastError();                                                                      \
  }
  ATTNFUSE_BWD(64)
  ATTNFUSE_BWD(128)
#undef ATTNFUSE_BWD
  return hipErrorInvalidValue;
}

}  // namespace attnfuse
