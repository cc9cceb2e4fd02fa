// Fused attention forward, bf16 in / bf16 out, fp32 accumulate, gfx950 MFMA.
//
// One workgroup = NW waves sharing one kv-head.  Wave w owns a 32-query tile
// of q-head  kvh * G + hg * hp + (w % hp)  at rows  qblk * 32 * RB + 32 * (w / hp)
// (RB = NW / hp row blocks).  The workgroup streams 64-key tiles of K and V
// through a double-buffered LDS ring:
//   global -> registers (issued one tile ahead) -> RoPE on the register
//   fragments (K rotated once per workgroup, fp32 math, "4.1 Fused RoPE") ->
//   LDS (K row-major, V transposed) -> MFMA.
// Per tile and wave:  S^T = K' Q'^T (bf16 MFMA, fp32 acc), score mods and
// masks only where the tile needs them, online softmax ("2 Background /
// FlashAttention and online softmax") with in-lane reductions and one
// cross-half swap, P^T -> bf16, O^T += V^T P^T.  Tiles that the causal /
// window band or the CSR block list rules out are never visited ("4.3
// Block-Sparse Attention": work proportional to the active blocks).
//
// Two waves share each SIMD.  The MFMA sections run at raised wave priority,
// so while one wave is in its softmax (vector ALU) the other one's matrix
// products win the issue slot and the two pipes overlap.  The running
// maximum is only moved when it grows by more than 2^8 (exp2 domain); the
// result is the same exact softmax and the O^T rescale becomes rare.  Row
// sums are accumulated with bf16 dot products of the very P values that feed
// the P V product, so the normalisation matches the weights used.
#pragma once

#include "common.h"
#include "tile_stage.h"

namespace attnfuse {

template <int D, int NW>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BN = 64;        // keys per tile
  static constexpr int KSTR = D + 8;   // K row stride in LDS (elements)
  static constexpr int VSTR = BN + 8;  // V^T row stride in LDS
  static constexpr int KBUF = BN * KSTR;
  static constexpr int VBUF = D * VSTR;
  static constexpr int BUF = KBUF + VBUF;  // one ring slot (elements)
};

// Offset (within a 64-key tile) of the key held in S^T subtile `st`, register
// r, by a lane in half lh: 32*st + 8*(r/4) + 4*lh + r%4.  kOff omits 4*lh.
__device__ __forceinline__ constexpr int kOff(int st, int r) { return 32 * st + 8 * (r / 4) + (r % 4); }

// Maximum of 32 values as a balanced tree (exposes ILP; pairs fold into v_max3).
__device__ __forceinline__ float tree_max32(const f32x16& a, const f32x16& b) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = fmaxf(a[i], b[i]);
#pragma unroll
  for (int w = 8; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
  return t[0];
}

template <int D, int NW, bool ROPE, bool SCOREMOD, bool SPARSE>
__global__ void __launch_bounds__(NW * 64)
fwd_bf16_kernel(const AttnParams p) {
  using C = FwdCfg<D, NW>;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;

  // ---- workgroup -> (b, kv-head, head group, query block) ----
  const int hp = p.hp;
  const int RB = NW / hp;
  const int rows_wg = 32 * RB;
  const int unit = blockIdx.x % p.n_units;
  const int qrank = blockIdx.x / p.n_units;
  const int qblk = p.longest_first ? (p.n_qblk - 1 - qrank) : qrank;
  const int n_hg = p.G / hp;
  const int hg = unit % n_hg;
  const int kvh = (unit / n_hg) % p.Hkv;
  const int b = unit / (n_hg * p.Hkv);
  const int h = kvh * p.G + hg * hp + (wave % hp);
  const int r0_wg = qblk * rows_wg;
  const int w0 = r0_wg + 32 * (wave / hp);  // first row of this wave
  const int i = w0 + lq;                    // this lane's query row
  const int iq = min(i, p.Nq - 1);
  const int wg_last = min(r0_wg + rows_wg, p.Nq) - 1;
  const int w_last = min(w0 + 31, p.Nq - 1);

  const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qsb + h * p.qsh;
  const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ksb + kvh * p.ksh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;

  // ---- key tiles this workgroup visits ----
  int n_tiles, t_begin = 0, s_begin = 0, tpb = 1;
  if (SPARSE) {
    const int* rp = p.row_ptr + (p.bs_head_stride ? (long long)h * p.bs_head_stride : 0);
    const int qbs = r0_wg / p.bm;
    const long long nnz = p.bs_nnz;
    const long long a = min(max((long long)rp[qbs], 0LL), nnz);
    const long long e = min(max((long long)rp[qbs + 1], a), nnz);
    s_begin = (int)a;
    tpb = p.bn / C::BN;
    n_tiles = (int)(e - a) * tpb;
  } else {
    int j_lo = 0, j_hi = p.Nk - 1;
    if (p.has_band) {
      j_lo = max(j_lo, r0_wg + max(p.band_lo, -kBandInf));
      j_hi = min(j_hi, (int)min((long long)wg_last + p.band_hi, (long long)kBandInf));
    }
    t_begin = j_lo / C::BN;
    n_tiles = (j_hi >= j_lo) ? (j_hi / C::BN - t_begin + 1) : 0;
  }
  // Column indices are clamped into [0, nkb]; column nkb (or anything past
  // the keys) lands at k0 >= Nk and is skipped, never loaded out of range.
  const int nkb = SPARSE ? (p.Nk + p.bn - 1) / p.bn : 0;
  auto tile_k0 = [&](int t) -> int {
    if (SPARSE) {
      const int col = min(max(p.col_idx[s_begin + t / tpb], 0), nkb);
      return col * p.bn + (t % tpb) * C::BN;
    }
    return (t_begin + t) * C::BN;
  };

  // ---- Q fragments: load, rotate once, keep as bf16 B operands ----
  bf16x8 qf[NKK];
  {
    const __bf16* qrow = qb + (long long)iq * p.qsn;
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      const int d0 = 16 * kk + 8 * lh;
      uint4 lo = ld16(qrow + d0);
      uint4 hi = ld16(qrow + d0 + D / 2);
      if (ROPE) {
        const uint32_t* row = p.rcs + (long long)(p.q_pos0 + iq) * (D / 2) + d0;
        rope_rotate_bf16x8_h(lo, hi, ld16(row), ld16(row + 4));
      }
      qf[kk] = __builtin_bit_cast(bf16x8, lo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, hi);
    }
  }

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;                 // running max, exp2 domain
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's partial row sums
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const float slope2 = (SCOREMOD && p.alibi) ? p.alibi[h] * kLog2e : 0.f;
  const int dpos = p.k_pos0 - p.q_pos0;

  TileStage<D, C::BN, C::NT, ROPE> stage;
  if (n_tiles > 0) {
    stage.load(p, kb, vb, tile_k0(0), p.Nk, tid);
    stage.store(smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = tile_k0(t);
    const bool more = t + 1 < n_tiles;
    if (more) stage.load(p, kb, vb, tile_k0(t + 1), p.Nk, tid);

    // Does this wave see the tile at all, and does it need element masks?
    // j - i spans [k0 - w_last, k0 + 63 - w0] over this wave's rows.
    bool skip = k0 >= p.Nk || w0 >= p.Nq;
    bool need_mask = k0 + C::BN > p.Nk;
    if (p.has_band) {
      const int dmin = k0 - w_last, dmax = k0 + C::BN - 1 - w0;
      skip |= (dmax < p.band_lo) || (dmin > p.band_hi);
      need_mask |= (dmin < p.band_lo) || (dmax > p.band_hi);
    }

    if (!skip) {
      const __bf16* ks = smem + (t & 1) * C::BUF;
      const __bf16* vs = ks + C::KBUF;

      // S^T = K' Q'^T for keys k0 .. k0+63 (two 32-key subtiles).
      f32x16 s[2];
      s[0] = f32x16{};
      s[1] = f32x16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (32 * st + lq) * C::KSTR + 16 * kk + 8 * lh);
          s[st] = mfma32(a, qf[kk], s[st]);
        }
      }
      __builtin_amdgcn_s_setprio(0);

      // Score mods and masks, then the tile maximum.
      const int jd = k0 + 4 * lh - i;  // j - i at register offset 0
      if (SCOREMOD) {
        const float tb = (float)(jd + dpos);
        const float* brow = nullptr;
        if (p.bias) brow = p.bias + b * p.bsb + h * p.bsh + (long long)iq * p.bsi;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[st][r] * p.scale_log2;
            x = __builtin_fmaf(slope2, tb + (float)kOff(st, r), x);
            if (brow) {
              const int j = min(k0 + 4 * lh + kOff(st, r), p.Nk - 1);
              x = __builtin_fmaf(brow[(long long)j * p.bsj], kLog2e, x);
            }
            s[st][r] = x;
          }
      }
      if (need_mask) {
        const int jb = k0 + 4 * lh;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kOff(st, r);
            bool ok = jb + off < p.Nk;
            if (p.has_band) ok = ok && (jd + off >= p.band_lo) && (jd + off <= p.band_hi);
            s[st][r] = ok ? s[st][r] : -INFINITY;
          }
      }
      float mx = tree_max32(s[0], s[1]);
      mx = fmaxf(mx, partner32(mx));
      if (!SCOREMOD) mx *= p.scale_log2;

      // Online softmax with a lazily moved maximum.
      const float m_new = fmaxf(m_run, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f)) {
        const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
#pragma unroll
        for (int q = 0; q < 4; ++q) l_part[q] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = SCOREMOD ? (s[st][r] - m_use) : __builtin_fmaf(s[st][r], p.scale_log2, -m_use);
          s[st][r] = fast_exp2(x);
        }

      // P^T as bf16 B operands: 16-key step c takes registers 8*(c%2) .. +7 of
      // subtile c/2; the row sum takes the same bf16 values.
      bf16x8 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int st = c / 2, r0 = 8 * (c % 2);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = pack_bf16x2(s[st][r0 + 2 * q], s[st][r0 + 2 * q + 1]);
          l_part[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[q]), ones,
                                                      l_part[q], false);
        }
        pf[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
      // O^T += V^T P^T
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (32 * dt + lq) * C::VSTR + 16 * c + 8 * lh);
          o[dt] = mfma32(a, pf[c], o[dt]);
        }
      __builtin_amdgcn_s_setprio(0);
    }

    if (more) stage.store(smem + ((t + 1) & 1) * C::BUF, tid);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, optional lse ----
  const float l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  const float l_tot = l_run + partner32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (i < p.Nq) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh + (long long)i * p.osn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * lh;
        uint2 w;
        w.x = pack_bf16x2(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv);
        w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = w;
      }
    if (p.lse && lh == 0)
      p.lse[((long long)b * p.Hq + h) * p.Nq + i] =
          l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace attnfuse
