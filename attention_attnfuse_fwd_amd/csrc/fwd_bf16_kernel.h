// Fused attention forward, bf16 in / bf16 out, fp32 accumulate, gfx950 MFMA.
//
// One workgroup = NW waves sharing one kv-head.  Wave w owns a 32-query tile
// of q-head  kvh * G + hg * hp + (w % hp)  at rows  qblk * 32 * RB + 32 * (w / hp)
// (RB = NW / hp row blocks).  The workgroup streams 64-key tiles of K and V
// through four-slot LDS rings:
//   global -> LDS by direct DMA, K four and V three tiles ahead (no
//   registers held) ->
//   K rotated in place in LDS two tiles ahead ("4.1 Fused RoPE": each key is
//   rotated once per workgroup, in fp32, by the thread that loaded it) ->
//   MFMA operands (K row fragments; V read transposed by ds_read_b64_tr_b16).
// Per tile and wave:  S^T = K' Q'^T (bf16 MFMA, fp32 acc), score mods and
// masks only where the tile needs them, online softmax ("2 Background /
// FlashAttention and online softmax") with in-lane reductions and one
// cross-half swap, P^T -> bf16, O^T += V^T P^T.  Tiles that the causal /
// window band or the CSR block list rules out are never visited ("4.3
// Block-Sparse Attention": work proportional to the active blocks).
//
// Software pipeline, iteration t (one barrier per iteration):
//   issue the DMA of K(t+4) and V(t+3), then wait for the group issued two
//   iterations earlier;  exp / pack / row sums of tile t while the MFMAs of
//   S(t+1) run;  masks of S(t+1);  score mods and row maximum of S(t+1) and
//   the RoPE rotation of K(t+2) while the MFMAs of O += V(t) P(t) run.
// The running maximum is only moved when it grows by more than 2^8 (exp2
// domain); the result is the same exact softmax and the O^T rescale becomes
// rare.  Row sums are accumulated with bf16 dot products of the very P values
// that feed the P V product, so the normalisation matches the weights used.
#pragma once

#include "common.h"

namespace attnfuse {

// LDS layout for head dim D (bytes): a ring of 4 K slots, a ring of 4 V
// slots and (RoPE) a ring of 4 angle slots.  A K slot holds the tile's RoPE
// halves, each [64 rows][D/2]; a V slot is [64 rows][D].  Every 16-byte chunk
// sits at an XOR-swizzled position inside its row so that the MFMA operand
// reads are free of bank conflicts; a DMA instruction fills 1 KiB of
// consecutive LDS, which the swizzle turns into a permutation of the chunks
// the lanes fetch.
template <int D>
struct TileLds {
  static constexpr int RING = 4;
  static constexpr int KSLOT = 128 * D;     // one K slot
  static constexpr int KHI = 64 * D;        // offset of the high halves in a K slot
  static constexpr int VSLOT = 128 * D;     // one V slot
  static constexpr int V_OFF = RING * KSLOT;
  static constexpr int CPH = D / 16;        // 16-byte chunks per K half row
  static constexpr int KROWS_I = 1024 / D;  // K half rows per DMA instruction
  static constexpr int NKP = D / 16;        // K (low, high) instruction pairs per tile
  static constexpr int CPR = D / 8;         // 16-byte chunks per V row
  static constexpr int VROWS_I = 512 / D;   // V rows per DMA instruction
  static constexpr int NVI = D / 8;         // V instructions per tile
  static constexpr int ANG = 4 * D;         // one angle row: cos[D/2], sin[D/2] in fp32
  static constexpr int A_OFF = V_OFF + RING * VSLOT;
  static constexpr int ASLOT = NKP * ANG;
};

// Swizzle of K half row j: rows that a 16-lane MFMA operand read touches
// together land on distinct banks (two half rows share a 256-byte bank line
// for D = 128, four for D = 64).
template <int D>
__device__ __forceinline__ constexpr int kswz(int j) {
  return (j / (256 / D)) % (D / 16);
}
// Swizzle of V row `key`: the four rows x 64 bytes that half a wave's
// transposing read covers fall on distinct banks, and so do the eight rows x
// 32 bytes of the other half-wave pairing.
template <int D>
__device__ __forceinline__ constexpr int vswz(int key) {
  return D == 128 ? ((4 * (key & 3)) ^ (2 * ((key >> 2) & 1)))
                  : ((4 * ((key >> 1) & 1)) ^ (2 * ((key >> 2) & 1)));
}

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

// Offset (within a 64-key tile) of the key held in S^T subtile `st`, register
// r, by a lane in half lh: 32*st + 8*(r/4) + 4*lh + r%4.  kOff omits 4*lh.
__device__ __forceinline__ constexpr int kOff(int st, int r) { return 32 * st + 8 * (r / 4) + (r % 4); }

template <int D, int NW, bool ROPE, bool SCOREMOD, bool SPARSE>
__global__ void __launch_bounds__(NW * 64)
fwd_bf16_kernel(const AttnParams p) {
  using L = TileLds<D>;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int RING = L::RING;
  constexpr int LDS_BYTES = L::A_OFF + (ROPE ? RING * L::ASLOT : 0);
  // DMA instructions per wave and tile.  V is spread evenly; K pairs may not
  // be (D = 64 with 8 waves: waves 0..3 take one pair each).
  static_assert(L::NVI % NW == 0, "V instructions must spread evenly over the waves");
  static_assert(D == 64 || NW % 2 == 0, "K pair swizzle needs an even wave count for D = 128");
  constexpr int NVW = L::NVI / NW;
  constexpr int NKW_HI = (L::NKP + NW - 1) / NW;
  constexpr int NKW_LO = L::NKP / NW;
  constexpr int GRP_HI = (ROPE ? NKW_HI : 0) + 2 * NKW_HI + NVW;
  constexpr int GRP_LO = (ROPE ? NKW_LO : 0) + 2 * NKW_LO + NVW;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  const uint32_t lds0 = lds_addr(smem);

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
    tpb = p.bn / 64;
    n_tiles = (int)(e - a) * tpb;
  } else {
    int j_lo = 0, j_hi = p.Nk - 1;
    if (p.has_band) {
      j_lo = max(j_lo, r0_wg + max(p.band_lo, -kBandInf));
      j_hi = min(j_hi, (int)min((long long)wg_last + p.band_hi, (long long)kBandInf));
    }
    t_begin = j_lo / 64;
    n_tiles = (j_hi >= j_lo) ? (j_hi / 64 - t_begin + 1) : 0;
  }
  // Column indices are clamped into [0, nkb]; column nkb (or anything past
  // the keys) lands at k0 >= Nk, is loaded clamped and masked out entirely.
  // The list is read with scalar loads, which do not count against vmcnt.
  const int nkb = SPARSE ? (p.Nk + p.bn - 1) / p.bn : 0;
  typedef __attribute__((address_space(4))) const int* cidx_t;
  auto tile_k0 = [&](int t) -> int {
    if (SPARSE) {
      const int col = min(max(((cidx_t)p.col_idx)[s_begin + t / tpb], 0), nkb);
      return col * p.bn + (t % tpb) * 64;
    }
    return (t_begin + t) * 64;
  };

  const int Nk = p.Nk, band_lo = p.band_lo, band_hi = p.band_hi;
  const bool has_band = p.has_band != 0;

  // ---- DMA roles of this thread ----
  const int nkw = wave < L::NKP % NW ? NKW_HI : NKW_LO;  // K pairs of this wave
  const int kjr = lane / L::CPH;                          // half row within a K instruction
  // Logical chunk this lane carries in every K instruction it issues (the
  // swizzle depends on the pair only through its parity, fixed per wave).
  const int kc = (lane % L::CPH) ^ kswz<D>(L::KROWS_I * wave + kjr);
  const int vrow = lane / L::CPR;

  // Angle-row source of this lane: lanes 0 .. D/8-1 fetch cos, the next D/8 sin.
  const float* const rcos = p.rcos;
  const float* const rsin = p.rsin;
  const float* const ang_src = ROPE ? ((lane < D / 8 ? rcos : rsin) + 4 * (lane % (D / 8))) : nullptr;
  const int rope_last = p.rope_len - 1, k_pos0 = p.k_pos0;
  const long long ksn = p.ksn, vsn = p.vsn;
  // First key of tile u, clamped into the key range.  Tiles past the list
  // reload the last tile, so every wave issues the same number of DMA
  // instructions per iteration (their slots are never read as data).
  auto tile_base = [&](int u, int& k0, int& rmax) {
    k0 = tile_k0(min(u, n_tiles - 1));
    const int kc0 = min(k0, Nk - 1);
    rmax = Nk - 1 - kc0;
    return kc0;
  };
  // DMA of K tile u (angle rows first when RoPE) into K / angle slot u % 4.
  auto issue_k = [&](int u) {
    int k0, rmax;
    const int kc0 = tile_base(u, k0, rmax);
    const __bf16* kt = kb + (long long)kc0 * ksn;
    const uint32_t slot = lds0 + (uint32_t)(u % RING) * L::KSLOT;
    if (ROPE) {
#pragma unroll
      for (int m = 0; m < NKW_HI; ++m) {
        const int kp = wave + NW * m;
        if (m < nkw && lane < D / 4) {
          // Row of the first key this pair covers; rows past the table only
          // belong to masked keys.
          const int pb = min(k_pos0 + k0 + L::KROWS_I * kp, rope_last);
          dma16(lds0 + L::A_OFF + (uint32_t)((u % RING) * L::NKP + kp) * L::ANG,
                ang_src + (long long)pb * (D / 2));
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NKW_HI; ++m) {
      const int kp = wave + NW * m;
      if (m < nkw) {
        const int r = min(L::KROWS_I * kp + kjr, rmax);
        const __bf16* src = kt + (long long)r * ksn + 8 * kc;
        dma16(slot + kp * 1024, src);
        dma16(slot + L::KHI + kp * 1024, src + D / 2);
      }
    }
  };
  // DMA of V tile u into V slot u % 4.
  auto issue_v = [&](int u) {
    int k0, rmax;
    const int kc0 = tile_base(u, k0, rmax);
    const __bf16* vt = vb + (long long)kc0 * vsn;
    const uint32_t slot = lds0 + L::V_OFF + (uint32_t)(u % RING) * L::VSLOT;
#pragma unroll
    for (int m = 0; m < NVW; ++m) {
      const int vi = wave + NW * m;
      const int key = L::VROWS_I * vi + vrow;
      const int c = (lane % L::CPR) ^ vswz<D>(key);
      const int r = min(key, rmax);
      dma16(slot + vi * 1024, vt + (long long)r * vsn + 8 * c);
    }
  };
  // The group issued at the top of iteration t is {K(t+4), V(t+3)}.  Waiting
  // until at most two groups are in flight retires the group of iteration
  // t-2: K(t+2) (rotated this iteration) and V(t+1) (read next iteration).
  auto wait_groups = [&]() {
    if constexpr (GRP_HI == GRP_LO) {
      vmcnt_wait<2 * GRP_HI>();
    } else {
      if (nkw == NKW_HI) vmcnt_wait<2 * GRP_HI>();
      else vmcnt_wait<2 * GRP_LO>();
    }
  };

  // ---- RoPE: local angles of this thread's K rows, then in-place rotation ----
  // A K instruction pair covers KROWS_I consecutive keys starting at a row
  // whose angles arrive with the tile; the lane's key sits kjr rows further,
  // so its angle is that row's angle plus kjr * theta_i (angle addition).
  float lcos[8], lsin[8];
  if (ROPE) {
    const int jr = min(kjr, rope_last);
    const F8 c = ld_f8(rcos + (long long)jr * (D / 2) + 8 * kc);
    const F8 s = ld_f8(rsin + (long long)jr * (D / 2) + 8 * kc);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lcos[e] = f8_at(c, e);
      lsin[e] = f8_at(s, e);
    }
  }
  auto rotate = [&](int u) {
    char* slot = smem + (u % RING) * L::KSLOT;
#pragma unroll
    for (int m = 0; m < NKW_HI; ++m) {
      const int kp = wave + NW * m;
      if (m < nkw) {
        const float* ang = reinterpret_cast<const float*>(smem + L::A_OFF + ((u % RING) * L::NKP + kp) * L::ANG);
        const F8 cb = ld_f8(ang + 8 * kc);
        const F8 sb = ld_f8(ang + D / 2 + 8 * kc);
        char* lo_p = slot + kp * 1024 + lane * 16;
        char* hi_p = lo_p + L::KHI;
        const uint4 lo = ld16(lo_p), hi = ld16(hi_p);
        const uint32_t* wl = reinterpret_cast<const uint32_t*>(&lo);
        const uint32_t* wh = reinterpret_cast<const uint32_t*>(&hi);
        uint32_t ol[4], oh[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float l2[2] = {bf16lo(wl[w]), bf16hi(wl[w])};
          float h2[2] = {bf16lo(wh[w]), bf16hi(wh[w])};
          float rl[2], rh[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int e = 2 * w + x;
            const float cB = f8_at(cb, e), sB = f8_at(sb, e);
            const float c = cB * lcos[e] - sB * lsin[e];
            const float s = sB * lcos[e] + cB * lsin[e];
            rl[x] = l2[x] * c - h2[x] * s;
            rh[x] = h2[x] * c + l2[x] * s;
          }
          ol[w] = pack_bf16x2(rl[0], rl[1]);
          oh[w] = pack_bf16x2(rh[0], rh[1]);
        }
        st16(lo_p, make_uint4(ol[0], ol[1], ol[2], ol[3]));
        st16(hi_p, make_uint4(oh[0], oh[1], oh[2], oh[3]));
      }
    }
  };

  // ---- operand addressing ----
  // K fragment (A operand of S^T): row 32*st + lq, chunk 2*kk' + lh of half
  // kk / (NKK/2).  The swizzle is the same for both subtiles.
  const int ksw = kswz<D>(lq);
  auto k_frag = [&](const char* ks, int st, int kk) -> bf16x8 {
    const int half = kk / (NKK / 2), c = 2 * (kk % (NKK / 2)) + lh;
    return *reinterpret_cast<const bf16x8*>(ks + half * L::KHI + (32 * st + lq) * D + 16 * (c ^ ksw));
  };
  // V^T fragment (A operand of O^T += V^T P^T) for 16-key step c and d tile
  // dt: MFMA k index 8*lh + e  <->  key 16c + 8*(e/4) + 4*lh + e%4, which is
  // the order of the P^T registers.  Two transposing reads of 4 keys each.
  const int g16 = lane >> 4, li = lane & 15;
  const int va = li >> 2, vbb = li & 3;
  const int vsw = vswz<D>(4 * lh + va);
  uint32_t voff[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    voff[dt] = (4 * lh + va) * 2 * D + 16 * ((4 * dt + 2 * (g16 & 1) + (vbb >> 1)) ^ vsw) + 8 * (vbb & 1);
  auto v_frag = [&](uint32_t vs, int c, int dt) -> bf16x8 {
    const i16x4 r0 = lds_read_tr4(vs + c * 32 * D + voff[dt]);
    const i16x4 r1 = lds_read_tr4(vs + c * 32 * D + 16 * D + voff[dt]);
    const i16x4 lohalf = r0, hihalf = r1;
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 a = {lohalf[0], lohalf[1], lohalf[2], lohalf[3], hihalf[0], hihalf[1], hihalf[2], hihalf[3]};
    return __builtin_bit_cast(bf16x8, a);
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
        const long long row = (long long)(p.q_pos0 + iq) * (D / 2) + d0;
        rope_rotate_bf16x8(lo, hi, ld_f8(rcos + row), ld_f8(rsin + row));
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

  // S^T of tile u (raw dot products).
  auto s_tile = [&](int u, f32x16 (&s)[2]) {
    const char* ks = smem + (u % RING) * L::KSLOT;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int st = 0; st < 2; ++st) s[st] = mfma32(k_frag(ks, st, kk), qf[kk], s[st]);
  };
  // Masks of tile u in place (only where the tile needs them: the key tail,
  // or the band edge crossing this wave's rows).
  const float scale_log2 = p.scale_log2;
  auto mask_scores = [&](int u, f32x16 (&s)[2]) {
    const int k0 = tile_k0(min(u, n_tiles - 1));
    bool need_mask = k0 + 64 > Nk;
    if (has_band) {
      const int dmin = k0 - w_last, dmax = k0 + 63 - w0;
      need_mask |= (dmin < band_lo) | (dmax > band_hi);
    }
    if (need_mask) {
      // Allowed register offsets form one interval [lo_off, hi_off].
      const int jd = k0 + 4 * lh - i;  // j - i at register offset 0
      int lo_off = -kBandInf, hi_off = Nk - 1 - (k0 + 4 * lh);
      if (has_band) {
        lo_off = band_lo - jd;
        hi_off = min(hi_off, band_hi - jd);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kOff(st, r);
          s[st][r] = ((off >= lo_off) & (off <= hi_off)) ? s[st][r] : -INFINITY;
        }
    }
  };
  // Score mods of tile u in place (scaled, exp2 domain), then the row maximum
  // of this lane's query column over both halves.  Without score mods the
  // scores stay raw and the maximum is scaled instead.
  auto mods_max = [&](int u, f32x16 (&s)[2]) -> float {
    if (SCOREMOD) {
      const int k0 = tile_k0(min(u, n_tiles - 1));
      const float tb = (float)(k0 + 4 * lh - i + dpos);
      const float* brow = nullptr;
      if (p.bias) brow = p.bias + b * p.bsb + h * p.bsh + (long long)iq * p.bsi;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[st][r] * scale_log2;
          x = __builtin_fmaf(slope2, tb + (float)kOff(st, r), x);
          if (brow) {
            const int j = min(k0 + 4 * lh + kOff(st, r), Nk - 1);
            x = __builtin_fmaf(brow[(long long)j * p.bsj], kLog2e, x);
          }
          s[st][r] = x;
        }
    }
    float mx = tree_max32(s[0], s[1]);
    mx = fmaxf(mx, partner32(mx));
    return SCOREMOD ? mx : mx * scale_log2;
  };

  const int n = n_tiles;
  f32x16 sc[2];
  float mx_cur = -INFINITY;
  // Prologue: K(0), K(1) loaded and rotated, V(0) loaded; the groups of
  // iterations -2 and -1 ({K(2), V(1)}, {K(3), V(2)}) in flight; S(0).
  if (n > 0) {
    issue_k(0);
    issue_k(1);
    issue_v(0);
  }
  vmcnt_wait<0>();  // also retires the Q / angle / slope loads above
  if (n > 0) {
    if (ROPE) {
      rotate(0);
      rotate(1);
    }
    issue_k(2);
    issue_v(1);
    issue_k(3);
    issue_v(2);
  }
  __syncthreads();
  if (n > 0) {
    s_tile(0, sc);
    mask_scores(0, sc);
    mx_cur = mods_max(0, sc);
  }
  // Iteration 0 refills K slot 0, which every wave has just read for S(0).
  __syncthreads();

  for (int t = 0; t < n; ++t) {
    issue_k(t + 4);
    issue_v(t + 3);
    wait_groups();

    // Online softmax of tile t with a lazily moved maximum.
    const float m_new = fmaxf(m_run, mx_cur);
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

    // S(t+1) on the matrix cores while tile t is exponentiated.
    f32x16 sn[2];
    s_tile(t + 1, sn);
    bf16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int st = c / 2, r0 = 8 * (c % 2);
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = sc[st][r0 + 2 * q], x1 = sc[st][r0 + 2 * q + 1];
        const float e0 = SCOREMOD ? (x0 - m_use) : __builtin_fmaf(x0, scale_log2, -m_use);
        const float e1 = SCOREMOD ? (x1 - m_use) : __builtin_fmaf(x1, scale_log2, -m_use);
        w[q] = pack_bf16x2(fast_exp2(e0), fast_exp2(e1));
        l_part[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[q]), ones, l_part[q], false);
      }
      pf[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    // One K fragment read, one MFMA and six vector instructions at a time.
#pragma unroll
    for (int k = 0; k < 2 * NKK; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    // Keep P(t) formed here, next to the S(t+1) MFMAs, rather than sunk past
    // the mask branch.
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(pf[c]));
    mask_scores(t + 1, sn);

    // O^T += V^T P^T for tile t while the score mods and maximum of S(t+1)
    // are formed and K(t+2) is rotated.
    const uint32_t vs = lds0 + L::V_OFF + (uint32_t)(t % RING) * L::VSLOT;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma32(v_frag(vs, c, dt), pf[c], o[dt]);
    mx_cur = mods_max(t + 1, sn);
    if (ROPE) rotate(t + 2);
    // Two LDS reads, one MFMA and eight vector instructions at a time.
#pragma unroll
    for (int k = 0; k < 4 * NDT; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __syncthreads();
    sc[0] = sn[0];
    sc[1] = sn[1];
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
