// Fused attention forward, bf16 in / bf16 out, fp32 accumulate, gfx950 MFMA.
//
// One workgroup = NW waves sharing one kv-head.  Wave w owns a 32-query tile
// of q-head  kvh * G + hg * hp + (w % hp)  at rows  qblk * 32 * RB + 32 * (w / hp)
// (RB = NW / hp row blocks).  The workgroup streams 64-key tiles of K and V
// through four-slot LDS rings:
//   global -> LDS by direct DMA, K four and V three tiles ahead (no
//   registers held) ->
//   K rotated in place in LDS two tiles ahead ("4.1 Fused RoPE": each key is
//   rotated once per workgroup by the thread that loaded it, in fp32 on the
//   exact bf16 values, against a precomputed fp16 (cos, sin) table whose
//   entries the thread fetched into a private LDS slot) ->
//   MFMA operands (K row fragments; V read transposed by ds_read_b64_tr_b16).
// Per tile and wave:  S^T = K' Q'^T (bf16 MFMA, fp32 acc), score mods and
// masks only where the tile needs them, online softmax ("2 Background /
// FlashAttention and online softmax") with in-lane reductions and one
// cross-half swap, P^T -> bf16, O^T += V^T P^T.  Tiles that the causal /
// window band or the CSR block list rules out are never visited ("4.3
// Block-Sparse Attention": work proportional to the active blocks).
//
// Software pipeline, iteration t (one barrier per iteration):
//   wait for the DMA group issued two iterations earlier (and the table
//   entries of the previous one);  the MFMAs of S(t+1) with the RoPE
//   rotation of K(t+2) between them;  masks of S(t+1);  the MFMAs of
//   O += V(t) P(t) with the exp / pack / row sums of S(t+1) between them.
//   The DMA of K(t+4) is issued one instruction per step in the first phase,
//   the table entries of K(t+3) and V(t+3) in the second.
// The running maximum is only moved when a tile's scores exceed it by more
// than 15 (exp2 domain); the result is the same exact softmax and the O^T
// rescale becomes rare.  Row sums come out of the matrix core: one more
// P V-shaped MFMA per 16 keys with an all-ones A operand sums the very bf16
// P values that feed the P V product, so the normalisation matches the
// weights used (and no vector dot product has to queue behind the MFMAs).
#pragma once

#include "common.h"

namespace attnfuse {

// LDS layout for head dim D (bytes): a ring of 4 K slots, a ring of 4 V
// slots and (RoPE) one table slot.  A K slot holds the tile's RoPE halves,
// each [64 rows][D/2]; a V slot is [64 rows][D]; the table slot holds, per K
// instruction pair, 2 KiB of fp16 (cos, sin) words: 32 bytes per thread, the
// 8 angles of the 8-element chunk it rotates, read back only by that thread.  Every 16-byte chunk
// sits at an XOR-swizzled position inside its row so that the MFMA operand
// reads are free of bank conflicts; a DMA instruction fills 1 KiB of
// consecutive LDS, which the swizzle turns into a permutation of the chunks
// the lanes fetch.
template <int D, int R = 4>
struct TileLds {
  static constexpr int RING = R;
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
  static constexpr int T_OFF = V_OFF + RING * VSLOT;
  static constexpr int TPAIR = 2048;        // table bytes per K instruction pair
  static constexpr int TSLOT = NKP * TPAIR;
  static constexpr int ROWB = 2 * D;        // bytes per table row (D/2 words)
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

// Largest bit pattern, read as a signed integer, of 32 floats: for a
// non-negative threshold T, the result exceeds bits(T) exactly when some
// value exceeds T or is a positive NaN (negative values compare below).
// Integer max3 needs no NaN canonicalisation, unlike fmaxf.
__device__ __forceinline__ int tree_max32_bits(const f32x16& a, const f32x16& b) {
  int t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    t[i] = max(max(__float_as_int(a[3 * i]), __float_as_int(a[3 * i + 1])), __float_as_int(a[3 * i + 2]));
    t[5 + i] = max(max(__float_as_int(b[3 * i]), __float_as_int(b[3 * i + 1])), __float_as_int(b[3 * i + 2]));
  }
  t[10] = max(__float_as_int(a[15]), __float_as_int(b[15]));
  const int u0 = max(max(t[0], t[1]), t[2]), u1 = max(max(t[3], t[4]), t[5]);
  const int u2 = max(max(t[6], t[7]), t[8]), u3 = max(t[9], t[10]);
  return max(max(u0, u1), max(u2, u3));
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

// LDS layout of the FP8 instances (bytes): Q and K stay OCP E4M3 codes and
// meet on the fp8 matrix core, so a K slot holds the tile's codes [64 rows][D]
// (16-byte chunks XOR-swizzled by row, k8swz); V is converted once per
// workgroup to bf16 into the same V slots as the bf16 instances, from a
// two-deep staging ring where each thread finds the 16 codes it loaded itself.
template <int D>
struct Fp8Lds {
  static constexpr int KSLOT = 64 * D;
  static constexpr int V_OFF = 4 * KSLOT;
  static constexpr int VSLOT = 128 * D;
  static constexpr int S_OFF = V_OFF + 4 * VSLOT;
  static constexpr int SSLOT = 64 * D;
  static constexpr int BYTES = S_OFF + 2 * SSLOT;
  static constexpr int NI = D / 16;          // DMA instructions per K (or V) tile
  static constexpr int ROWS_I = 1024 / D;    // rows per DMA instruction
  static constexpr int CPR = D / 16;         // 16-byte chunks per row
};
// Swizzle of fp8 K row j: the 16 rows a 16-lane group reads at one chunk
// column land on distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ constexpr int k8swz(int j) {
  return D == 128 ? (j >> 1) & 7 : (j >> 2) & 3;
}

// BIAS: an additive bias may be present (else only ALiBi slopes, with
// SCOREMOD); the instances without it keep the registers of the bias tile.
// FP8: Q, K, V are OCP E4M3 codes with per-tensor scales (folded into
// p.scale_log2 and p.v_scale); S = K Q^T runs on the fp8 matrix core, P V on
// bf16 (eight waves, no RoPE, no bias).
template <int D, int NW, bool ROPE, bool SCOREMOD, bool SPARSE, bool BIAS, bool FP8 = false>
__global__ void __launch_bounds__(NW * 64)
fwd_bf16_kernel(const AttnParams p) {
  // Two-slot rings for the shallow schedule (see fwd_bf16_shallow).
  constexpr bool SHALLOW = !FP8 && fwd_bf16_shallow(D, NW, SPARSE, BIAS);
  using L = TileLds<D, SHALLOW ? 2 : 4>;
  using L8 = Fp8Lds<D>;
  static_assert(!FP8 || (NW == 8 && !ROPE && !BIAS), "fp8 instances: eight waves, no RoPE, no bias");
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NK8 = D / 64;  // fp8 MFMA k-steps over the head dim
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int RING = L::RING;
  constexpr int LDS_RING = L::T_OFF + (ROPE ? L::TSLOT : 0);
  // The ping-pong prologue stages each wave's Q rows (32 rows of 2*D bytes)
  // in K slot 3, V slots 2 and 3 and one more area of the same size.
  constexpr int LDS_BF16 = LDS_RING + (NW == 8 ? 128 * D : 0);
  // The epilogue stages 32 rows of 2 * D + 16 bytes per wave.
  constexpr int LDS_EPI = NW * 32 * (2 * D + 16);
  constexpr int LDS_BYTES = FP8 ? (L8::BYTES > LDS_EPI ? L8::BYTES : LDS_EPI) : LDS_BF16;
  static_assert(FP8 || LDS_BYTES == fwd_bf16_lds_bytes(D, NW, ROPE, SPARSE, BIAS), "host LDS model");
  static_assert(LDS_EPI <= LDS_BF16, "the epilogue staging fits in the rings");
  // DMA instructions per wave and tile.  V is spread evenly; K pairs may not
  // be (D = 64 with 8 waves: waves 0..3 take one pair each).
  static_assert(L::NVI % NW == 0, "V instructions must spread evenly over the waves");
  static_assert(D == 64 || NW % 2 == 0, "K pair swizzle needs an even wave count for D = 128");
  constexpr int NVW = L::NVI / NW;
  constexpr int NKW_HI = (L::NKP + NW - 1) / NW;
  constexpr int NKW_LO = L::NKP / NW;
  constexpr int TPK = ROPE ? 2 : 0;  // table instructions per K pair
  constexpr bool PP = NW == 8;       // ping-pong schedule (two waves per SIMD)
  // Score mods: the first score MFMAs of a tile start from a splat of the
  // lane's offset (ALiBi at the register's base key, minus the running
  // maximum), leaving one FMA per score for the ALiBi step; the D = 128
  // eight-wave instance has no 16 registers to spare (it holds the bias tile
  // fetched ahead) and starts from 0, adding the offset per score.
  constexpr bool CSPLAT = SCOREMOD && !(D == 128 && NW == 8 && BIAS);
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, lh = lane >> 5;

  // ---- workgroup -> (b, kv-head, head group, query block) ----
  const int hp = p.hp;
  const int RB = NW / hp;
  const int rows_wg = 32 * RB;
  const int unit = blockIdx.x % p.n_units;
  const int qrank = blockIdx.x / p.n_units;
  // A paired workgroup (see AttnParams::pair) runs a second query block,
  // qrank, after qblk (-1: none).  A chained workgroup (block-sparse, two or
  // four waves, see AttnParams::chain) runs p.chain consecutive query blocks
  // of its head, from qblk on.
  constexpr bool PAIRABLE = PP && !SPARSE && !BIAS;
  constexpr bool CHAIN = SPARSE && !PP && !BIAS;
  const int qblk = p.longest_first ? (p.n_qblk - 1 - qrank) : (CHAIN ? qrank * p.chain : qrank);
  const int qblk2 = (PAIRABLE && p.pair && qrank < qblk) ? qrank : -1;
  const int n_hg = p.G / hp;
  const int hg = unit % n_hg;
  const int kvh = (unit / n_hg) % p.Hkv;
  const int b = unit / (n_hg * p.Hkv);
  const int h = kvh * p.G + hg * hp + (wave % hp);
  // Rows of the query block being processed (switched between the blocks of
  // a paired workgroup).
  int r0_wg, w0, i, iq, wg_last, w_last;
  auto set_rows = [&](int qb) {
    r0_wg = qb * rows_wg;
    w0 = r0_wg + 32 * (wave / hp);  // first row of this wave
    i = w0 + lq;                    // this lane's query row
    iq = min(i, p.Nq - 1);
    wg_last = min(r0_wg + rows_wg, p.Nq) - 1;
    w_last = min(w0 + 31, p.Nq - 1);
  };
  set_rows(qblk);

  const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + b * p.qsb + h * p.qsh;
  const __bf16* kb = reinterpret_cast<const __bf16*>(p.k) + b * p.ksb + kvh * p.ksh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;

  // ---- key tiles this workgroup visits ----
  // Dense lists: the band's key range [j_lo, j_hi] of rows r0..rlast, as
  // tiles [tb, tb + nt).
  auto dense_range = [&](int r0, int rlast, int& tb, int& nt) {
    int j_lo = 0, j_hi = p.Nk - 1;
    if (p.has_band) {
      j_lo = max(j_lo, r0 + max(p.band_lo, -kBandInf));
      j_hi = min(j_hi, (int)min((long long)rlast + p.band_hi, (long long)kBandInf));
    }
    tb = j_lo / 64;
    nt = (j_hi >= j_lo) ? (j_hi / 64 - tb + 1) : 0;
  };
  int n_tiles, t_begin = 0, s_begin = 0, tpb = 1;
  // Chained blocks: the CSR rows of consecutive query blocks are adjacent,
  // so their key lists form one stream; block c's tiles end at stream tile
  // seg_end(c).  (A workgroup's rows must be one CSR block row.)
  int n_chain = 1, qbs0 = 0;
  const int* rp = nullptr;
  long long rp_a = 0;
  if (SPARSE) {
    rp = p.row_ptr + (p.bs_head_stride ? (long long)h * p.bs_head_stride : 0);
    qbs0 = r0_wg / p.bm;
    if (CHAIN && p.bm == rows_wg) n_chain = max(1, min(p.chain, p.n_qblk - qblk));
    const long long nnz = p.bs_nnz;
    const long long a = min(max((long long)rp[qbs0], 0LL), nnz);
    const long long e = min(max((long long)rp[qbs0 + n_chain], a), nnz);
    s_begin = (int)a;
    rp_a = a;
    tpb = p.bn / 64;
    n_tiles = (int)(e - a) * tpb;
  } else {
    dense_range(r0_wg, wg_last, t_begin, n_tiles);
  }
  // Paired: the second block's tiles follow the first block's in one stream;
  // stream tile u >= seg_split is tile u - seg_split of the second block,
  // whose key tiles start at t_begin2.
  int seg_split = 1 << 30, n_first = n_tiles, n_second = 0, t_begin2 = 0;
  if (qblk2 >= 0) {
    dense_range(qblk2 * rows_wg, min((qblk2 + 1) * rows_wg, p.Nq) - 1, t_begin2, n_second);
    seg_split = n_tiles;
    n_tiles += n_second;
  }
  // Column indices are clamped into [0, nkb]; column nkb (or anything past
  // the keys) lands at k0 >= Nk, is loaded clamped and masked out entirely.
  // The list is read with scalar loads, which do not count against vmcnt.
  const int nkb = SPARSE ? (p.Nk + p.bn - 1) / p.bn : 0;
  // With ALiBi slopes (positive: the bias grows towards the diagonal) a dense
  // key list is visited from its last tile to its first, so the running
  // maximum is set by the first tile and later tiles rarely move it (visited
  // the other way, the maximum climbs by up to slope * 64 * log2(e) per tile
  // and almost every tile takes the exact rescaling path).  The softmax does
  // not depend on the order; masks and positions follow the tile's keys.
  const bool rev = !SPARSE && SCOREMOD && p.alibi != nullptr;
  typedef __attribute__((address_space(4))) const int* cidx_t;
  auto tile_k0 = [&](int t) -> int {
    if (SPARSE) {
      const int col = min(max(((cidx_t)p.col_idx)[s_begin + t / tpb], 0), nkb);
      return col * p.bn + (t % tpb) * 64;
    }
    const bool s2 = t >= seg_split;  // (rev: each block's tiles from its last key tile down)
    const int loc = s2 ? t - seg_split : t;
    return ((s2 ? t_begin2 : t_begin) + (rev ? (s2 ? n_second : n_first) - 1 - loc : loc)) * 64;
  };

  // End of chained block c's tiles in the stream, kept within [lo, n_tiles]
  // (a malformed row_ptr gives wrong numbers, never a bad access).
  auto seg_end = [&](int c, int lo) -> int {
    const long long e = min(max((long long)rp[qbs0 + c + 1], rp_a), p.bs_nnz);
    return min(max((int)(e - rp_a) * tpb, lo), n_tiles);
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

  const float* const rcos = p.rcos;
  const float* const rsin = p.rsin;
  const int rope_last = p.rope_len - 1, k_pos0 = p.k_pos0;
  // Byte offset of this lane's first table word inside its row.
  const uint32_t tcol = 32u * (uint32_t)kc;
  const long long ksn = p.ksn, vsn = p.vsn;
  // Per-lane byte offsets inside a tile (row strides are below 2^24
  // elements, so 64 rows fit in 32 bits): K low chunk of row r at
  // r * ksn2 + kcol, V chunk of row r at r * vsn2 + vcol(m).
  const uint32_t ksn2 = (uint32_t)(2 * ksn), vsn2 = (uint32_t)(2 * vsn);
  const uint32_t kcol = 16u * (uint32_t)kc;
  // First key of tile u, clamped into the key range.  Tiles past the list
  // reload the last tile, so every wave issues the same number of DMA
  // instructions per iteration (their slots are never read as data).
  auto tile_base = [&](int u, int& k0, int& rmax) {
    k0 = tile_k0(min(u, n_tiles - 1));
    const int kc0 = min(k0, Nk - 1);
    rmax = Nk - 1 - kc0;
    return kc0;
  };
  // Iteration t issues the group {K(t+4); table entries of K(t+3), V(t+3)},
  // one instruction at a time between its MFMAs (a burst would stall on the
  // memory pipe): K in the first phase, the rest in the second, after the
  // rotation of that iteration has read the table slot.  At the top of
  // iteration t only the V part of the group of t-1 may still be in flight
  // (vmcnt retires in issue order): that retires the group of t-2, i.e.
  // K(t+2) (rotated this iteration) and V(t+1) (read next iteration), and
  // the table entries of K(t+2).  Without RoPE the whole group of t-1 may be
  // in flight.
  const int grp = (2 + TPK) * nkw + NVW;  // instructions per group (this wave)
  auto wait_group = [&]() {
    if constexpr (ROPE) {
      vmcnt_wait<NVW>();
    } else if constexpr (NKW_HI == NKW_LO) {
      vmcnt_wait<2 * NKW_HI + NVW>();
    } else {
      if (nkw == NKW_HI) vmcnt_wait<2 * NKW_HI + NVW>();
      else vmcnt_wait<2 * NKW_LO + NVW>();
    }
  };
  // Scalar bases of one iteration's group.
  struct Group {
    int k0t;                 // first key of the tile whose table entries are fetched
    const __bf16* kt;        // K tile base (clamped)
    const __bf16* vt;        // V tile base (clamped)
    int rmax_k, rmax_v;      // last valid row offsets
    uint32_t kslot, vslot;
  };
  auto make_group = [&](int uk, int ut, int uv) -> Group {
    Group g;
    int k0k, k0v, rk, rt, rv;
    const int kck = tile_base(uk, k0k, rk);
    const int kcv = tile_base(uv, k0v, rv);
    tile_base(ut, g.k0t, rt);
    g.kt = kb + (long long)kck * ksn;
    g.vt = vb + (long long)kcv * vsn;
    g.rmax_k = rk;
    g.rmax_v = rv;
    g.kslot = lds0 + (uint32_t)(uk % RING) * L::KSLOT;
    g.vslot = lds0 + L::V_OFF + (uint32_t)(uv % RING) * L::VSLOT;
    return g;
  };
  // Per-lane DMA offsets of unclamped rows, fixed for the whole loop; a row
  // clamp min(row, rmax) * stride + col becomes min(offset, rmax * stride + col).
  uint32_t koff[NKW_HI], vdoff[NVW], vc16[NVW];
#pragma unroll
  for (int m = 0; m < NKW_HI; ++m) koff[m] = (uint32_t)(L::KROWS_I * (wave + NW * m) + kjr) * ksn2 + kcol;
#pragma unroll
  for (int j = 0; j < NVW; ++j) {
    const int key = L::VROWS_I * (wave + NW * j) + vrow;
    vc16[j] = 16u * (uint32_t)((lane % L::CPR) ^ vswz<D>(key));
    vdoff[j] = (uint32_t)key * vsn2 + vc16[j];
  }
  const uint32_t toff = (uint32_t)kjr * (uint32_t)L::ROWB + tcol;
  // Instruction i of a group, in issue order: K low / high per pair, then
  // (RoPE) two table instructions per pair, then V.
  const uint32_t tslot = lds0 + L::T_OFF;
  auto dma_item = [&](const Group& g, int i) {
    if (i < 2 * nkw) {
      const int m = i / 2, hi = i % 2;
      const int kp = wave + NW * m;
      // min(row, rmax) * ksn2 + kcol, with the row part precomputed (rows
      // are below 64, so the clamp bound is taken at most 63 rows: no
      // 32-bit overflow).
      const uint32_t off = min(koff[m], (uint32_t)min(g.rmax_k, 63) * ksn2 + kcol);
      dma16_off(g.kslot + (hi ? L::KHI : 0) + kp * 1024, hi ? g.kt + D / 2 : g.kt, off);
    } else if (i < (2 + TPK) * nkw) {
      const int m = (i - 2 * nkw) / 2, x = (i - 2 * nkw) % 2;
      const int kp = wave + NW * m;
      // The pair covers KROWS_I keys from position prow; rows past the
      // table only belong to masked keys and re-read its last row.
      const int prow = k_pos0 + g.k0t + L::KROWS_I * kp;
      const int row0 = min(prow, rope_last);
      const uint32_t off = min(toff, (uint32_t)min(rope_last - row0, 63) * (uint32_t)L::ROWB + tcol);
      dma16_off(tslot + (uint32_t)kp * L::TPAIR + 1024u * x, p.rcs + (long long)row0 * (D / 2),
                off + 16u * x);
    } else {
      const int j = i - (2 + TPK) * nkw;
      const int vi = wave + NW * j;
      const uint32_t off = min(vdoff[j], (uint32_t)min(g.rmax_v, 63) * vsn2 + vc16[j]);
      dma16_off(g.vslot + vi * 1024, g.vt, off);
    }
  };
  // A whole group at once (prologue); with_v = false issues the K part only,
  // with_t = false skips the table part.
  constexpr int GRP_MAX = (2 + TPK) * NKW_HI + NVW;
  auto issue_group = [&](int uk, int ut, int uv, bool with_t, bool with_v) __attribute__((always_inline)) {
    const Group g = make_group(uk, ut, uv);
#pragma unroll
    for (int i = 0; i < GRP_MAX; ++i) {
      const bool is_t = i >= 2 * nkw && i < (2 + TPK) * nkw;
      const bool is_v = i >= (2 + TPK) * nkw;
      if (i < grp && (with_t || !is_t) && (with_v || !is_v)) dma_item(g, i);
    }
  };

  // ---- RoPE of K in place: prologue tiles ----
  // Tiles 0 and 1 are rotated before the loop with table words read straight
  // from global memory, fetched together with the first tiles and Q (one
  // memory round trip); the loop rotates later tiles from the table slot.
  uint4 ptab[2][NKW_HI][2];
  auto fetch_direct = [&](int u) {
    const int k0u = tile_k0(min(u, n_tiles - 1));
#pragma unroll
    for (int m = 0; m < NKW_HI; ++m) {
      if (m < nkw) {
        const int kp = wave + NW * m;
        const int row = min(k_pos0 + k0u + L::KROWS_I * kp + kjr, rope_last);
        const uint32_t* tr = p.rcs + (long long)row * (D / 2) + 8 * kc;
        ptab[u][m][0] = ld16(tr);
        ptab[u][m][1] = ld16(tr + 4);
      }
    }
  };
  auto rotate_direct = [&](int u) {
    char* slot = smem + (u % RING) * L::KSLOT;
#pragma unroll
    for (int m = 0; m < NKW_HI; ++m) {
      const int kp = wave + NW * m;
      if (m < nkw) {
        const uint4 t0 = ptab[u][m][0], t1 = ptab[u][m][1];
        char* lo_p = slot + kp * 1024 + lane * 16;
        char* hi_p = lo_p + L::KHI;
        uint4 lo = ld16(lo_p), hi = ld16(hi_p);
        rope_rotate_bf16x8_t(lo, hi, t0, t1);
        st16(lo_p, lo);
        st16(hi_p, hi);
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
  // Lane part of the K fragment address for chunk column c = kk % (NKK/2).
  uint32_t klane[NKK / 2];
#pragma unroll
  for (int c = 0; c < NKK / 2; ++c) klane[c] = (uint32_t)(lq * D + 16 * ((2 * c + lh) ^ ksw));
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
  // The softmax scale (times log2 e, for exp2) is applied here, in fp32,
  // before the single bf16 rounding of the rotated row, so the score MFMAs
  // produce exp2-domain scores directly.
  // Issued in two parts so that the loads share the prologue's single wait
  // with the first tiles: load_q_issue() fetches the row chunks and their
  // angles (packed fp16 (cos, sin) words: their 2^-12 rounding is far below
  // the bf16 rounding of the rotated row, at half the bytes of fp32 cos and
  // sin), load_q_finish() rotates and scales them in fp32.
  bf16x8 qf[NKK];
  uint4 qlo[NKK / 2], qhi[NKK / 2];
  uint4 qa[ROPE ? NKK / 2 : 1], qb2[ROPE ? NKK / 2 : 1];
  auto load_q_issue = [&]() {
    const __bf16* qrow = qb + (long long)iq * p.qsn;
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      const int d0 = 16 * kk + 8 * lh;
      qlo[kk] = ld16(qrow + d0);
      qhi[kk] = ld16(qrow + d0 + D / 2);
      if (ROPE) {
        const uint32_t* row = p.rcs + (long long)(p.q_pos0 + iq) * (D / 2) + d0;
        qa[kk] = ld16(row);
        qb2[kk] = ld16(row + 4);
      }
    }
  };
  auto load_q_finish = [&]() {
    const float qscale = p.scale_log2;
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      uint4 lo = qlo[kk], hi = qhi[kk];
      if (ROPE) {
        rope_rotate_bf16x8_h(lo, hi, qa[kk], qb2[kk], qscale);
      } else {
        lo = scale_bf16x8(lo, qscale);
        hi = scale_bf16x8(hi, qscale);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, lo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, hi);
    }
  };

  // Ping-pong prologue: the wave's 32 Q rows reach a private LDS area by
  // direct loads in which 16 (D = 128) or 8 lanes cover one whole row, then
  // come back in fragment layout (chunks XOR-swizzled by row against bank
  // conflicts); the angles are loaded as before.
  constexpr int QCPR = D / 8;        // 16-byte chunks per row
  constexpr int QRPI = 64 / QCPR;    // rows per load instruction
  constexpr int QAREA = 64 * D;      // bytes per wave (32 rows)
  const uint32_t qarea = [&]() -> uint32_t {
    const int a = wave / 2;
    const uint32_t base = a == 0 ? 3u * L::KSLOT
                        : a == 1 ? (uint32_t)(L::V_OFF + 2 * L::VSLOT)
                        : a == 2 ? (uint32_t)(L::V_OFF + 3 * L::VSLOT)
                                 : (uint32_t)LDS_RING;
    return lds0 + base + (uint32_t)(wave % 2) * QAREA;
  }();
  auto load_q_issue_staged = [&]() {
    const int wq = min(w0, p.Nq - 1);  // first row of this wave, clamped
    const __bf16* qw = qb + (long long)wq * p.qsn;
#pragma unroll
    for (int m = 0; m < 32 / QRPI; ++m) {
      const int r = QRPI * m + lane / QCPR;
      const int c = (lane % QCPR) ^ (r % QCPR);
      const int rg = min(w0 + r, p.Nq - 1) - wq;
      dma16_off(qarea + 1024u * m, qw, (uint32_t)(rg * p.qsn + 8 * c) * 2u);
    }
    // The angle rows (D/2 words = 2*D bytes each) are read the same whole-
    // row way, into registers; q_rows_from_lds() reshapes them through the
    // same area once the Q rows have left it.
    if (ROPE) {
#pragma unroll
      for (int m = 0; m < 32 / QRPI; ++m) {
        const int r = QRPI * m + lane / QCPR;
        const uint32_t* row = p.rcs + (long long)(p.q_pos0 + min(w0 + r, p.Nq - 1)) * (D / 2);
        const uint4 v = ld16(row + 4 * (lane % QCPR));
        if (m % 2 == 0) qa[m / 2] = v;
        else qb2[m / 2] = v;
      }
    }
  };
  auto q_rows_from_lds = [&]() {
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      const int c = 2 * kk + lh;
      qlo[kk] = __builtin_bit_cast(uint4, lds_read16(qarea + lq * 2 * D + 16 * (c ^ (lq % QCPR))));
      qhi[kk] = __builtin_bit_cast(uint4, lds_read16(qarea + lq * 2 * D + 16 * ((c + QCPR / 2) ^ (lq % QCPR))));
    }
    if (ROPE) {
      char* const qs = smem + (qarea - lds0);
#pragma unroll
      for (int m = 0; m < 32 / QRPI; ++m) {
        const int r = QRPI * m + lane / QCPR;
        st16(qs + r * 2 * D + 16 * ((lane % QCPR) ^ (r % QCPR)), m % 2 == 0 ? qa[m / 2] : qb2[m / 2]);
      }
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk) {
        const int c = 4 * kk + 2 * lh;
        qa[kk] = ld16(qs + lq * 2 * D + 16 * (c ^ (lq % QCPR)));
        qb2[kk] = ld16(qs + lq * 2 * D + 16 * ((c + 1) ^ (lq % QCPR)));
      }
    }
  };

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  // Row sums: ol = ones . P^T, so every register of a lane holds the sum of
  // its query column.
  f32x16 ol = f32x16{};
  const bf16x8 ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                        (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  float m_run = -INFINITY;  // running max, exp2 domain
  float slope2 = 0.f;  // ALiBi slope times log2(e), loaded in the prologue
  const int dpos = p.k_pos0 - p.q_pos0;
  const float* const brow =
      (SCOREMOD && BIAS && p.bias) ? p.bias + b * p.bsb + h * p.bsh + (long long)iq * p.bsi : nullptr;
  const long long bsj = p.bsj;
  // Bias fetched a tile ahead (two-wave-per-SIMD schedule, unit key stride,
  // Nk a multiple of 4, 16-byte aligned rows): lane (lq, lh) needs, for
  // g = 0..7, the four keys k0 + 8g + 4lh .. + 3 of its query row (S^T
  // subtile g / 4, registers 4 (g % 4) .. + 3), one 16-byte load each.  Runs
  // past the keys are clamped in bounds; those scores are masked.
  const bool bias_vec = PP && SCOREMOD && brow && bsj == 1 && Nk >= 4 && (Nk & 3) == 0 &&
                        __builtin_amdgcn_ballot_w64((reinterpret_cast<uintptr_t>(brow) & 15) != 0) == 0;
  float4 bias4[8];
  auto bias_fetch = [&](int k0) {
    if (!bias_vec) return;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      bias4[g] = *reinterpret_cast<const float4*>(brow + min(k0 + 8 * g + 4 * lh, Nk - 4));
  };

  // Dense key lists: the block's tile in key order u starts at key
  // 64 * (tb + u), so the tiles that need no mask (inside the key range and,
  // with a band, wholly inside it for every row of this wave) form one
  // interval [mlo, mhi], computed once per block instead of per tile.
  int mlo = 0, mhi = -1;
  // (n_seg, tb: tiles and first key tile of the query block being processed.)
  auto set_masks = [&](int n_seg, int tb) {
    mlo = 0;
    mhi = -1;
    if (!SPARSE) {
      auto fdiv = [](long long a) -> long long { return a >= 0 ? a / 64 : -((-a + 63) / 64); };
      long long lo = 0, hi = min((long long)n_seg - 1, fdiv((long long)Nk - 64) - tb);
      if (has_band) {
        lo = max(lo, -fdiv(-((long long)band_lo + w_last)) - tb);          // k0 - w_last >= band_lo
        hi = min(hi, fdiv((long long)band_hi + w0 - 63) - tb);             // k0 + 63 - w0 <= band_hi
      }
      if (lo <= hi) {
        mlo = (int)lo;
        mhi = (int)hi;
      }
    }
  };
  set_masks(n_first, t_begin);
  // Masks of S^T tile u in place (only where the tile needs them: the key
  // tail, or the band edge crossing this wave's rows).  A tile past the list
  // (the last iteration's look-ahead) is masked out entirely.
  auto mask_scores = [&](int u, f32x16 (&s)[2]) {
    const bool beyond = u >= n_tiles;
    bool need_mask;
    if (SPARSE) {
      const int k0 = tile_k0(min(u, n_tiles - 1));
      need_mask = beyond || k0 + 64 > Nk;
      if (has_band) {
        const int dmin = k0 - w_last, dmax = k0 + 63 - w0;
        need_mask |= (dmin < band_lo) | (dmax > band_hi);
      }
    } else {
      // tile's place in its block's key order (< 0 past the list)
      const bool s2 = u >= seg_split;
      const int loc = s2 ? u - seg_split : u;
      const int pu = rev ? (s2 ? n_second : n_first) - 1 - loc : loc;
      need_mask = (pu < mlo) | (pu > mhi);
    }
    if (need_mask) {
      const int k0 = tile_k0(min(u, n_tiles - 1));
      // Allowed register offsets form one interval [lo_off, hi_off].
      const int jd = (k0 - w0) + (4 * lh - lq);  // j - i at register offset 0 (i = w0 + lq)
      int lo_off = -kBandInf, hi_off = Nk - 1 - (k0 + 4 * lh);
      if (has_band) {
        lo_off = band_lo - jd;
        hi_off = min(hi_off, band_hi - jd);
      }
      if (beyond) hi_off = lo_off - 1;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kOff(st, r);
          s[st][r] = ((off >= lo_off) & (off <= hi_off)) ? s[st][r] : -INFINITY;
        }
    }
  };

  // ---- online softmax ("2 Background / FlashAttention and online softmax") ----
  // A tile is exponentiated against the running maximum it arrives with:
  // p = 2^(score - m_run).  Only when some exponent exceeds 15 (or is NaN),
  // and for the first tile with live keys, the exact path takes the tile
  // maximum, rescales O and the row sums, and exponentiates again.  Every p
  // is then at most 2^15 and the result is the same exact softmax.
  constexpr float kTrig = 15.f;  // largest exp2 argument taken without the exact path
  auto neg_m = [&]() -> float { return (m_run == -INFINITY) ? 0.f : -m_run; };
  // Per-lane, per-tile part of the exp2 argument: score mods' lane offset.
  // With score mods minus the running maximum joins this offset (the MFMAs
  // start from it, or from 0 in the instance without the registers).
  auto mod_base = [&](int k0) -> float {
    return SCOREMOD ? __builtin_fmaf(slope2, (float)(k0 + 4 * lh - i + dpos), neg_m()) : 0.f;
  };
  // The first score MFMA of every tile takes its C operand from minit, a
  // splat of minus the running maximum (updated only when the maximum
  // moves), so the MFMAs leave the exp2 argument itself: the scale is folded
  // into Q and no per-tile initialisation is needed.
  f32x16 minit = f32x16{};
  // exp2 argument of register r of subtile st: the accumulator plus, with
  // score mods, the lane's offset, the register's ALiBi step and the bias.
  auto arg = [&](const f32x16 (&s)[2], int st, int r, int k0) -> float {
    float x = s[st][r];
    if constexpr (FP8) {
      // The fp8 products are unscaled code dot products: one FMA applies the
      // folded scales (and joins the ALiBi step and minus the running maximum).
      const float base = SCOREMOD ? __builtin_fmaf(slope2, (float)kOff(st, r), mod_base(k0)) : neg_m();
      return __builtin_fmaf(p.scale_log2, x, base);
    }
    if (SCOREMOD) {
      if (CSPLAT) x = __builtin_fmaf(slope2, (float)kOff(st, r), x);
      else x += __builtin_fmaf(slope2, (float)kOff(st, r), mod_base(k0));
      if (brow) {
        float bv;
        if (bias_vec) {
          const float4 b4 = bias4[4 * st + r / 4];
          bv = (r % 4 == 0) ? b4.x : (r % 4 == 1) ? b4.y : (r % 4 == 2) ? b4.z : b4.w;
        } else {
          const int j = min(k0 + 4 * lh + kOff(st, r), Nk - 1);
          bv = brow[(long long)j * bsj];
        }
        x = __builtin_fmaf(bv, kLog2e, x);
      }
    }
    return x;
  };
  // P pair x: registers r, r+1 of subtile st -> word q of P^T fragment c.
  // The exp2 arguments are left in s for the overflow check and the exact
  // path.
  auto exp_pair = [&](f32x16 (&s)[2], int x, int k0) -> uint32_t {
    const int c = x / 4, q = x % 4, st = c / 2, r = 8 * (c % 2) + 2 * q;
    s[st][r] = arg(s, st, r, k0);
    s[st][r + 1] = arg(s, st, r + 1, k0);
    return pack_bf16x2(fast_exp2(s[st][r]), fast_exp2(s[st][r + 1]));
  };
  // The same work in three stages, so that a pipelined loop can give each
  // step independent instructions: (1) the exp2 arguments, left in s;
  // (2) the two exponentials; (3) pack to bf16.
  auto exp_stage1 = [&](f32x16 (&s)[2], int x, int k0) {
    if (!SCOREMOD) return;
    const int c = x / 4, q = x % 4, st = c / 2, r = 8 * (c % 2) + 2 * q;
    (void)q;
    s[st][r] = arg(s, st, r, k0);
    s[st][r + 1] = arg(s, st, r + 1, k0);
  };
  auto exp_stage2 = [&](const f32x16 (&s)[2], int x, float (&e)[2]) {
    const int c = x / 4, q = x % 4, st = c / 2, r = 8 * (c % 2) + 2 * q;
    (void)q;
    e[0] = fast_exp2(s[st][r]);
    e[1] = fast_exp2(s[st][r + 1]);
  };
  auto exp_stage3 = [&](int x, const float (&e)[2]) -> uint32_t {
    const uint32_t w = pack_bf16x2(e[0], e[1]);
    asm volatile("" ::"v"(w));  // anchor it to this step (no sinking towards its use)
    return w;
  };
  // Check the tile's exponents; on the rare exact path re-exponentiate
  // against the tile maximum (O^T and the row sums must already hold every
  // earlier tile's product).  s holds the exp2 arguments relative to m_use.
  // While no key has been seen (m_run = -inf) every tile takes the exact
  // path, which then establishes the maximum.
  auto finish_tile = [&](f32x16 (&s)[2], float m_use, uint32_t (&pw)[16]) {
    const bool trig = tree_max32_bits(s[0], s[1]) > __float_as_int(kTrig) || m_run == -INFINITY;
    if (__builtin_amdgcn_ballot_w64(trig)) {
      const float mx_l = tree_max32(s[0], s[1]);
      const float mx = fmaxf(mx_l, partner32(mx_l)) + m_use;
      const float m_new = fmaxf(m_run, mx);
      float shift = 0.f;
      if (m_new != -INFINITY) {
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        minit = f32x16{} - m_new;
        shift = m_use - m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) ol[r] *= alpha;
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int c = x / 4, q = x % 4, st = c / 2, r = 8 * (c % 2) + 2 * q;
        pw[x] = pack_bf16x2(fast_exp2(s[st][r] + shift), fast_exp2(s[st][r + 1] + shift));
      }
    }
  };
  auto to_frags = [](const uint32_t (&pw)[16], bf16x8 (&pf)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pf[c] = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));
  };

  const int n = n_tiles;
  bf16x8 pfa[4], pfb[4];  // P^T of the tile the next iteration multiplies with V (ping-pong)
  // S(0) -> P(0) in the prologue, shared by both schedules.
  // S(u0) -> P(u0) into pf (u0 = 0, or the first tile of a paired
  // workgroup's second block), K'(u0) read from its ring slot.
  auto first_tile_at = [&](int u0, bf16x8 (&pf)[4]) {
    const int k00 = tile_k0(u0);
    const uint32_t ks0 = lds0 + (uint32_t)(u0 % RING) * L::KSLOT;
    auto kf0 = [&](int st, int kk) -> bf16x8 {  // k_frag, addressed through klane
      return lds_read16(ks0 + klane[kk % (NKK / 2)] + (kk / (NKK / 2)) * L::KHI + 32 * st * D);
    };
    f32x16 s0[2];
#pragma unroll
    for (int k = 0; k < 2 * NKK; ++k)
      s0[k & 1] = mfma32(kf0(k & 1, k >> 1), qf[k >> 1], k < 2 ? (SCOREMOD ? (CSPLAT ? f32x16{} + mod_base(k00) : f32x16{}) : minit) : s0[k & 1]);
    mask_scores(u0, s0);
    uint32_t pw[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) pw[x] = exp_pair(s0, x, k00);
    finish_tile(s0, -neg_m(), pw);
    to_frags(pw, pf);
  };
  auto first_tile = [&]() { first_tile_at(0, pfa); };
  // Paired and chained workgroups, at the switch between two blocks: the
  // finished block's output, O^T / l straight from registers in 8-byte
  // pieces, and its lse ...
  auto store_block_regs = [&]() {
    const int i_a = i;
    const float l_a = ol[0], m_a = m_run;
    const float inv = l_a > 0.f ? p.v_scale / l_a : 0.f;
    __bf16* const orow = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh + (long long)i_a * p.osn;
    if (i_a < p.Nq) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 w;
          w.x = pack_bf16x2(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv);
          w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * g + 4 * lh) = w;
        }
    }
    if (i_a < p.Nq && p.lse && lh == 0)
      p.lse[((long long)b * p.Hq + h) * p.Nq + i_a] =
          l_a > 0.f ? (m_a + __builtin_log2f(l_a)) * kLn2 : -INFINITY;
  };
  // ... and a fresh softmax state for the next block.
  auto reset_softmax = [&]() {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    ol = f32x16{};
    m_run = -INFINITY;
    minit = f32x16{};
  };
  // A paired workgroup's switch: then the second block's rows (its Q loads
  // can be issued after this) and masks.
  auto finish_first_block = [&]() {
    store_block_regs();
    set_rows(qblk2);
  };
  auto start_second_block = [&]() {
    reset_softmax();
    set_masks(n_second, t_begin2);
  };
  // A paired workgroup runs two query blocks over one stream of key tiles.
  // The first block's last step computes S(seg_split) with its own Q, so
  // that tile's softmax waits for the second block's Q.
  const bool paired = PAIRABLE && qblk2 >= 0 && n_first > 0 && n_second > 0;
  // Steps T0 .. T1-1 of a ping-pong schedule with step function STEP (P(t)
  // sits in pfa for even t - T0); the last step takes the softmax of S(T1)
  // only if LAST.  (A macro: every use is a separate copy of the loop, so
  // none keeps another's state live.)
#define ATTNFUSE_RUN_STEPS(STEP, T0, T1, LAST)                    \
  {                                                               \
    int t_ = (T0);                                                \
    const int t1_ = (T1);                                         \
    const bool last_ = (LAST);                                    \
    for (; t_ + 1 < t1_; t_ += 2) {                               \
      STEP(t_, pfa, pfb, true);                                   \
      STEP(t_ + 1, pfb, pfa, last_ || t_ + 2 < t1_);              \
    }                                                             \
    if (t_ < t1_) STEP(t_, pfa, pfb, last_);                      \
  }
  if constexpr (FP8) {
    // ---- fp8 ping-pong schedule ----
    // The two-waves-per-SIMD alternation of the bf16 schedule below, with
    // S(t+1) = K(t+1) Q^T on the fp8 matrix core (Q codes in registers, K
    // codes in LDS) and P V on bf16.  Vector cluster of step t: DMA of K(t+3)
    // and of V(t+2) into the staging ring, conversion of the thread's own codes
    // of V(t+1) (landed by the wait that opens the cluster) into bf16 V slot
    // (t+1) % 4, softmax of S(t+1).  The waves with a DMA role issue one K and
    // one V instruction per tile (D = 128: all eight; D = 64: waves 0-3).
    const bool m_first = wave < NW / 2;
    const bool dma_wave = wave < L8::NI;
    const uint8_t* const kb8 = reinterpret_cast<const uint8_t*>(p.k) + b * p.ksb + kvh * p.ksh;
    const uint8_t* const vb8 = reinterpret_cast<const uint8_t*>(p.v) + b * p.vsb + kvh * p.vsh;
    // Instruction `wave` of a tile covers rows ROWS_I * wave ..; lane: row
    // row8, 16-byte chunk position pos8 (K: global chunk pos8 ^ k8swz(row8)).
    const int row8 = L8::ROWS_I * wave + lane / L8::CPR;
    const int pos8 = lane % L8::CPR;
    const uint32_t kcol8 = 16u * (uint32_t)(pos8 ^ k8swz<D>(row8));
    const uint32_t vcol8 = 16u * (uint32_t)pos8;
    const uint32_t ksnb = (uint32_t)ksn, vsnb = (uint32_t)vsn;  // row strides in bytes (< 2^24)
    auto dma_k8 = [&](int u) {
      int k0, rmax;
      const int kc0 = tile_base(u, k0, rmax);
      const uint32_t off = (uint32_t)min(row8, min(rmax, 63)) * ksnb + kcol8;
      dma16_off(lds0 + (uint32_t)(u % RING) * L8::KSLOT + 1024u * (uint32_t)wave, kb8 + (long long)kc0 * ksn,
                off);
    };
    auto dma_v8 = [&](int u) {
      int k0, rmax;
      const int kc0 = tile_base(u, k0, rmax);
      const uint32_t off = (uint32_t)min(row8, min(rmax, 63)) * vsnb + vcol8;
      dma16_off(lds0 + L8::S_OFF + (uint32_t)(u % 2) * L8::SSLOT + 1024u * (uint32_t)wave,
                vb8 + (long long)kc0 * vsn, off);
    };
    // This thread's 16 codes of V tile u (row row8, columns 16 * pos8 ..) ->
    // two bf16 chunks of V slot u % 4 at their swizzled places.
    auto convert_v8 = [&](int u) {
      const uint4 c = ld16(smem + L8::S_OFF + (u % 2) * L8::SSLOT + 1024 * wave + 16 * lane);
      char* const dst = smem + L8::V_OFF + (u % RING) * L8::VSLOT + row8 * 2 * D;
      st16(dst + 16 * ((2 * pos8) ^ vswz<D>(row8)), e4m3x8_to_bf16x8(make_uint2(c.x, c.y)));
      st16(dst + 16 * ((2 * pos8 + 1) ^ vswz<D>(row8)), e4m3x8_to_bf16x8(make_uint2(c.z, c.w)));
    };
    // Q codes as B operands: lane (lq, lh) holds bytes 64 kk + 32 lh .. + 31
    // of its query row (K fragments split k the same way).
    i32x8 qf8[NK8];
    auto load_q8 = [&]() {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + b * p.qsb + h * p.qsh + (long long)iq * p.qsn;
#pragma unroll
      for (int kk = 0; kk < NK8; ++kk) {
        const uint4 a = ld16(qrow + 64 * kk + 32 * lh), c = ld16(qrow + 64 * kk + 32 * lh + 16);
        qf8[kk] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
      }
    };
    // K fragment (A operand): row 32 st + lq, bytes 64 kk + 32 lh .. + 31.
    const int k8s = k8swz<D>(lq);  // = k8swz(32 st + lq) for both subtiles
    auto kf8 = [&](uint32_t ks, int st, int kk) -> i32x8 {
      const uint32_t rowb = ks + (uint32_t)(32 * st + lq) * D;
      const uint4 a = __builtin_bit_cast(uint4, lds_read16(rowb + 16 * ((4 * kk + 2 * lh) ^ k8s)));
      const uint4 c = __builtin_bit_cast(uint4, lds_read16(rowb + 16 * ((4 * kk + 2 * lh + 1) ^ k8s)));
      return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
    };
    constexpr int NS8 = 2 * NK8;     // fp8 S MFMAs per tile: (subtile, k step)
    constexpr int NPV = 4 * NDT;     // P V MFMAs per tile
    constexpr int EVERY = NPV / NS8;
    static_assert(NPV % NS8 == 0, "S MFMAs spread evenly over the P V steps");
    if (n > 0) {
      if (dma_wave) {
        dma_k8(0);
        dma_v8(0);
        if (n > 1) {
          dma_k8(1);
          dma_v8(1);
        }
        if (n > 2) dma_k8(2);
      }
    }
    load_q8();
    if (SCOREMOD && p.alibi) slope2 = p.alibi[h] * kLog2e;
    vmcnt_wait<0>();
    if (n > 0 && dma_wave) {
      convert_v8(0);
      if (n > 1) convert_v8(1);
    }
    __syncthreads();
    // S(u0) -> P(u0) into pf from K(u0)'s ring slot (u0 = 0, or the first
    // tile of a paired workgroup's second block).
    auto first_tile8_at = [&](int u0, bf16x8 (&pf)[4]) {
      const int k00 = tile_k0(u0);
      const uint32_t ks0 = lds0 + (uint32_t)(u0 % RING) * L8::KSLOT;
      f32x16 s0[2];
#pragma unroll
      for (int j = 0; j < NS8; ++j)
        s0[j & 1] = mfma32_f8(kf8(ks0, j & 1, j >> 1), qf8[j >> 1], j < 2 ? f32x16{} : s0[j & 1]);
      mask_scores(u0, s0);
      uint32_t pw[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) pw[x] = exp_pair(s0, x, k00);
      finish_tile(s0, -neg_m(), pw);
      to_frags(pw, pf);
    };
    if (n > 0) first_tile8_at(0, pfa);
    constexpr int PF = 2;
    f32x16 sn[2];
    auto mcluster8 = [&](int t, const bf16x8 (&pf)[4]) {
      __builtin_amdgcn_s_setprio(1);
      const uint32_t ks = lds0 + (uint32_t)((t + 1) % RING) * L8::KSLOT;
      const uint32_t vs = lds0 + L8::V_OFF + (uint32_t)(t % RING) * L8::VSLOT;
      uint32_t vbase[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vbase[dt] = vs + voff[dt];
      auto vf = [&](int c, int dt) -> bf16x8 {
        const i16x4 r0 = lds_read_tr4(vbase[dt] + c * 32 * D);
        const i16x4 r1 = lds_read_tr4(vbase[dt] + c * 32 * D + 16 * D);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        return __builtin_bit_cast(bf16x8, a);
      };
      bf16x8 vfr[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) vfr[k] = vf(k / NDT, k % NDT);
      i32x8 a8 = kf8(ks, 0, 0);
#pragma unroll
      for (int k = 0; k < NPV; ++k) {
        if (k + PF < NPV) vfr[(k + PF) % (PF + 1)] = vf((k + PF) / NDT, (k + PF) % NDT);
        if (k % EVERY == 0) {
          const int j = k / EVERY;
          sn[j & 1] = mfma32_f8(a8, qf8[j >> 1], j < 2 ? f32x16{} : sn[j & 1]);
          if (j + 1 < NS8) a8 = kf8(ks, (j + 1) & 1, (j + 1) >> 1);
        }
        o[k % NDT] = mfma32(vfr[k % (PF + 1)], pf[k / NDT], o[k % NDT]);
        if (k % NDT == NDT - 1) ol = mfma32(ones8, pf[k / NDT], ol);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    auto vcluster8 = [&](int t, int st, bool has_s, bf16x8 (&pf_next)[4]) {
      vmcnt_wait<0>();
      if (dma_wave) {
        if (t + 3 < n) dma_k8(t + 3);
        if (t + 2 < n) dma_v8(t + 2);
        if (t >= 1 && t + 1 < n) convert_v8(t + 1);
      }
      if (has_s) {
        const int k0s = tile_k0(min(st, n - 1));
        mask_scores(st, sn);
        uint32_t pw[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) pw[x] = exp_pair(sn, x, k0s);
        finish_tile(sn, -neg_m(), pw);
        to_frags(pw, pf_next);
      }
    };
    const int dstep = m_first ? 0 : 1;
    if (n > 0 && !m_first) {
      vcluster8(0, 0, false, pfb);
      __syncthreads();
    }
    auto step8 = [&](int t, const bf16x8 (&pf_cur)[4], bf16x8 (&pf_nxt)[4], bool has_s)
        __attribute__((always_inline)) {
      mcluster8(t, pf_cur);
      __syncthreads();
      vcluster8(t + dstep, t + 1, has_s, pf_nxt);
      __syncthreads();
    };
    ATTNFUSE_RUN_STEPS(step8, 0, paired ? seg_split : n, !paired)
    if (paired) {
      // The switch between the blocks of a paired workgroup, as in the bf16
      // schedule below: the first half waits out one barrier slot, the
      // second block's first tile comes from K(seg_split)'s ring slot.
      if (m_first) __syncthreads();
      finish_first_block();
      load_q8();
      start_second_block();
      first_tile8_at(seg_split, pfa);
      if (!m_first) __syncthreads();
      ATTNFUSE_RUN_STEPS(step8, seg_split, n, true)
    }
    if (n > 0 && m_first) __syncthreads();
  } else if constexpr (PP) {
    // ---- ping-pong schedule (two waves per SIMD) ----
    // Waves w and w + NW/2 share a SIMD.  Each wave alternates an MFMA
    // cluster M(t) (S(t+1) = K'(t+1) Q'^T and O^T += V(t)^T P(t)^T, 32 MFMAs,
    // operands from LDS) with a vector cluster (softmax of the S tile just
    // computed, in-place RoPE of one K tile, DMA issue); a barrier closes
    // every cluster.  The second half of the workgroup starts with one extra
    // vector cluster, so on every SIMD one wave keeps the matrix core busy
    // while its partner does the vector work.
    // Half-step timing (slot 2t: first half runs M(t), second half a vector
    // cluster; slot 2t+1: the other way round): in slots 2t and 2t+1 both
    // halves rotate their pairs of K(t+2) and issue the DMA of K(t+3), its
    // table entries and V(t+2).  A vector cluster first waits for every DMA
    // its wave issued in its previous vector cluster; with four-slot rings
    // every slot is refilled only after both halves have read it.
    const bool m_first = wave < NW / 2;
    // Tiles past the list are never loaded here (every vector cluster waits
    // for all of its wave's loads, so no fixed instruction count is needed):
    // their scores are masked out entirely and they never meet V.
    if (n > 0) {
      issue_group(0, 0, 0, false, true);                  // K(0), V(0)
      if (n > 1) issue_group(1, 1, 1, false, true);       // K(1), V(1)
      if (n > 2) issue_group(2, 2, 2, true, false);       // K(2) and its table entries
      if (ROPE) {
        fetch_direct(0);
        fetch_direct(1);
      }
    }
    load_q_issue_staged();
    if (SCOREMOD && p.alibi) slope2 = p.alibi[h] * kLog2e;
    if (n > 0) bias_fetch(tile_k0(0));
    vmcnt_wait<0>();
    // Q rows leave their staging area (K slot 3, V slots 2-3, ...) before
    // the barrier, after which those slots are refilled.  K(0) and K(1),
    // which every wave reads, are rotated before the barrier; the private Q
    // rotation and the first tile follow it.
    q_rows_from_lds();
    if (n > 0 && ROPE) {
      rotate_direct(0);
      rotate_direct(1);
    }
    __syncthreads();
    load_q_finish();
    if (n > 0) first_tile();
    if (n > 1) bias_fetch(tile_k0(1));  // waited for by the next vector cluster

    constexpr int NST = 2 * NKK;  // MFMA pairs per cluster (S step + PV step)
    static_assert(NST == 4 * NDT, "one S and one PV MFMA per step");
    // Fragment prefetch distance (1 with score mods: their bias registers
    // stay live through the MFMA cluster).
    constexpr int PF = SCOREMOD ? 1 : 2;
    f32x16 sn[2];                 // S(t+1) from an MFMA cluster to the next vector cluster
    // The MFMA cluster runs at raised wave priority: when both waves of a SIMD
    // can issue, the matrix core is fed first (otherwise the older wave wins
    // and the second half's MFMA clusters stretch).
    auto mcluster = [&](int t, const bf16x8 (&pf)[4]) {
      __builtin_amdgcn_s_setprio(1);
      const float cb = CSPLAT ? mod_base(tile_k0(min(t + 1, n - 1))) : 0.f;
      // One VGPR base per K chunk column and per V d tile for this step's
      // slots; the rest of every operand address is an instruction offset.
      const uint32_t ks = lds0 + (uint32_t)((t + 1) % RING) * L::KSLOT;
      const uint32_t vs = lds0 + L::V_OFF + (uint32_t)(t % RING) * L::VSLOT;
      uint32_t kbase[NKK / 2], vbase[NDT];
#pragma unroll
      for (int c = 0; c < NKK / 2; ++c) kbase[c] = ks + klane[c];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vbase[dt] = vs + voff[dt];
      auto kf = [&](int st, int kk) -> bf16x8 {
        return lds_read16(kbase[kk % (NKK / 2)] + (kk / (NKK / 2)) * L::KHI + 32 * st * D);
      };
      auto vf = [&](int c, int dt) -> bf16x8 {
        const i16x4 r0 = lds_read_tr4(vbase[dt] + c * 32 * D);
        const i16x4 r1 = lds_read_tr4(vbase[dt] + c * 32 * D + 16 * D);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 a = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        return __builtin_bit_cast(bf16x8, a);
      };
      bf16x8 afr[PF + 1], vfr[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        afr[k] = kf(k & 1, k >> 1);
        vfr[k] = vf(k / NDT, k % NDT);
      }
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        if (k + PF < NST) {
          afr[(k + PF) % (PF + 1)] = kf((k + PF) & 1, (k + PF) >> 1);
          vfr[(k + PF) % (PF + 1)] = vf((k + PF) / NDT, (k + PF) % NDT);
        }
        sn[k & 1] = mfma32(afr[k % (PF + 1)], qf[k >> 1], k < 2 ? (SCOREMOD ? (CSPLAT ? f32x16{} + cb : f32x16{}) : minit) : sn[k & 1]);
        o[k % NDT] = mfma32(vfr[k % (PF + 1)], pf[k / NDT], o[k % NDT]);
        if (k % NDT == NDT - 1) ol = mfma32(ones8, pf[k / NDT], ol);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // Vector cluster of step t; st = index of the S tile to turn into P
    // (absent for the second half's first step).
    auto vcluster = [&](int t, int st, bool has_s, bf16x8 (&pf_next)[4]) {
      vmcnt_wait<0>();
      const Group g = make_group(t + 3, t + 3, t + 2);
      const bool k_live = t + 3 < n, v_live = t + 2 < n;
      // K(t+3) and V(t+2) first: their slots were last read two steps ago.
      if (k_live) {
#pragma unroll
        for (int i = 0; i < 2 * NKW_HI; ++i)
          if (i < 2 * nkw) dma_item(g, i);
      }
      if (v_live) {
#pragma unroll
        for (int j = 0; j < NVW; ++j) dma_item(g, (2 + TPK) * nkw + j);
      }
      // Operands of the rotation of K(t+2).
      char* kslot2 = smem + ((t + 2) % RING) * L::KSLOT;
      const char* tsl = smem + L::T_OFF + lane * 16;
      uint4 rl[NKW_HI], rh[NKW_HI], rt0[NKW_HI], rt1[NKW_HI];
      if (ROPE) {
#pragma unroll
        for (int m = 0; m < NKW_HI; ++m) {
          const int kp = wave + NW * m;
          if (m < nkw) {
            rl[m] = ld16(kslot2 + kp * 1024 + lane * 16);
            rh[m] = ld16(kslot2 + L::KHI + kp * 1024 + lane * 16);
            rt0[m] = ld16(tsl + kp * L::TPAIR);
            rt1[m] = ld16(tsl + kp * L::TPAIR + 1024);
          }
        }
      }
      if (has_s) {
        const int k0s = tile_k0(min(st, n - 1));
        // A tile no key of which this wave's rows may see (the band's far
        // edge, a window's start, past the keys): P = 0 without the masks
        // and the exponentials; it leaves m, l and O as they are.  (Not in
        // the RoPE instances: at their register limit the test spills.)
        const bool dead = !ROPE && (st >= n || k0s >= Nk ||
                                    (has_band && (k0s + 63 - w0 < band_lo || k0s - w_last > band_hi)));
        if (dead) {
#pragma unroll
          for (int c = 0; c < 4; ++c) pf_next[c] = bf16x8{};
        } else {
          mask_scores(st, sn);
          uint32_t pw[16];
#pragma unroll
          for (int x = 0; x < 16; ++x) pw[x] = exp_pair(sn, x, k0s);
          finish_tile(sn, -neg_m(), pw);
          to_frags(pw, pf_next);
        }
        if (st + 1 < n) bias_fetch(tile_k0(st + 1));
      }
      if (ROPE) {
        // Table entries of K(t+3) go into the slot read above: those reads
        // completed during the softmax; wait for them, then issue.
        lgkmcnt_wait<0>();
        if (k_live) {
#pragma unroll
          for (int i = 2 * NKW_HI; i < (2 + TPK) * NKW_HI; ++i)
            if (i - 2 * NKW_HI < TPK * nkw) dma_item(g, i - 2 * NKW_HI + 2 * nkw);
        }
#pragma unroll
        for (int m = 0; m < NKW_HI; ++m) {
          const int kp = wave + NW * m;
          if (m < nkw) {
            rope_rotate_bf16x8_t(rl[m], rh[m], rt0[m], rt1[m]);
            st16(kslot2 + kp * 1024 + lane * 16, rl[m]);
            st16(kslot2 + L::KHI + kp * 1024 + lane * 16, rh[m]);
          }
        }
      }
    };
    // Both halves run the same loop; the second half's vector clusters work
    // one step ahead on K and V (their slot 2t+2 belongs to step t+1).
    const int dstep = m_first ? 0 : 1;
    if (n > 0 && !m_first) {
      vcluster(0, 0, false, pfb);
      __syncthreads();
    }
    auto step = [&](int t, const bf16x8 (&pf_cur)[4], bf16x8 (&pf_nxt)[4], bool has_s)
        __attribute__((always_inline)) {
      mcluster(t, pf_cur);
      __syncthreads();
      vcluster(t + dstep, t + 1, has_s, pf_nxt);
      __syncthreads();
    };
    ATTNFUSE_RUN_STEPS(step, 0, paired ? seg_split : n, !paired)
    if (paired) {
      // Both halves are past step seg_split - 1 here (the second half has
      // also run its vector cluster of step seg_split).  K'(seg_split),
      // K'(seg_split + 1), V(seg_split), V(seg_split + 1) are in their
      // slots; the next tiles' loads are in flight.
      if (m_first) __syncthreads();
      finish_first_block();
      load_q_issue();  // the second block's Q rows and angles (direct loads: every slot is busy)
      start_second_block();
      load_q_finish();
      first_tile_at(seg_split, pfa);
      // The second half sits out one slot, restoring the alternation.
      if (!m_first) __syncthreads();
      ATTNFUSE_RUN_STEPS(step, seg_split, n, true)
    }
    // Same barrier count in both halves: the first half's closing barrier
    // matches the second half's extra vector cluster.
    if (n > 0 && m_first) __syncthreads();
  } else if constexpr (SHALLOW) {
    // ---- shallow schedule: two-slot rings; four workgroups share a CU, so
    // each SIMD runs two waves of different workgroups ----
    // Iteration t: wait for the loads of iteration t-1 (V(t), K(t+1) and
    // its table entries); load K(t+2) into K(t)'s slot and V(t+1) into
    // V(t-1)'s (both last read before the previous barrier); O^T += V^T P^T
    // for tile t with the rotation of K(t+1) between its MFMAs, then this
    // thread's table entries of K(t+2) (its entries of K(t+1) are consumed);
    // barrier; S(t+1) = K'(t+1) Q'^T, masks, softmax into P(t+1); barrier.
    // Every load has an iteration to land, and the other workgroup's wave on
    // the SIMD runs while a wave waits.
    auto issue_t = [&](int ut) __attribute__((always_inline)) {
      const Group g = make_group(ut, ut, ut);
#pragma unroll
      for (int i = 0; i < GRP_MAX; ++i)
        if (i >= 2 * nkw && i < (2 + TPK) * nkw) dma_item(g, i);
    };
    // Prologue: K(0), its table entries and V(0); Q; K(0) rotated; K(1) and
    // its table entries in flight; P(0).
    if (n > 0) issue_group(0, 0, 0, true, true);
    load_q_issue();
    if (SCOREMOD && p.alibi) slope2 = p.alibi[h] * kLog2e;
    vmcnt_wait<0>();
    const char* const tl = smem + L::T_OFF + lane * 16;
    // This thread's chunks of K(u), pair m: operands (rot_read), then the
    // rotation and the stores (rot_write).
    struct RotPair {
      uint4 lo, hi, t0, t1;
      uint32_t off;  // byte offset of the low chunk in smem
    };
    auto rot_read = [&](int u, int m) -> RotPair {
      const int kp = wave + NW * m;
      RotPair r;
      r.off = (uint32_t)((u % RING) * L::KSLOT + kp * 1024 + lane * 16);
      r.t0 = ld16(tl + kp * L::TPAIR);
      r.t1 = ld16(tl + kp * L::TPAIR + 1024);
      r.lo = ld16(smem + r.off);
      r.hi = ld16(smem + r.off + L::KHI);
      return r;
    };
    auto rot_write = [&](RotPair r) {
      rope_rotate_bf16x8_t(r.lo, r.hi, r.t0, r.t1);
      st16(smem + r.off, r.lo);
      st16(smem + r.off + L::KHI, r.hi);
    };
    if (n > 0) {
      if (ROPE) {
#pragma unroll
        for (int m = 0; m < NKW_HI; ++m)
          if (m < nkw) rot_write(rot_read(0, m));
      }
      issue_group(1, 1, 1, true, false);
    }
    __syncthreads();
    load_q_finish();
    if (n > 0) first_tile();
    // Iteration 0 refills K slot 0, which every wave has just read for S(0).
    __syncthreads();

    constexpr int NSA = 2 * NKK;  // S MFMAs per tile
    constexpr int NSB = 4 * NDT;  // P V MFMAs per tile
    constexpr int PF = 2;         // fragment prefetch distance
    static_assert(2 * NKW_HI <= NSB, "rotation steps fit the P V steps");
    auto iteration = [&](int t, const bf16x8 (&pf)[4], bf16x8 (&pf_next)[4], bool has_s)
        __attribute__((always_inline)) {
      vmcnt_wait<0>();
      issue_group(t + 2, t + 2, t + 1, false, true);
      // O^T += V^T P^T (tile t); pair m of the rotation of K(t+1): operands
      // at step 2m, arithmetic and stores at step 2m + 1.
      const uint32_t vs = lds0 + L::V_OFF + (uint32_t)(t % RING) * L::VSLOT;
      bf16x8 vfr[PF + 1];
      RotPair rp[NKW_HI];
#pragma unroll
      for (int k = 0; k < PF; ++k) vfr[k] = v_frag(vs, k / NDT, k % NDT);
#pragma unroll
      for (int k = 0; k < NSB; ++k) {
        if (k + PF < NSB) vfr[(k + PF) % (PF + 1)] = v_frag(vs, (k + PF) / NDT, (k + PF) % NDT);
        o[k % NDT] = mfma32(vfr[k % (PF + 1)], pf[k / NDT], o[k % NDT]);
        if (k % NDT == NDT - 1) ol = mfma32(ones8, pf[k / NDT], ol);
        if (ROPE) {
#pragma unroll
          for (int m = 0; m < NKW_HI; ++m)
            if (m < nkw) {
              if (k == 2 * m) rp[m] = rot_read(t + 1, m);
              if (k == 2 * m + 1) rot_write(rp[m]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ROPE) issue_t(t + 2);
      __syncthreads();
      // S(t+1) = K'(t+1) Q'^T, masks, softmax into P(t+1).
      const char* ks = smem + ((t + 1) % RING) * L::KSLOT;
      const int k0n = tile_k0(min(t + 1, n - 1));
      f32x16 sn[2];
      bf16x8 afr[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) afr[k] = k_frag(ks, k & 1, k >> 1);
#pragma unroll
      for (int k = 0; k < NSA; ++k) {
        if (k + PF < NSA) afr[(k + PF) % (PF + 1)] = k_frag(ks, (k + PF) & 1, (k + PF) >> 1);
        sn[k & 1] = mfma32(afr[k % (PF + 1)], qf[k >> 1], k < 2 ? (SCOREMOD ? (CSPLAT ? f32x16{} + mod_base(k0n) : f32x16{}) : minit) : sn[k & 1]);
      }
      mask_scores(t + 1, sn);
      uint32_t pw[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) pw[x] = exp_pair(sn, x, k0n);
      if (has_s) finish_tile(sn, -neg_m(), pw);
      to_frags(pw, pf_next);
      __syncthreads();
    };
    // One block of a chain at a time, as in the four-slot schedule below.
    int seg0 = 0;
    for (int c = 0; c < n_chain; ++c) {
      const bool last_seg = c == n_chain - 1;
      const int seg1 = last_seg ? n : seg_end(c, seg0);
      if (c > 0) {
        store_block_regs();
        set_rows(qblk + c);
        load_q_issue();
        reset_softmax();
        load_q_finish();
        if (seg1 > seg0) first_tile_at(seg0, pfa);
        __syncthreads();
      }
      ATTNFUSE_RUN_STEPS(iteration, seg0, seg1, last_seg)
      seg0 = seg1;
    }
  } else {
    // Prologue: K(0), K(1) loaded and rotated, V(0) loaded; the groups of
    // iterations -2 and -1 ({K(2), V(1)}, {K(3), V(2)}) in flight; P(0).
    if (n > 0) {
      issue_group(0, 0, 0, false, true);
      issue_group(1, 1, 1, false, false);
      if (ROPE) {
        fetch_direct(0);
        fetch_direct(1);
      }
    }
    // Q and the slope load while the first tiles arrive.
    load_q_issue();
    if (SCOREMOD && p.alibi) slope2 = p.alibi[h] * kLog2e;
    vmcnt_wait<0>();
    if (n > 0) {
      if (ROPE) {
        rotate_direct(0);
        rotate_direct(1);
      }
      // Groups of iterations -2 and -1: {K(2), V(1)}, {K(3), table of K(2), V(2)}.
      issue_group(2, 2, 1, false, true);
      issue_group(3, 2, 2, true, true);
    }
    __syncthreads();
    load_q_finish();
    if (n > 0) first_tile();
    // Iteration 0 refills K slot 0, which every wave has just read for S(0).
    __syncthreads();

    // ---- main loop: hand-scheduled phases, one MFMA per step ----
    // Phase A: the MFMAs of S(t+1); between them the RoPE rotation of K(t+2).
    // Phase B: the MFMAs of O^T += V^T P^T for tile t; between them the
    // exp / pack / row sums that turn S(t+1) into P(t+1).  Fragments are read
    // PF steps ahead; sched_barrier keeps each step's instructions together so
    // the vector work fills the MFMA shadow.
    constexpr int NSA = 2 * NKK;                     // phase A steps
    constexpr int NSB = 4 * NDT;                     // phase B steps
    constexpr int NROT = ROPE ? 8 * NKW_HI : 0;      // rotation items, one element pair each
    constexpr int AIPS = (NROT + NSA - 3) / (NSA - 2);  // per step from step 2 on
    constexpr int XPB = 16 / NSB;                    // exp pairs per phase B step
    constexpr int PF = 2;                            // fragment prefetch distance

    // Group instruction slots: every other step of phase A carries the K part
    // (IPDA instructions per slot), every other step of phase B the table and
    // V parts (IPDB per slot).
    constexpr int IPDA = (2 * NKW_HI + NSA / 2 - 1) / (NSA / 2);
    constexpr int IPDB = (TPK * NKW_HI + NVW + NSB / 2 - 1) / (NSB / 2);
    auto dma_slot_a = [&](const Group& g, int slot) {
  #pragma unroll
      for (int j = slot * IPDA; j < (slot + 1) * IPDA; ++j)
        if (j < 2 * NKW_HI && j < 2 * nkw) dma_item(g, j);
    };
    auto dma_slot_b = [&](const Group& g, int slot) {
  #pragma unroll
      for (int j = slot * IPDB; j < (slot + 1) * IPDB; ++j)
        if (j < TPK * NKW_HI + NVW && 2 * nkw + j < grp) dma_item(g, 2 * nkw + j);
    };
    // has_s = false: S(t+1) belongs to the next chained block (its Q is not
    // loaded yet), so its softmax is not taken.
    auto iteration = [&](int t, const bf16x8 (&pf)[4], bf16x8 (&pf_next)[4], bool has_s) {
      wait_group();
      const Group g = make_group(t + 4, t + 3, t + 3);

      // ---- phase A ----
      const char* ks = smem + ((t + 1) % RING) * L::KSLOT;
      const int k0n = tile_k0(min(t + 1, n - 1));
      f32x16 sn[2];
      bf16x8 afr[PF + 1];
  #pragma unroll
      for (int k = 0; k < PF; ++k) afr[k] = k_frag(ks, k & 1, k >> 1);
      // Rotation of K(t+2): pair m, elements e = 0..7 of this lane's chunk, in
      // two halves of four.  A half's operands (two words of the low chunk, two
      // of the high chunk, four table words) are read from LDS two steps before
      // its first item, so at most one and a half halves are held at a time.
      char* kslot2 = smem + ((t + 2) % RING) * L::KSLOT;
      const char* tsl = smem + L::T_OFF + lane * 16;
      uint2 rlo[NKW_HI][2], rhi[NKW_HI][2];
      uint4 rtb[NKW_HI][2];
      uint32_t olw[NKW_HI][4], ohw[NKW_HI][4];
      float rl_even[NKW_HI], rh_even[NKW_HI];
      auto rot_load = [&](int m, int hf) {
        const int kp = wave + NW * m;
        if (m < nkw) {
          rtb[m][hf] = ld16(tsl + kp * L::TPAIR + 1024 * hf);
          rlo[m][hf] = *reinterpret_cast<const uint2*>(kslot2 + kp * 1024 + lane * 16 + 8 * hf);
          rhi[m][hf] = *reinterpret_cast<const uint2*>(kslot2 + L::KHI + kp * 1024 + lane * 16 + 8 * hf);
        }
      };
      auto rot_item = [&](int ri) {
        const int m = ri / 8, e = ri % 8, hf = e / 4, e4 = e % 4;
        if (m < nkw) {
          const uint32_t wl = (e4 < 2) ? rlo[m][hf].x : rlo[m][hf].y;
          const uint32_t wh = (e4 < 2) ? rhi[m][hf].x : rhi[m][hf].y;
          const uint32_t tw = e4 == 0 ? rtb[m][hf].x : e4 == 1 ? rtb[m][hf].y : e4 == 2 ? rtb[m][hf].z : rtb[m][hf].w;
          float rl, rh;
          rope_elem(wl, wh, e & 1, tw, rl, rh);
          if (e & 1) {
            olw[m][e / 2] = pack_bf16x2(rl_even[m], rl);
            ohw[m][e / 2] = pack_bf16x2(rh_even[m], rh);
          } else {
            rl_even[m] = rl;
            rh_even[m] = rh;
          }
        }
      };
  #pragma unroll
      for (int k = 0; k < NSA; ++k) {
        if (k + PF < NSA) afr[(k + PF) % (PF + 1)] = k_frag(ks, (k + PF) & 1, (k + PF) >> 1);
        sn[k & 1] = mfma32(afr[k % (PF + 1)], qf[k >> 1], k < 2 ? (SCOREMOD ? (CSPLAT ? f32x16{} + mod_base(k0n) : f32x16{}) : minit) : sn[k & 1]);
        if (k & 1) dma_slot_a(g, k / 2);
        if (ROPE) {
          // Item ri runs at step 2 + ri / AIPS; its half's operands two steps earlier.
  #pragma unroll
          for (int hh = 0; hh < 2 * NKW_HI; ++hh)
            if ((4 * hh) / AIPS == k) rot_load(hh / 2, hh % 2);
          if (k >= 2) {
  #pragma unroll
            for (int ri = (k - 2) * AIPS; ri < (k - 1) * AIPS; ++ri)
              if (ri < NROT) rot_item(ri);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ROPE) {
  #pragma unroll
        for (int m = 0; m < NKW_HI; ++m) {
          const int kp = wave + NW * m;
          if (m < nkw) {
            st16(kslot2 + kp * 1024 + lane * 16, make_uint4(olw[m][0], olw[m][1], olw[m][2], olw[m][3]));
            st16(kslot2 + L::KHI + kp * 1024 + lane * 16, make_uint4(ohw[m][0], ohw[m][1], ohw[m][2], ohw[m][3]));
          }
        }
      }
      mask_scores(t + 1, sn);

      // ---- phase B ----
      const uint32_t vs = lds0 + L::V_OFF + (uint32_t)(t % RING) * L::VSLOT;
      bf16x8 vfr[PF + 1];
  #pragma unroll
      for (int k = 0; k < PF; ++k) vfr[k] = v_frag(vs, k / NDT, k % NDT);
      uint32_t pw[16];
      float ex[16][2];
  #pragma unroll
      for (int k = 0; k < NSB; ++k) {
        if (k + PF < NSB) vfr[(k + PF) % (PF + 1)] = v_frag(vs, (k + PF) / NDT, (k + PF) % NDT);
        o[k % NDT] = mfma32(vfr[k % (PF + 1)], pf[k / NDT], o[k % NDT]);
        if (k % NDT == NDT - 1) ol = mfma32(ones8, pf[k / NDT], ol);
        if (k & 1) dma_slot_b(g, k / 2);
        // Pairs of step k: arguments now, exponentials one step later, pack
        // and row sum two steps later.
  #pragma unroll
        for (int x = k * XPB; x < (k + 1) * XPB; ++x) exp_stage1(sn, x, k0n);
  #pragma unroll
        for (int x = (k - 1) * XPB; x < k * XPB; ++x)
          if (x >= 0) exp_stage2(sn, x, ex[x]);
  #pragma unroll
        for (int x = (k - 2) * XPB; x < (k - 1) * XPB; ++x)
          if (x >= 0) pw[x] = exp_stage3(x, ex[x]);
        __builtin_amdgcn_sched_barrier(0);
      }
  #pragma unroll
      for (int x = (NSB - 1) * XPB; x < NSB * XPB; ++x) exp_stage2(sn, x, ex[x]);
  #pragma unroll
      for (int x = (NSB - 2) * XPB; x < NSB * XPB; ++x) pw[x] = exp_stage3(x, ex[x]);
      if (has_s) finish_tile(sn, -neg_m(), pw);
      to_frags(pw, pf_next);
      __syncthreads();
    };
    // Steps unrolled by two so that the P tiles swap roles without copies,
    // one block of a chain at a time.  At a switch: the finished block's
    // output from registers, the next block's rows, Q (loaded and rotated)
    // and softmax state, then S of its first tile from that tile's ring
    // slot (K' is in place: tile u is rotated in iteration u - 2, and its
    // slot is refilled in iteration u, after the barrier below).
    int seg0 = 0;
    for (int c = 0; c < n_chain; ++c) {
      const bool last_seg = c == n_chain - 1;
      const int seg1 = last_seg ? n : seg_end(c, seg0);
      if (c > 0) {
        store_block_regs();
        set_rows(qblk + c);
        load_q_issue();
        reset_softmax();
        load_q_finish();
        if (seg1 > seg0) first_tile_at(seg0, pfa);
        __syncthreads();
      }
      ATTNFUSE_RUN_STEPS(iteration, seg0, seg1, last_seg)
      seg0 = seg1;
    }
  }
#undef ATTNFUSE_RUN_STEPS
  // No DMA may land in LDS after the workgroup ends, and the epilogue reuses
  // the ring slots: every wave's loads must have landed first.
  vmcnt_wait<0>();
  __syncthreads();

  // ---- epilogue: O = O^T / l, optional lse ----
  // A lane holds one query row's values in 8-byte pieces spread over the
  // row; staged through LDS (rows padded against bank conflicts), they leave
  // as whole 16-byte chunks of consecutive rows, so each store instruction
  // writes a few complete rows.
  const float l_tot = ol[0];
  const float inv = l_tot > 0.f ? p.v_scale / l_tot : 0.f;  // v_scale: fp8 V dequantisation (else 1)
  constexpr int OROW = 2 * D + 16;  // bytes per staged row
  char* const ost = smem + wave * 32 * OROW;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * lh;
      uint2 w;
      w.x = pack_bf16x2(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv);
      w.y = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
      *reinterpret_cast<uint2*>(ost + lq * OROW + 2 * d) = w;
    }
  constexpr int CPRO = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPRO;  // rows per store instruction
  __bf16* const obase = reinterpret_cast<__bf16*>(p.o) + b * p.osb + h * p.osh;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = k * RPI + lane / CPRO, ch = lane % CPRO;
    const uint4 v = ld16(ost + row * OROW + 16 * ch);
    if (w0 + row < p.Nq) st16(obase + (long long)(w0 + row) * p.osn + 8 * ch, v);
  }
  if (i < p.Nq && p.lse && lh == 0)
    p.lse[((long long)b * p.Hq + h) * p.Nq + i] =
        l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
}

}  // namespace attnfuse
