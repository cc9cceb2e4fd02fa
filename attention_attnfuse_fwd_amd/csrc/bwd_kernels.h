// Attention backward ("4.4 Backward Pass"), the FlashAttention-2 split into
// passes none of which needs atomics:
//   0. with RoPE: Q' = RoPE(Q) and K' = RoPE(K) into the workspace, rounded
//      once to bf16 (the forward rounds its rotated operands the same way);
//      the three passes below read them many times over
//   1. delta[b, h, i] = sum_d dO[i, d] O[i, d]            (row reduction)
//   2. per (b, kv-head, block of 128 keys): dK and dV, looping over the
//      q-heads of the group and the 64-row query tiles the masks allow
//   3. per (b, q-head, block of 128 query rows): dQ, looping over 64-key tiles
// Probabilities are re-derived tile by tile from the forward's saved
// L = m + ln l:  P = exp(S - L),  dS = P (dP - delta),  dQ' = scale dS K',
// dK' = scale dS^T Q',  dV = P^T dO; the RoPE gradients rotate dQ' and dK'
// back by the negative angle (the rotation is orthogonal).
//
// All products run on bf16 MFMA (32x32x16, fp32 accumulate) with P and dS
// rounded to bf16.  Tiles are staged through swizzled row-major LDS, double
// buffered: the next tile's loads are in flight during the current tile's
// products (the dK/dV pass moves its Q' and dO tiles by direct global -> LDS
// DMA, which holds no registers) and one barrier separates tiles.  LDS
// operands of the products are read two products ahead.  The transposed operands
// (dO^T, Q'^T, K'^T) are read with ds_read_b64_tr_b16.  Each wave classifies
// its part of a tile as fully visible (no mask arithmetic), fully masked
// (skipped) or partial (per-element band and bound tests).
//
// The kernels live in this header; bwd_d64.hip and bwd_d128.hip instantiate
// them for one head dim each (compiled with different register options).
#pragma once

#include <climits>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attnfuse {

namespace {

constexpr int kBwdThreads = 256;    // default thread count of the row stages
constexpr int kMaxSparseSteps = 8192;  // dK/dV step masks held in LDS
constexpr int kKvThreads = 512;     // 8 waves, two per SIMD (dK/dV)
constexpr int kDqThreads = 512;     // 8 waves, two per SIMD (dQ)
constexpr int kDqRows = 256;        // query rows per dQ workgroup

// LDS tiles are unpadded row-major [rows][D] bf16 with the 16-byte chunks of
// row r permuted by chunk ^ swz(r), chosen so that both access patterns are
// free of bank conflicts on the 64-bank LDS: a row read (16 lanes, 16
// consecutive rows, one chunk each) and a transposed read (32 lanes, four
// consecutive rows, four consecutive chunks each).  D = 128 rows fill the 256
// bytes of the banks; D = 64 rows share them in pairs.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {  // bytes
  return r * D * 2 + 16 * (c ^ swz<D>(r));
}

// Transposed A operand (32 rows of the result x 16 contraction steps) from a
// tile in LDS, for MFMA k index 8*kb + e  <->  tile row row0 + 8*(e/4) + 4*kb
// + e%4 (the order in which a 32x32 accumulator holds its rows), result row =
// column col0 + lane % 32.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(uint32_t tile, int row0, int col0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  const int kb = g >> 1, c16 = 16 * (g & 1);
  const int a = i >> 2, bq = i & 3;
  const int r = row0 + 4 * kb + a, col = col0 + c16 + 4 * bq;
  const uint32_t r1 = tile + (uint32_t)(tile_off<D>(r, col >> 3) + 2 * (col & 7));
  const uint32_t r2 = tile + (uint32_t)(tile_off<D>(r + 8, col >> 3) + 2 * (col & 7));
  const i16x4 x = lds_read_tr4(r1), y = lds_read_tr4(r2);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Row-major A / B operand: 8 consecutive elements of row `row`, columns
// 16*kk + 8*kb .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const __bf16* tile, int row, int kk) {
  const int kb = (threadIdx.x & 63) >> 5;
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) +
                                          tile_off<D>(row, 2 * kk + kb));
}

// Per-lane LDS byte offsets, computed once: the swizzle of a row depends only
// on its index mod 16, so moving by whole 16-row groups (subtile, chunk, wave
// row block) is a constant added to these.
//   row[kk]: row_frag of row lq, chunk 2 kk + kb
//   tr[2 dt + h]: tr_frag of rows 4 kb + a + 8 h, column 32 dt + c16 + 4 bq
template <int D>
struct LdsOffsets {
  uint32_t row[D / 16];
  uint32_t tr[D / 16];
  __device__ __forceinline__ LdsOffsets() {
    const int lane = threadIdx.x & 63;
    const int lq = lane & 31, kb = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = (uint32_t)tile_off<D>(lq, 2 * kk + kb);
    const int g = lane >> 4, i = lane & 15;
    const int tkb = g >> 1, c16 = 16 * (g & 1), a = i >> 2, bq = i & 3;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = 32 * dt + c16 + 4 * bq;
        tr[2 * dt + h] = (uint32_t)(tile_off<D>(4 * tkb + a + 8 * h, col >> 3) + 2 * (col & 7));
      }
  }
  // A operand from row-major rows row0 + lq (row0 a multiple of 16), chunk kk.
  __device__ __forceinline__ bf16x8 rowf(uint32_t tile, int row0, int kk) const {
    return lds_read16(tile + row[kk] + (uint32_t)(row0 * D * 2));
  }
  // Transposed A operand: tile rows row0 + 8 (e/4) + 4 kb + e%4 (row0 a multiple
  // of 16), result rows = columns 32 dt + lane % 32.
  __device__ __forceinline__ bf16x8 trf(uint32_t tile, int row0, int dt) const {
    const uint32_t base = tile + (uint32_t)(row0 * D * 2);
    const i16x4 x = lds_read_tr4(base + tr[2 * dt]), y = lds_read_tr4(base + tr[2 * dt + 1]);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// 8 bf16 values of row `row` (global, element stride sn), columns c .. c+7.
__device__ __forceinline__ uint4 ld_row8(const __bf16* base, long long sn, int row, int c) {
  return ld16(base + (long long)row * sn + c);
}

// Rows [r0, r0 + R) of a [N, D] bf16 matrix (rows clamped to N - 1), staged
// in two steps so the next tile's loads can be in flight while the current
// one is multiplied: load() reads this thread's share into registers,
// store() writes it to a swizzled LDS tile.
template <int D, int R, int NT = kBwdThreads>
struct RowStage {
  static constexpr int CPR = D / 8;                          // 16-byte chunks per row
  static constexpr int U = (R * CPR + NT - 1) / NT;
  uint4 x[U];
  __device__ __forceinline__ void load(const __bf16* src, long long sn, int r0, int N) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = threadIdx.x + NT * k;
      if ((R * CPR) % NT == 0 || u < R * CPR)
        x[k] = ld_row8(src, sn, min(r0 + u / CPR, N - 1), 8 * (u % CPR));
    }
  }
  __device__ __forceinline__ void store(__bf16* tile) const {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int u = threadIdx.x + NT * k;
      if ((R * CPR) % NT == 0 || u < R * CPR)
        st16(reinterpret_cast<char*>(tile) + tile_off<D>(u / CPR, u % CPR), x[k]);
    }
  }
};

// Rows [r0, r0 + 64) of a [N, D] bf16 plane (row stride sn elements, rows
// clamped to N - 1; r0 may lie past the last row) into a swizzled LDS tile
// by direct global -> LDS DMA.  The tile's D / 8 pieces of 1 KB (RPD rows
// each) are shared by the NW waves; lane l of a piece writes position l % CPR
// of row l / CPR, which holds chunk (l % CPR) ^ swz(row).  The load is
// counted by vmcnt only (the caller waits for it before the barrier that
// publishes the tile).  Row offsets from the first row are 32-bit: the host
// keeps row strides below 2^24 elements.
template <int D, int NW>
__device__ __forceinline__ void dma_tile64(uint32_t tile_lds, const __bf16* plane, long long sn, int r0,
                                           int N) {
  constexpr int CPR = D / 8, RPD = 64 / CPR, PIECES = 64 / RPD, PPW = PIECES / NW;
  static_assert(PPW * NW == PIECES, "the waves share the pieces of a tile evenly");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = min(r0, N - 1);
  const __bf16* base = plane + (long long)rb * sn;
#pragma unroll
  for (int m = 0; m < PPW; ++m) {
    const int piece = wave * PPW + m, r = piece * RPD + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(r);
    const int row = min(r0 + r, N - 1);
    dma16_off(tile_lds + 1024 * piece, base, (uint32_t)((long long)(row - rb) * sn * 2 + 16 * c));
  }
}

// Register fragments of one row (lane's row) as a B operand over the head
// dim: f[kk] = row[16 kk + 8 kb .. +7].
template <int D>
__device__ __forceinline__ void row_frags(bf16x8 (&f)[D / 16], const __bf16* src, long long sn,
                                          int row) {
  const int kb = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = __builtin_bit_cast(bf16x8, ld_row8(src, sn, row, 16 * kk + 8 * kb));
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

// Workgroup -> (unit, block rank) with rank 0 (the longest block under a
// causal band) dispatched first for every unit, and, when the units split
// evenly over the 8 XCDs (consecutive workgroup ids go to consecutive XCDs),
// each XCD's workgroups on a contiguous range of units so that the units'
// shared operands stay in that XCD's L2.
__device__ __forceinline__ void bwd_tile_of(int nunits, int& unit, int& rank) {
  const int id = blockIdx.x;
  if (nunits % 8 == 0) {
    const int upx = nunits / 8, m = id / 8;
    unit = (id % 8) * upx + m % upx;
    rank = m / upx;
  } else {
    unit = id % nunits;
    rank = id / nunits;
  }
}

// An accumulator row as held by store_grad_row's acc, stored unscaled in fp32.
template <int D>
__device__ __forceinline__ void store_part_row(float* dst, const f32x16 (&acc)[D / 32]) {
  const int kb = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g + 4 * kb) =
          make_float4(acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
}

constexpr int kSmAlibi = 1, kSmBias = 2;

// P = exp2(S scale log2e - L log2e) and dS = P (dP - delta) for one 32x32
// block held as accumulators s (scores) and dp, packed to bf16 as two
// 16-row MFMA B operands (chunk c holds the accumulator rows 8c .. 8c+7).
// Accumulator row r of the lane is block row row0 + 8 (r/4) + 4 kb + r%4.
// ROWQ: block rows are queries and the lane's column is key `col`; else
// block rows are keys and the lane's column is query `col`.  L2[r] holds
// L log2e of the row's query (+inf for rows without keys, so that P = 0),
// Dl[r] its delta.  MASK applies the key bound and the band per element.
// Only the chunks C0 .. C1-1 are computed (and only their L2 / Dl entries read).
// SM: score modifiers, kSmAlibi (slope2 = ALiBi slope * log2 e, dpos = key
// position - query position of index 0 pairs) and kSmBias (bias_bh = the
// (b, h) plane of the additive bias).
template <bool MASK, int SM, bool ROWQ, bool WANTP, int C0 = 0, int C1 = 2>
__device__ __forceinline__ void p_ds(const f32x16& s, const f32x16& dp, const float (&L2)[16],
                                     const float (&Dl)[16], int row0, int col, const AttnParams& p,
                                     float slope2, int dpos, const float* bias_bh, bf16x8 (&pf)[2],
                                     bf16x8 (&dsf)[2]) {
  const int kb = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int c = C0; c < C1; ++c) {
    uint32_t wp[4], wd[4];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      float pv[2], dsv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 8 * c + 2 * q2 + e;
        const int row = row0 + 8 * (r / 4) + 4 * kb + r % 4;
        const int i = ROWQ ? row : col, j = ROWQ ? col : row;
        float x = __builtin_fmaf(s[r], p.scale_log2, -L2[r]);
        if (SM & kSmAlibi) x = __builtin_fmaf(slope2, (float)(j - i + dpos), x);
        if (SM & kSmBias)  // indices clamped: masked-out rows and keys still read in bounds
          x = __builtin_fmaf(bias_bh[(long long)min(i, p.Nq - 1) * p.bsi + (long long)min(j, p.Nk - 1) * p.bsj],
                             kLog2e, x);
        float pr = fast_exp2(x);
        if (MASK) {
          const bool ok = (j < p.Nk) & (j - i >= p.band_lo) & (j - i <= p.band_hi);
          pr = ok ? pr : 0.f;
        }
        pv[e] = pr;
        dsv[e] = pr * (dp[r] - Dl[r]);
      }
      if (WANTP) wp[q2] = pack_bf16x2(pv[0], pv[1]);
      wd[q2] = pack_bf16x2(dsv[0], dsv[1]);
    }
    if (WANTP) pf[c] = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
    dsf[c] = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
  }
}

// CSR row of query block qb for q-head h: offsets [beg, end) into col_idx,
// clamped to [0, nnz] (a malformed mask gives wrong numbers, never an
// out-of-bounds read).  Columns are clamped to [0, number of key blocks].
struct CsrRow {
  int beg, end;
};
typedef __attribute__((address_space(4))) const int* csr_ptr_t;  // scalar loads
__device__ __forceinline__ CsrRow csr_row(const AttnParams& p, int h, int qb) {
  const int* rp = p.row_ptr + (p.bs_head_stride ? (long long)h * p.bs_head_stride : 0);
  const long long nnz = p.bs_nnz;
  const long long a = min(max((long long)((csr_ptr_t)rp)[qb], 0LL), nnz);
  const long long e = min(max((long long)((csr_ptr_t)rp)[qb + 1], a), nnz);
  return CsrRow{(int)a, (int)e};
}
__device__ __forceinline__ int csr_col(const AttnParams& p, int e) {
  const int nkb = (p.Nk + p.bn - 1) / p.bn;
  return min(max(((csr_ptr_t)p.col_idx)[e], 0), nkb);
}

}  // namespace

// ---- pass 0: Q' / K' = RoPE(x) into a contiguous [B][H][N][D] copy ----
template <int D>
__global__ void __launch_bounds__(256) bwd_rotate_kernel(const __bf16* x, long long sb, long long sh,
                                                         long long sn, int H, int N, long long rows,
                                                         int pos0, const AttnParams p, __bf16* y) {
  constexpr int CH = D / 16;  // chunk pairs per row
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * CH) return;
  const int c = (int)(idx % CH);
  const long long row = idx / CH;
  const int n = (int)(row % N);
  const long long bh = row / N;
  const int hh = (int)(bh % H), bb = (int)(bh / H);
  const __bf16* src = x + bb * sb + hh * sh + n * sn;
  uint4 lo = ld16(src + 8 * c), hi = ld16(src + D / 2 + 8 * c);
  const long long t = (long long)min(pos0 + n, p.rope_len - 1) * (D / 2) + 8 * c;
  rope_rotate_bf16x8(lo, hi, ld_f8(p.rcos + t), ld_f8(p.rsin + t));
  __bf16* dst = y + row * D;
  st16(dst + 8 * c, lo);
  st16(dst + D / 2 + 8 * c, hi);
}

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

// ---- pass 3: dQ.  8 waves (two per SIMD) x 32 query rows of one q-head;
// key tiles of 64.  Each wave keeps its rows' Q' and dO as MFMA operands and
// its dQ' accumulators in registers (at most 256 per wave), and walks the
// tile's two 32-key subtiles one after the other: S^T, dP^T, dS^T, dQ'^T.
// With a block mask (SPARSE) a workgroup is 2 waves = 64 rows, inside one
// CSR block row, and visits only that row's listed key blocks.
template <int D, int SM, bool SPARSE>
__global__ void __launch_bounds__(SPARSE ? 128 : kDqThreads, 1) bwd_dq_kernel(const AttnParams p,
                                                                            const BwdParams g) {
  constexpr int NKK = D / 16, NDT = D / 32, TILE = 64 * D;
  constexpr int NT = SPARSE ? 128 : kDqThreads, ROWS = NT / 2;
  __shared__ __attribute__((aligned(16))) __bf16 smem[4 * TILE];  // (K', V) x 2 buffers
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int lq = lane & 31;
  const int nqb = (p.Nq + ROWS - 1) / ROWS;
  int bh, rank;
  bwd_tile_of(p.B * p.Hq, bh, rank);
  const int qblk = nqb - 1 - rank;  // later query blocks see more keys under a causal band
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int kvh = h / p.G;
  const int r0 = qblk * ROWS;
  const int i0 = r0 + 32 * wave;  // the wave's first row
  const int i = i0 + lq;
  const int iq = min(i, p.Nq - 1);
  const int wlast = min(i0 + 31, p.Nq - 1);

  const __bf16* kb = g.kr + b * g.kr_sb + kvh * g.kr_sh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;

  // The lane's query row: Q' and dO as B operands over the head dim.
  bf16x8 qf[NKK], df[NKK];
  row_frags<D>(qf, g.qr + b * g.qr_sb + h * g.qr_sh, g.qr_sn, iq);
  row_frags<D>(df, g.dout + b * p.osb + h * p.osh, p.osn, iq);
  const long long row_id = ((long long)b * p.Hq + h) * p.Nq + iq;
  const float lse = p.lse[row_id];
  float L2[16], Dl[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    L2[r] = (i < p.Nq && lse != -INFINITY) ? lse * kLog2e : INFINITY;
    Dl[r] = g.delta[row_id];
  }
  const float slope2 = (SM & kSmAlibi) ? p.alibi[h] * kLog2e : 0.f;
  const float* bias_bh = (SM & kSmBias) ? p.bias + b * p.bsb + h * p.bsh : nullptr;
  const int dpos = p.k_pos0 - p.q_pos0;

  // Key tiles the block visits: the band's range (the band is j - i in index
  // space), or the listed key blocks of the block's CSR row.
  const int wg_last = min(r0 + ROWS - 1, p.Nq - 1);
  int ntiles, kt0 = 0, s_begin = 0, tpb = 1;
  if (SPARSE) {
    const CsrRow row = csr_row(p, h, r0 / p.bm);
    s_begin = row.beg;
    tpb = p.bn / 64;
    ntiles = (row.end - row.beg) * tpb;
  } else {
    int j_lo = 0, j_hi = p.Nk - 1;
    if (p.has_band) {
      j_lo = max(j_lo, (int)max((long long)r0 + p.band_lo, 0LL));
      j_hi = min(j_hi, (int)min((long long)wg_last + p.band_hi, (long long)p.Nk - 1));
    }
    kt0 = (j_lo / 64) * 64;
    ntiles = j_hi >= j_lo ? (j_hi - kt0) / 64 + 1 : 0;
  }
  // First key of tile t; a listed column past the keys lands at k0 >= Nk and
  // is skipped (its loads are clamped to the last key).
  auto tile_k0 = [&](int t) -> int {
    if (SPARSE) return csr_col(p, s_begin + t / tpb) * p.bn + (t % tpb) * 64;
    return kt0 + 64 * t;
  };
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  RowStage<D, 64, NT> kst, vst;
  if (ntiles > 0) {
    kst.load(kb, g.kr_sn, tile_k0(0), p.Nk);
    vst.load(vb, p.vsn, tile_k0(0), p.Nk);
    kst.store(smem);
    vst.store(smem + TILE);
    if (ntiles > 1) {
      kst.load(kb, g.kr_sn, tile_k0(1), p.Nk);
      vst.load(vb, p.vsn, tile_k0(1), p.Nk);
    }
  }
  __syncthreads();
  const LdsOffsets<D> lo;
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = tile_k0(t);
    const uint32_t ks_lds = lds_addr(smem) + (uint32_t)((t & 1) * 2 * TILE * 2), vs_lds = ks_lds + TILE * 2;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // The wave's rows i0 .. wlast against keys ka .. kl.
      const int ka = k0 + 32 * st, kl = min(ka + 31, p.Nk - 1);
      const bool skip = i0 >= p.Nq || ka >= p.Nk ||
                        (p.has_band && (kl - i0 < p.band_lo || ka - wlast > p.band_hi));
      if (skip) continue;  // dS = 0
      const bool full = i0 + 31 < p.Nq && ka + 31 < p.Nk &&
                        (!p.has_band || (ka - (i0 + 31) >= p.band_lo && ka + 31 - i0 <= p.band_hi));
      // S^T and dP^T (lane = query column), alternating products; each
      // product's LDS operand is read PF products ahead, so that its latency
      // hides behind the products in between.
      constexpr int NS = 2 * NKK, PF = 2;
      auto s_frag = [&](int k) { return lo.rowf((k & 1) ? vs_lds : ks_lds, 32 * st, k >> 1); };
      bf16x8 fr[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) fr[k] = s_frag(k);
      f32x16 sa, da;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k + PF < NS) fr[(k + PF) % (PF + 1)] = s_frag(k + PF);
        if (k & 1)
          da = mfma32(fr[k % (PF + 1)], df[k >> 1], k < 2 ? f32x16{} : da);
        else
          sa = mfma32(fr[k % (PF + 1)], qf[k >> 1], k < 2 ? f32x16{} : sa);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The first transposed K' operands of the dQ products are read before
      // the exponentials.
      constexpr int NQ = 2 * NDT;
      auto q_frag = [&](int k) { return lo.trf(ks_lds, 32 * st + 16 * (k / NDT), k % NDT); };
      bf16x8 tq[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) tq[k] = q_frag(k);
      // dS^T = P^T (dP^T - delta), packed to bf16 in 16-key chunks.
      bf16x8 dsf[2], unused[2];
      if (full)
        p_ds<false, SM, false, false>(sa, da, L2, Dl, ka, i, p, slope2, dpos, bias_bh, unused, dsf);
      else
        p_ds<true, SM, false, false>(sa, da, L2, Dl, ka, i, p, slope2, dpos, bias_bh, unused, dsf);
      // dQ'^T += K'^T dS^T (chunk-major, so that consecutive products
      // update different accumulators).
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        if (k + PF < NQ) tq[(k + PF) % (PF + 1)] = q_frag(k + PF);
        acc[k % NDT] = mfma32(tq[k % (PF + 1)], dsf[k / NDT], acc[k % NDT]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t + 1 < ntiles) {  // the other buffer was last read before the previous barrier
      __bf16* nk = smem + ((t + 1) & 1) * 2 * TILE;
      kst.store(nk);
      vst.store(nk + TILE);
      if (t + 2 < ntiles) {
        kst.load(kb, g.kr_sn, tile_k0(t + 2), p.Nk);
        vst.load(vb, p.vsn, tile_k0(t + 2), p.Nk);
      }
    }
    __syncthreads();
  }
  if (i < p.Nq) {
    __bf16* dst = g.dq + b * p.qsb + h * p.qsh + (long long)i * p.qsn;
    store_grad_row<D>(dst, acc, p.scale_log2 / kLog2e, p.rcos != nullptr, p, p.q_pos0 + i);
  }
}

// ---- pass 2: dK, dV.  8 waves (two per SIMD) over 128 keys of one kv-head;
// query tiles of 64.  Waves w and w + 4 own the same 32 keys (the result
// columns) and take the tile's first and second 32 query rows; their dK' and
// dV accumulators are added through LDS at the end.  K' and V of the block
// stay in LDS (read as B operands each step) so that a wave needs at most 256
// registers.
template <int D, int SM, bool SPARSE>
__global__ void __launch_bounds__(kKvThreads, 1) bwd_dkdv_kernel(const AttnParams p, const BwdParams g) {
  constexpr int NKK = D / 16, NDT = D / 32, TILE = 64 * D, BLK = 128 * D;
  // [K' block | V block] then (Q', dO) x 2 buffers; reused for the final sums
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * BLK + 4 * TILE];
  __shared__ __attribute__((aligned(16))) float stat[2][2][64];  // [buffer][L log2e, delta][row]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int lq = lane & 31, lh = lane >> 5;
  const int kw = wave & 3, st = wave >> 2;  // key group, query half of each tile
  int bk, rank;
  bwd_tile_of(p.B * p.Hkv, bk, rank);  // key block 0 sees the most queries under a causal band
  const int kblk = rank / g.kv_parts, part = rank % g.kv_parts;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int k0 = kblk * 128;
  const int jw = k0 + 32 * kw;  // the wave's first key
  const int j = jw + lq;        // the lane's key (result column)
  const int jwl = min(jw + 31, p.Nk - 1);
  const __bf16* kblk_s = smem;
  const __bf16* vblk_s = smem + BLK;
  __bf16* tiles = smem + 2 * BLK;

  {  // K' and V rows of the block (clamped to Nk - 1) into LDS
    const __bf16* kb = g.kr + b * g.kr_sb + kvh * g.kr_sh;
    const __bf16* vb = reinterpret_cast<const __bf16*>(p.v) + b * p.vsb + kvh * p.vsh;
    RowStage<D, 128, kKvThreads> ks, vs;
    ks.load(kb, g.kr_sn, k0, p.Nk);
    vs.load(vb, p.vsn, k0, p.Nk);
    ks.store(smem);
    vs.store(smem + BLK);
  }
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

  // (head, query tile) steps: the group's q-heads one after the other, each
  // over the 64-row query tiles the band allows; this workgroup's part of them.
  const int qt0 = (i_lo / 64) * 64;
  const int ntq = i_hi >= i_lo ? (i_hi - qt0) / 64 + 1 : 0;
  const int t_begin = (int)((long long)part * ntq * p.G / g.kv_parts);
  const int t_end = (int)((long long)(part + 1) * ntq * p.G / g.kv_parts);
  // A step's Q' and dO tiles (64 rows each) go global -> LDS by direct DMA;
  // the lse and delta of its rows go through registers (64 threads) into the
  // stat area.
  float st_l2 = 0.f, st_delta = 0.f;
  auto dma_step = [&](int t, int buf) {
    const int h = kvh * p.G + t / ntq, q0 = qt0 + 64 * (t % ntq);
    const uint32_t t_lds = lds_addr(tiles + buf * 2 * TILE);
    dma_tile64<D, kKvThreads / 64>(t_lds, g.qr + b * g.qr_sb + h * g.qr_sh, g.qr_sn, q0, p.Nq);
    dma_tile64<D, kKvThreads / 64>(t_lds + TILE * 2, g.dout + b * p.osb + h * p.osh, p.osn, q0, p.Nq);
    if (threadIdx.x < 64) {
      const int ii = q0 + (int)threadIdx.x;
      const long long rr = ((long long)b * p.Hq + h) * p.Nq + min(ii, p.Nq - 1);
      const float l = p.lse[rr];
      st_l2 = (ii < p.Nq && l != -INFINITY) ? l * kLog2e : INFINITY;
      st_delta = g.delta[rr];
    }
  };
  auto store_stat = [&](int buf) {
    if (threadIdx.x < 64) {
      stat[buf][0][threadIdx.x] = st_l2;
      stat[buf][1][threadIdx.x] = st_delta;
    }
  };
  // With a block mask a step is visited only when its CSR row lists one of
  // the workgroup's key blocks (bit 0: the block of key k0, bit 1: the block
  // of the last key; the same block sets both), and a wave computes only when
  // its own key block is listed.  Dense steps are all visited.
  // The masks of up to kMaxSparseSteps steps are found by all threads at once
  // (one CSR row scan each) and kept in LDS; longer step ranges scan a row
  // per step.
  const int kb_lo = SPARSE ? k0 / p.bn : 0, kb_hi = SPARSE ? k_last / p.bn : 0;
  const int wbit = (SPARSE && jw / p.bn != kb_lo) ? 2 : 1;
  auto vis_scan = [&](int t) -> int {
    const int h = kvh * p.G + t / ntq, q0 = qt0 + 64 * (t % ntq);
    const int* rp = p.row_ptr + (p.bs_head_stride ? (long long)h * p.bs_head_stride : 0);
    const int qb = q0 / p.bm, nkb = (p.Nk + p.bn - 1) / p.bn;
    const long long a = min(max((long long)rp[qb], 0LL), p.bs_nnz);
    const long long e = min(max((long long)rp[qb + 1], a), p.bs_nnz);
    int m = 0;
    for (long long x = a; x < e; ++x) {
      const int c = min(max(p.col_idx[x], 0), nkb);
      m |= (c == kb_lo ? 1 : 0) | (c == kb_hi ? 2 : 0);
    }
    return m;
  };
  __shared__ uint8_t vis_s[SPARSE ? kMaxSparseSteps : 1];
  const bool vis_in_lds = SPARSE && t_end - t_begin <= kMaxSparseSteps;
  if (vis_in_lds) {
    for (int t = t_begin + (int)threadIdx.x; t < t_end; t += kKvThreads) vis_s[t - t_begin] = (uint8_t)vis_scan(t);
    __syncthreads();
  }
  auto vis = [&](int t) -> int {
    if (!SPARSE) return 3;
    if (vis_in_lds) return __builtin_amdgcn_readfirstlane((int)vis_s[t - t_begin]);
    return __builtin_amdgcn_readfirstlane(vis_scan(t));
  };
  auto next_vis = [&](int t) {
    if (SPARSE)
      while (t < t_end && vis(t) == 0) ++t;
    return t;
  };
  int cur = next_vis(t_begin);
  int nxt = cur < t_end ? next_vis(cur + 1) : t_end;
  if (cur < t_end) {
    dma_step(cur, 0);
    store_stat(0);
    vmcnt_wait<0>();
  }
  __syncthreads();
  for (int buf = 0; cur < t_end; buf ^= 1) {
    // The next step's tiles go to the other buffer while this step runs
    // (that buffer was last read before the previous barrier).
    if (nxt < t_end) dma_step(nxt, buf ^ 1);
    const int t = cur;
    const int h = kvh * p.G + t / ntq, q0 = qt0 + 64 * (t % ntq);
    const __bf16* qs = tiles + buf * 2 * TILE;
    const __bf16* dos = qs + TILE;
    const uint32_t qs_lds = lds_addr(qs), dos_lds = lds_addr(dos);
    // The wave's keys jw .. jwl against query rows ia .. ib.
    const int ia = q0 + 32 * st, ib = min(ia + 31, p.Nq - 1);
    const bool skip = ia >= p.Nq || jw >= p.Nk ||
                      (p.has_band && (jwl - ia < p.band_lo || jw - ib > p.band_hi)) ||
                      (SPARSE && !(vis(t) & wbit));
    // S and dP (32 query rows x the wave's 32 keys; lane = key column),
    // alternating products; each product's two LDS operands are read PF
    // products ahead.
    f32x16 sa = f32x16{}, da = f32x16{};
    if (!skip) {
      constexpr int NS = 2 * NKK, PF = 2;
      auto a_frag = [&](int k) { return row_frag<D>((k & 1) ? dos : qs, 32 * st + lq, k >> 1); };
      auto b_frag = [&](int k) { return row_frag<D>((k & 1) ? vblk_s : kblk_s, 32 * kw + lq, k >> 1); };
      bf16x8 fa[PF + 1], fb[PF + 1];
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        fa[k] = a_frag(k);
        fb[k] = b_frag(k);
      }
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k + PF < NS) {
          fa[(k + PF) % (PF + 1)] = a_frag(k + PF);
          fb[(k + PF) % (PF + 1)] = b_frag(k + PF);
        }
        if (k & 1)
          da = mfma32(fa[k % (PF + 1)], fb[k % (PF + 1)], da);
        else
          sa = mfma32(fa[k % (PF + 1)], fb[k % (PF + 1)], sa);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!skip) {  // else P = dS = 0
      const bool full = ia + 31 < p.Nq && jw + 31 < p.Nk &&
                        (!p.has_band || (jw - (ia + 31) >= p.band_lo && jw + 31 - ia <= p.band_hi));
      const float slope2 = (SM & kSmAlibi) ? p.alibi[h] * kLog2e : 0.f;
      const float* bias_bh = (SM & kSmBias) ? p.bias + b * p.bsb + h * p.bsh : nullptr;
      // Per 16-row chunk: P and dS (bf16), then dV^T += dO^T P, dK'^T += Q'^T dS.
      auto chunk = [&](auto c_tag) {
        constexpr int c = decltype(c_tag)::value;
        float L2[16], Dl[16];  // only rows 8c .. 8c+7 are read
#pragma unroll
        for (int a4 = 2 * c; a4 < 2 * c + 2; ++a4) {
          const float4 l4 = *reinterpret_cast<const float4*>(&stat[buf][0][32 * st + 8 * a4 + 4 * lh]);
          const float4 d4 = *reinterpret_cast<const float4*>(&stat[buf][1][32 * st + 8 * a4 + 4 * lh]);
          L2[4 * a4] = l4.x; L2[4 * a4 + 1] = l4.y; L2[4 * a4 + 2] = l4.z; L2[4 * a4 + 3] = l4.w;
          Dl[4 * a4] = d4.x; Dl[4 * a4 + 1] = d4.y; Dl[4 * a4 + 2] = d4.z; Dl[4 * a4 + 3] = d4.w;
        }
        constexpr int NG = 2 * NDT, PF = 2;
        auto t_frag = [&](int k) { return tr_frag<D>((k & 1) ? qs_lds : dos_lds, 32 * st + 16 * c, 32 * (k >> 1)); };
        bf16x8 tf[PF + 1];
#pragma unroll
        for (int k = 0; k < PF; ++k) tf[k] = t_frag(k);
        bf16x8 pf[2], dsf[2];
        if (full)
          p_ds<false, SM, true, true, c, c + 1>(sa, da, L2, Dl, ia, j, p, slope2, dpos, bias_bh, pf, dsf);
        else
          p_ds<true, SM, true, true, c, c + 1>(sa, da, L2, Dl, ia, j, p, slope2, dpos, bias_bh, pf, dsf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NG; ++k) {
          if (k + PF < NG) tf[(k + PF) % (PF + 1)] = t_frag(k + PF);
          if (k & 1)
            dk[k >> 1] = mfma32(tf[k % (PF + 1)], dsf[c], dk[k >> 1]);
          else
            dv[k >> 1] = mfma32(tf[k % (PF + 1)], pf[c], dv[k >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      chunk(std::integral_constant<int, 0>{});
      chunk(std::integral_constant<int, 1>{});
    }
    if (nxt < t_end) store_stat(buf ^ 1);
    vmcnt_wait<0>();  // the next step's tiles have landed
    __syncthreads();
    cur = nxt;
    nxt = nxt < t_end ? next_vis(nxt + 1) : t_end;
  }
  // Waves 4..7 hand their sums to waves 0..3 (dK' in the tile area, dV in the
  // block area; every wave has passed the loop's last barrier).
  {
    float4* red_k = reinterpret_cast<float4*>(tiles) + kw * (NDT * 4 * 64);
    float4* red_v = reinterpret_cast<float4*>(smem) + kw * (NDT * 4 * 64);
    if (st == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          red_k[(dt * 4 + g4) * 64 + lane] =
              make_float4(dk[dt][4 * g4], dk[dt][4 * g4 + 1], dk[dt][4 * g4 + 2], dk[dt][4 * g4 + 3]);
          red_v[(dt * 4 + g4) * 64 + lane] =
              make_float4(dv[dt][4 * g4], dv[dt][4 * g4 + 1], dv[dt][4 * g4 + 2], dv[dt][4 * g4 + 3]);
        }
    }
    __syncthreads();
    if (st == 1) return;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 x = red_k[(dt * 4 + g4) * 64 + lane], y = red_v[(dt * 4 + g4) * 64 + lane];
        dk[dt][4 * g4] += x.x; dk[dt][4 * g4 + 1] += x.y; dk[dt][4 * g4 + 2] += x.z; dk[dt][4 * g4 + 3] += x.w;
        dv[dt][4 * g4] += y.x; dv[dt][4 * g4 + 1] += y.y; dv[dt][4 * g4 + 2] += y.z; dv[dt][4 * g4 + 3] += y.w;
      }
  }
  if (j < p.Nk) {
    if (g.kv_parts == 1) {
      __bf16* dkd = g.dk + b * p.ksb + kvh * p.ksh + (long long)j * p.ksn;
      __bf16* dvd = g.dv + b * p.vsb + kvh * p.vsh + (long long)j * p.vsn;
      store_grad_row<D>(dkd, dk, p.scale_log2 / kLog2e, p.rcos != nullptr, p, p.k_pos0 + j);
      store_grad_row<D>(dvd, dv, 1.f, false, p, 0);
    } else {
      const long long rows_k = (long long)p.B * p.Hkv * p.Nk;
      const long long krow = ((long long)b * p.Hkv + kvh) * p.Nk + j;
      store_part_row<D>(g.kv_part + ((2LL * part) * rows_k + krow) * D, dk);
      store_part_row<D>(g.kv_part + ((2LL * part + 1) * rows_k + krow) * D, dv);
    }
  }
}

// ---- pass 2b (kv_parts > 1): dK = scale * RoPE^-1(sum of the dK' parts), dV = sum ----
template <int D>
__global__ void __launch_bounds__(256) bwd_kv_reduce_kernel(const AttnParams p, const BwdParams g) {
  constexpr int CH = D / 16;  // chunk pairs per row
  const long long rows_k = (long long)p.B * p.Hkv * p.Nk;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows_k * CH) return;
  const int c = (int)(idx % CH);
  const long long row = idx / CH;
  const int j = (int)(row % p.Nk);
  const long long bh = row / p.Nk;
  const int kvh = (int)(bh % p.Hkv), b = (int)(bh / p.Hkv);
  float k_lo[8] = {}, k_hi[8] = {}, v_lo[8] = {}, v_hi[8] = {};
  for (int part = 0; part < g.kv_parts; ++part) {
    const float* pk = g.kv_part + ((2LL * part) * rows_k + row) * D;
    const float* pv = g.kv_part + ((2LL * part + 1) * rows_k + row) * D;
    const F8 a = ld_f8(pk + 8 * c), bb = ld_f8(pk + D / 2 + 8 * c);
    const F8 x = ld_f8(pv + 8 * c), y = ld_f8(pv + D / 2 + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      k_lo[e] += f8_at(a, e);
      k_hi[e] += f8_at(bb, e);
      v_lo[e] += f8_at(x, e);
      v_hi[e] += f8_at(y, e);
    }
  }
  const float scale = p.scale_log2 / kLog2e;
  if (p.rcos) {
    const long long t = (long long)min(p.k_pos0 + j, p.rope_len - 1) * (D / 2) + 8 * c;
    const F8 cs = ld_f8(p.rcos + t), sn = ld_f8(p.rsin + t);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float co = f8_at(cs, e), si = f8_at(sn, e), lo = k_lo[e], hi = k_hi[e];
      k_lo[e] = lo * co + hi * si;
      k_hi[e] = hi * co - lo * si;
    }
  }
  uint32_t wk0[4], wk1[4], wv0[4], wv1[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wk0[w] = pack_bf16x2(scale * k_lo[2 * w], scale * k_lo[2 * w + 1]);
    wk1[w] = pack_bf16x2(scale * k_hi[2 * w], scale * k_hi[2 * w + 1]);
    wv0[w] = pack_bf16x2(v_lo[2 * w], v_lo[2 * w + 1]);
    wv1[w] = pack_bf16x2(v_hi[2 * w], v_hi[2 * w + 1]);
  }
  __bf16* dkd = g.dk + b * p.ksb + kvh * p.ksh + (long long)j * p.ksn;
  __bf16* dvd = g.dv + b * p.vsb + kvh * p.vsh + (long long)j * p.vsn;
  st16(dkd + 8 * c, make_uint4(wk0[0], wk0[1], wk0[2], wk0[3]));
  st16(dkd + D / 2 + 8 * c, make_uint4(wk1[0], wk1[1], wk1[2], wk1[3]));
  st16(dvd + 8 * c, make_uint4(wv0[0], wv0[1], wv0[2], wv0[3]));
  st16(dvd + D / 2 + 8 * c, make_uint4(wv1[0], wv1[1], wv1[2], wv1[3]));
}

template <int D, int SM>
static void launch_bwd_main(const AttnParams& p, const BwdParams& g, unsigned grid_k,
                            hipStream_t stream) {
  const bool sparse = p.row_ptr != nullptr;
  const int rows_q = sparse ? 64 : kDqRows;
  const unsigned grid_q = (unsigned)((long long)p.B * p.Hq * ((p.Nq + rows_q - 1) / rows_q));
  if (grid_k > 0) {
    if (sparse)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, SM, true>), dim3(grid_k), dim3(kKvThreads), 0, stream, p, g);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, SM, false>), dim3(grid_k), dim3(kKvThreads), 0, stream, p, g);
  }
  if (grid_q > 0) {
    if (sparse)
      hipLaunchKernelGGL((bwd_dq_kernel<D, SM, true>), dim3(grid_q), dim3(128), 0, stream, p, g);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, SM, false>), dim3(grid_q), dim3(kDqThreads), 0, stream, p, g);
  }
}

template <int D>
static hipError_t launch_bwd_d(const AttnParams& p, const BwdParams& g, hipStream_t stream) {
  const long long rows_q = (long long)p.B * p.Hq * p.Nq;
  const long long rows_k = (long long)p.B * p.Hkv * p.Nk;
  constexpr int CH = D / 16;
  if (g.qrot && rows_q > 0)
    hipLaunchKernelGGL(bwd_rotate_kernel<D>, dim3((unsigned)((rows_q * CH + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<const __bf16*>(p.q), p.qsb, p.qsh, p.qsn, p.Hq, p.Nq,
                       rows_q, p.q_pos0, p, g.qrot);
  if (g.krot && rows_k > 0)
    hipLaunchKernelGGL(bwd_rotate_kernel<D>, dim3((unsigned)((rows_k * CH + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<const __bf16*>(p.k), p.ksb, p.ksh, p.ksn, p.Hkv, p.Nk,
                       rows_k, p.k_pos0, p, g.krot);
  constexpr int rpb = 256 / (D / 8);
  if (rows_q > 0)
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((rows_q + rpb - 1) / rpb)), dim3(256), 0,
                       stream, p, g);
  const unsigned grid_k = (unsigned)((long long)p.B * p.Hkv * ((p.Nk + 127) / 128) * g.kv_parts);
  const int sm = (p.alibi ? kSmAlibi : 0) | (p.bias ? kSmBias : 0);
  if (sm == 0) launch_bwd_main<D, 0>(p, g, grid_k, stream);
  else if (sm == kSmAlibi) launch_bwd_main<D, kSmAlibi>(p, g, grid_k, stream);
  else if (sm == kSmBias) launch_bwd_main<D, kSmBias>(p, g, grid_k, stream);
  else launch_bwd_main<D, kSmAlibi | kSmBias>(p, g, grid_k, stream);
  if (g.kv_parts > 1 && rows_k > 0)
    hipLaunchKernelGGL(bwd_kv_reduce_kernel<D>, dim3((unsigned)((rows_k * CH + 255) / 256)), dim3(256), 0,
                       stream, p, g);
  return hipGetLastError();
}

}  // namespace attnfuse
