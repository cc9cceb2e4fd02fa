// Device-side building blocks shared by the gfx950 attention kernels.
//
// Fragment conventions (CDNA4 v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (32 x 16, row-major M x K): lane l holds row l % 32, K elements
//     8 * (l / 32) .. 8 * (l / 32) + 7.
//   B operand (16 x 32, K x N):           lane l holds column l % 32, K elements
//     8 * (l / 32) .. + 7.
//   C / D (32 x 32 fp32, 16 registers):   lane l, register r holds row
//     8 * (r / 4) + 4 * (l / 32) + (r % 4), column l % 32.
// The attention kernels compute S^T = K' . Q'^T (keys on rows, queries on
// columns) so that a lane owns one query column: the row-wise softmax then
// reduces in-lane plus one swap with lane l ^ 32, and the probability tile
// P^T is already the B operand of O^T += V^T . P^T with no data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfuse {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBandInf = 1 << 30;  // "unbounded" band edge in index space

// Kernel parameters (host fills, passed by value).
// bf16 prefill kernel shapes shared by the kernel and the host's launch
// model.  The two-wave block-sparse instance at D = 64 (no additive bias)
// keeps two-slot K and V rings (40 KB of LDS with the RoPE table slot), so
// four workgroups, two waves per SIMD, share a CU; the other instances keep
// four-slot rings.
constexpr bool fwd_bf16_shallow(int D, int NW, bool sparse, bool bias) {
  return D == 64 && NW == 2 && sparse && !bias;
}
// LDS bytes of a bf16 prefill workgroup (not the fp8 instances): K and V
// rings of 64-key slots, the RoPE table slot, and for eight waves one more
// Q staging area.
constexpr int fwd_bf16_lds_bytes(int D, int NW, bool rope, bool sparse, bool bias) {
  return 2 * (fwd_bf16_shallow(D, NW, sparse, bias) ? 2 : 4) * 128 * D + (rope ? (D / 16) * 2048 : 0) +
         (NW == 8 ? 128 * D : 0);
}

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, Hq, Hkv, Nq, Nk, G;  // G = Hq / Hkv
  long long qsb, qsh, qsn;
  long long ksb, ksh, ksn;
  long long vsb, vsh, vsn;
  long long osb, osh, osn;
  float scale_log2;           // softmax scale times log2(e)
  const float* rcos;          // fp32 RoPE tables [len][D/2] (fp32 kernels) or nullptr
  const float* rsin;
  const uint32_t* rcs;        // fp16 (cos, sin) pairs [len][D/2] (decode) or nullptr
  int rope_len;               // rows in the RoPE tables
  float rope_log2_theta;      // log2 of the RoPE base (decode's small angles)
  int q_pos0, k_pos0;
  // Allowed iff band_lo <= j - i <= band_hi (row/column index space; the
  // position offset k_pos0 - q_pos0 is already folded in).  has_band = 0
  // skips the test.
  int has_band, band_lo, band_hi;
  const float* alibi;         // slopes [Hq] or nullptr
  const float* bias;          // fp32 bias or nullptr
  long long bsb, bsh, bsi, bsj;
  const int* row_ptr;         // CSR block mask or nullptr
  const int* col_idx;
  int bm, bn;
  long long bs_head_stride, bs_nnz;
  float* lse;                 // [B, Hq, Nq] or nullptr
  // prefill grid decomposition
  int hp;                     // q-heads per workgroup
  int n_units;                // B * Hkv * (G / hp)
  int n_qblk;                 // query blocks per unit
  int longest_first;          // schedule later (longer) query blocks first
  // Paired workgroups (causal, dense, eight waves): workgroup j of a unit runs
  // query block n_qblk - 1 - j and then block j, as one stream of key tiles.
  int pair;
  // Chained workgroups (block-sparse, two- and four-wave kernels): workgroup
  // j of a unit runs query blocks chain * j .. chain * j + chain - 1 (those
  // that exist) as one stream of key tiles; 1 = one block per workgroup.
  int chain;
  // split-KV decode
  int splits, chunk, n_hgrp;
  float* ws;
  float v_scale;              // output multiplier (fp8 V cache dequantisation; 1 otherwise)
};

// Backward pass buffers (the kernels read the forward's q, k, v, out, lse
// and strides from AttnParams).
struct BwdParams {
  const __bf16* dout;  // [B, Hq, Nq, D], strides of out
  float* delta;        // [B, Hq, Nq] rowsum(dO * O), workspace
  __bf16* dq;          // strides of q
  __bf16* dk;          // strides of k
  __bf16* dv;          // strides of v
  // Q and K as the products read them (element strides of batch, head, row):
  // the rotated copies qrot / krot when RoPE is on, else q and k themselves.
  const __bf16* qr;
  const __bf16* kr;
  long long qr_sb, qr_sh, qr_sn, kr_sb, kr_sh, kr_sn;
  __bf16* qrot;        // [B, Hq, Nq, D] contiguous workspace, or nullptr
  __bf16* krot;        // [B, Hkv, Nk, D] contiguous workspace, or nullptr
  // kv_parts > 1: each (kv-head, key block) is split over kv_parts workgroups
  // that write fp32 partial sums [part][dK', dV][B * Hkv * Nk][D] to kv_part.
  int kv_parts;
  float* kv_part;
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float partner32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Eight FP8 E4M3 codes (bytes of x, in order) -> eight bf16 values, exact
// (every E4M3 value is a bf16 value; gfx950 conversion with a unit scale).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 x) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// S += A B on the fp8 matrix core (v_mfma_f32_32x32x64_f8f6f4, both operands
// OCP E4M3, unit block scales, fp32 accumulate).  Lane l holds row (A) /
// column (B) l % 32 and 32 of the 64 k values; the k values of lane-half g
// of A meet those of lane-half g of B, so any split of k into the two
// halves' 32 bytes gives the product as long as both operands use it.
__device__ __forceinline__ f32x16 mfma32_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Streaming loads (non-temporal hint): data read once, such as a decode's
// KV cache, should not displace what the caches hold for reuse.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8_stream(const void* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 8 consecutive fp32 values (two 16-byte loads).
struct F8 {
  float4 a, b;
};
__device__ __forceinline__ F8 ld_f8(const float* p) {
  F8 r;
  r.a = *reinterpret_cast<const float4*>(p);
  r.b = *reinterpret_cast<const float4*>(p + 4);
  return r;
}
__device__ __forceinline__ float f8_at(const F8& f, int e) {
  switch (e) {
    case 0: return f.a.x; case 1: return f.a.y; case 2: return f.a.z; case 3: return f.a.w;
    case 4: return f.b.x; case 5: return f.b.y; case 6: return f.b.z; default: return f.b.w;
  }
}

// NeoX rotation of one (low, high) pair of 8-element bf16 chunks, times k:
//   lo' = k (lo * c - hi * s),  hi' = k (hi * c + lo * s)
// (fp32 math, one bf16 rounding of the result).
__device__ __forceinline__ void rope_rotate_bf16x8(uint4& lo, uint4& hi, const F8& c, const F8& s,
                                                   float k = 1.f) {
  const uint32_t* wl = reinterpret_cast<const uint32_t*>(&lo);
  const uint32_t* wh = reinterpret_cast<const uint32_t*>(&hi);
  uint32_t ol[4], oh[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float l0 = bf16lo(wl[w]), l1 = bf16hi(wl[w]);
    const float h0 = bf16lo(wh[w]), h1 = bf16hi(wh[w]);
    const float c0 = f8_at(c, 2 * w) * k, c1 = f8_at(c, 2 * w + 1) * k;
    const float s0 = f8_at(s, 2 * w) * k, s1 = f8_at(s, 2 * w + 1) * k;
    ol[w] = pack_bf16x2(l0 * c0 - h0 * s0, l1 * c1 - h1 * s1);
    oh[w] = pack_bf16x2(h0 * c0 + l0 * s0, h1 * c1 + l1 * s1);
  }
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

// Eight bf16 values times k (fp32 product, one bf16 rounding).
__device__ __forceinline__ uint4 scale_bf16x8(const uint4& x, float k) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&x);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16lo(w[i]) * k, bf16hi(w[i]) * k);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// NeoX rotation of element e (0 or 1) of a bf16 word pair, with the angle
// given as an fp16 (cos, sin) word t (cos in the low half):
//   rl = l c - h s,  rh = h c + l s   (fp32 arithmetic on the exact bf16
// values).  wl / wh hold elements (2w, 2w+1) of the low / high half.  Each
// product reads its fp16 factor straight from a half of t (v_fma_mix_f32:
// the products are written as FMAs with a +0 addend, which the compiler
// cannot turn into plain multiplies), so the table needs no unpacking.  Plain
// VALU arithmetic: the bf16 dot-product instructions would queue behind the
// matrix core, which the partner wave keeps busy.
__device__ __forceinline__ void rope_elem(uint32_t wl, uint32_t wh, int e, uint32_t t, float& rl,
                                          float& rh) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const float l = e ? bf16hi(wl) : bf16lo(wl);
  const float h = e ? bf16hi(wh) : bf16lo(wh);
  const h2_t a = __builtin_bit_cast(h2_t, t);
  const float c = (float)a[0], s = (float)a[1];
  const float hs = __builtin_fmaf(h, s, 0.0f), ls = __builtin_fmaf(l, s, 0.0f);
  rl = __builtin_fmaf(l, c, -hs);
  rh = __builtin_fmaf(h, c, ls);
}

// Rotation of one (low, high) pair of 8-element bf16 chunks with fp16
// (cos, sin) words t0 (elements 0-3) and t1 (elements 4-7).
__device__ __forceinline__ void rope_rotate_bf16x8_t(uint4& lo, uint4& hi, const uint4& t0,
                                                     const uint4& t1) {
  const uint32_t tw[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
  const uint32_t* wl = reinterpret_cast<const uint32_t*>(&lo);
  const uint32_t* wh = reinterpret_cast<const uint32_t*>(&hi);
  uint32_t ol[4], oh[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float l0, h0, l1, h1;
    rope_elem(wl[w], wh[w], 0, tw[2 * w], l0, h0);
    rope_elem(wl[w], wh[w], 1, tw[2 * w + 1], l1, h1);
    ol[w] = pack_bf16x2(l0, l1);
    oh[w] = pack_bf16x2(h0, h1);
  }
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// NeoX rotation of one (low, high) pair of 8-element bf16 chunks, times k,
// with the angles' (cos, sin) given as fp16 pairs (one 32-bit word per angle,
// cos in the low half): fp32 math, bf16 result.
__device__ __forceinline__ void rope_rotate_bf16x8_h(uint4& lo, uint4& hi, const uint4& cs0,
                                                     const uint4& cs1, float k = 1.f) {
  const uint32_t cw[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
  const uint32_t* wl = reinterpret_cast<const uint32_t*>(&lo);
  const uint32_t* wh = reinterpret_cast<const uint32_t*>(&hi);
  uint32_t ol[4], oh[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float l0 = bf16lo(wl[w]), l1 = bf16hi(wl[w]);
    const float h0 = bf16lo(wh[w]), h1 = bf16hi(wh[w]);
    const f16x2 a = __builtin_bit_cast(f16x2, cw[2 * w]);
    const f16x2 b = __builtin_bit_cast(f16x2, cw[2 * w + 1]);
    const float c0 = (float)a[0] * k, s0 = (float)a[1] * k, c1 = (float)b[0] * k, s1 = (float)b[1] * k;
    ol[w] = pack_bf16x2(l0 * c0 - h0 * s0, l1 * c1 - h1 * s1);
    oh[w] = pack_bf16x2(h0 * c0 + l0 * s0, h1 * c1 + l1 * s1);
  }
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

// NeoX rotation of one (low, high) pair of 8-element bf16 chunks by the
// angles a_e + j * w_e, e = 0..7: fp16 (cos, sin) words of a_e (b0, b1),
// w_e / (2 pi) = wrev0 * ratio^e, and j small (|j * w_e| / (2 pi) a few
// revolutions: the hardware sine and cosine take revolutions).  cos(a + b) =
// cos a cos b - sin a sin b, sin(a + b) = sin a cos b + cos a sin b, all in
// fp32, then the rotation and one bf16 rounding.
__device__ __forceinline__ void rope_rotate_bf16x8_step(uint4& lo, uint4& hi, const uint4& b0,
                                                        const uint4& b1, float wrev0, float ratio,
                                                        float j) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  const uint32_t* wl = reinterpret_cast<const uint32_t*>(&lo);
  const uint32_t* wh = reinterpret_cast<const uint32_t*>(&hi);
  uint32_t ol[4], oh[4];
  float x = j * wrev0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float c[2], s[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * w + q;
      const h2_t a = __builtin_bit_cast(h2_t, bw[e]);
      const float ca = (float)a[0], sa = (float)a[1];
      if (e > 0) x *= ratio;
      // Loop-invariant across steps: keep the compiler from hoisting (and
      // holding) every step's sines and cosines in registers.
      asm volatile("" : "+v"(x));
      const float cbv = __builtin_amdgcn_cosf(x), sbv = __builtin_amdgcn_sinf(x);
      c[q] = __builtin_fmaf(ca, cbv, -sa * sbv);
      s[q] = __builtin_fmaf(sa, cbv, ca * sbv);
    }
    const float l0 = bf16lo(wl[w]), l1 = bf16hi(wl[w]);
    const float h0 = bf16lo(wh[w]), h1 = bf16hi(wh[w]);
    ol[w] = pack_bf16x2(__builtin_fmaf(l0, c[0], -h0 * s[0]), __builtin_fmaf(l1, c[1], -h1 * s[1]));
    oh[w] = pack_bf16x2(__builtin_fmaf(h0, c[0], l0 * s[0]), __builtin_fmaf(h1, c[1], l1 * s[1]));
  }
  lo = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  hi = make_uint4(oh[0], oh[1], oh[2], oh[3]);
}

// ---- direct global -> LDS staging (gfx950) ----

// Byte offset of a __shared__ object inside the workgroup's LDS allocation.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// Every lane moves 16 bytes from its own global address into LDS at
// lds_base + 16 * lane (lds_base must be wave-uniform).  The load completes
// asynchronously and is counted by vmcnt only; the compiler does not track
// it, so the caller orders it with vmcnt_wait() and barriers.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* g) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(g)
               : "memory", "m0");
}

// Same, with the global address split into a wave-uniform 64-bit base and a
// per-lane unsigned 32-bit byte offset (one VGPR instead of two).
__device__ __forceinline__ void dma16_off(uint32_t lds_base, const void* base, uint32_t off) {
  // base is wave-uniform by construction; readfirstlane keeps it in SGPRs
  // where the compiler cannot prove that itself.  (readfirstlane returns an
  // int: each half goes through uint32_t so that widening never sign-extends.)
  const uint64_t b64 = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(off), "s"(reinterpret_cast<const void*>(bs))
               : "memory", "m0");
}

// 16-byte LDS read at a byte address (constant parts of the address fold
// into the instruction's offset field).
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4*)(size_t)addr);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Issued through the builtin so
// the compiler's own wait bookkeeping sees it.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(N) (LDS / scalar-memory counter), vmcnt and expcnt
// untouched.
template <int N>
__device__ __forceinline__ void lgkmcnt_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is four bits");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte blocks that lanes 4e + i / 4 (e = 0..3) address, as
// its element e.  Pointed at four rows x 32 bytes of a row-major bf16 tile
// (lane 4a + b at row a, columns 4b .. 4b + 3), lane i gets column i of the
// four rows.
__device__ __forceinline__ i16x4 lds_read_tr4(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(size_t)addr);
}

// Column of key `k` (index within a tile) in the transposed V tile in LDS.
// Keys are stored with bits 2 and 3 of the index swapped, so that the 8
// probabilities a lane holds for one 16-key MFMA step (S^T accumulator rows
// 8*(r/4) + 4*(l/32) + r%4) meet 8 contiguous V^T elements.
__device__ __forceinline__ constexpr int vcol(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Transpose a 4-key x 8-d bf16 block (4 x uint4, one per key) into 8 rows of
// 4 keys (uint2 per d) and store row dd at dst + dd * row_stride (elements).
__device__ __forceinline__ void store_vt_4x8(__bf16* dst, int row_stride, const uint4 (&v)[4]) {
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint2 even = make_uint2(lo16x2(w0[w], w1[w]), lo16x2(w2[w], w3[w]));
    uint2 odd = make_uint2(hi16x2(w0[w], w1[w]), hi16x2(w2[w], w3[w]));
    *reinterpret_cast<uint2*>(dst + (2 * w) * row_stride) = even;
    *reinterpret_cast<uint2*>(dst + (2 * w + 1) * row_stride) = odd;
  }
}

}  // namespace attnfuse
