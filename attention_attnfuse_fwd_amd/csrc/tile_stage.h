// Cooperative K/V tile staging: global -> registers -> (RoPE) -> LDS.
//
// A tile is BN consecutive keys of one kv-head.  K goes to LDS row-major
// ([BN][D + 8], rotated when ROPE), V goes transposed ([D][BN + 8], key
// columns permuted by vcol()).  The load*() calls only issue global loads, so
// a kernel can call them a tile (or two) ahead and hide their latency behind
// MFMA work; store() then rotates and writes LDS.  With KV8 the cache holds
// OCP FP8 E4M3 codes: half the bytes are loaded, and store() converts them
// to bf16 exactly (every E4M3 value is a bf16 value) before the rotation.
#pragma once

#include <type_traits>

#include "common.h"

namespace attnfuse {

// K part: unit = (key j, 8-wide chunk c of the low half) covering d in
// [8c, 8c + 8) and its RoPE partner [D/2 + 8c, D/2 + 8c + 8).  Consecutive
// units walk the chunks of one row (coalesced 16-byte loads); the row order
// within each block of 16 keys is permuted so that the rows a 16-lane group
// stores together sit CPR rows apart, which puts their 16-byte chunks on
// disjoint LDS banks (the row stride is D + 8 elements).
template <int D, int BN, int NT, bool ROPE, bool KV8 = false>
struct KStage {
  using T = typename std::conditional<KV8, uint8_t, __bf16>::type;  // cache element
  static constexpr int KSTR = D + 8;
  static constexpr int CPR = D / 16;                 // chunk pairs per row
  static constexpr int UNITS = BN * CPR;
  static constexpr int U = (UNITS + NT - 1) / NT;
  static constexpr int RPG = 16 / CPR;               // rows per 16-lane group

  __device__ __forceinline__ static int row_of(int unit) {
    const int jr = unit / CPR;
    const int jl = jr & 15;
    return (jr & ~15) | ((jl % RPG) * CPR + jl / RPG);
  }

  static_assert(NT % CPR == 0, "a lane keeps one chunk column for all its units");

  uint4 lo[KV8 ? 1 : U], hi[KV8 ? 1 : U];      // bf16 rows
  uint2 lo8[KV8 ? U : 1], hi8[KV8 ? U : 1];    // fp8 rows
  // Angles by addition: the key at position base + j (base = the step's
  // first key, 0 <= j < BN) is rotated by base * w + j * w, so only the
  // step's base row of the table is read (fp16 (cos, sin) pairs of the
  // lane's 8 angles); the small angles j * w come from the hardware sine and
  // cosine (|j * w| / 2 pi < BN / 2 pi revolutions) with w computed once.
  uint4 cb[2];     // table row `base`
  float wrev0;     // w / (2 pi) of the lane's first frequency, r = 8 * (tid % CPR)
  float ratio;     // w_{r+1} / w_r = theta^(-2/D) (the same for every lane)
  int base;

  // The lane's frequencies w_r = theta^(-2r/D), r = 8 * (tid % CPR) + e,
  // as wrev0 * ratio^e.
  __device__ __forceinline__ void init(const AttnParams& p, int tid) {
    if (!ROPE) return;
    const int c = tid % CPR;
    wrev0 = exp2f(-2.0f * (float)(8 * c) / (float)D * p.rope_log2_theta) * 0.15915494309189535f;
    ratio = exp2f(-2.0f / (float)D * p.rope_log2_theta);
  }

  // Raw K rows k0 .. k0+BN-1 (rows at or past key_end are clamped to key_end - 1).
  __device__ __forceinline__ void load(const AttnParams& p, const T* kb, int k0, int key_end,
                                       int tid) {
    base = p.k_pos0 + k0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int j = row_of(unit), c = unit % CPR;
        const int kj = min(k0 + j, key_end - 1);
        const T* src = kb + (long long)kj * p.ksn + 8 * c;
        if constexpr (KV8) {
          lo8[u] = ld8_stream(src);
          hi8[u] = ld8_stream(src + D / 2);
        } else {
          lo[u] = ld16_stream(src);
          hi[u] = ld16_stream(src + D / 2);
        }
      }
    }
  }
  // (cos, sin) table entries of the step's base row (rows clamped at the end
  // of the keys are masked out, so they take angle base + j as well).
  __device__ __forceinline__ void load_tables(const AttnParams& p, int tid) {
    if (!ROPE) return;
    const uint32_t* brow = p.rcs + (long long)base * (D / 2) + 8 * (tid % CPR);
    cb[0] = ld16(brow);
    cb[1] = ld16(brow + 4);
  }
  __device__ __forceinline__ void store(__bf16* ks, int tid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int j = row_of(unit), c = unit % CPR;
        uint4 l, h;
        if constexpr (KV8) {
          l = e4m3x8_to_bf16x8(lo8[u]);
          h = e4m3x8_to_bf16x8(hi8[u]);
        } else {
          l = lo[u];
          h = hi[u];
        }
        if (ROPE) rope_rotate_bf16x8_step(l, h, cb[0], cb[1], wrev0, ratio, (float)j);
        st16(ks + j * KSTR + 8 * c, l);
        st16(ks + j * KSTR + D / 2 + 8 * c, h);
      }
    }
  }
};

// V part: unit = (run of 4 keys, 8-wide d chunk); stored transposed.  Runs
// vary fastest across lanes, so the 8-byte writes a 16-lane group issues for
// one d row land side by side in that row (no bank conflicts); each load
// instruction still reads 64-byte pieces of 16 key rows.
template <int D, int BN, int NT, bool KV8 = false>
struct VStage {
  using T = typename std::conditional<KV8, uint8_t, __bf16>::type;  // cache element
  static constexpr int VSTR = BN + 8;
  static constexpr int RUNS = BN / 4;
  static constexpr int UNITS = RUNS * (D / 8);
  static constexpr int U = (UNITS + NT - 1) / NT;

  uint4 v[KV8 ? 1 : U][4];    // bf16 rows
  uint2 v8[KV8 ? U : 1][4];   // fp8 rows

  __device__ __forceinline__ void load(const AttnParams& p, const T* vb, int k0, int key_end,
                                       int tid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int run = unit % RUNS, dc = unit / RUNS;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int kj = min(k0 + 4 * run + b, key_end - 1);
          const T* src = vb + (long long)kj * p.vsn + 8 * dc;
          if constexpr (KV8) v8[u][b] = ld8_stream(src);
          else v[u][b] = ld16_stream(src);
        }
      }
    }
  }
  __device__ __forceinline__ void store(__bf16* vs, int tid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int unit = tid + u * NT;
      if (UNITS % NT == 0 || unit < UNITS) {
        const int run = unit % RUNS, dc = unit / RUNS;
        if constexpr (KV8) {
          uint4 w[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) w[b] = e4m3x8_to_bf16x8(v8[u][b]);
          store_vt_4x8(vs + (8 * dc) * VSTR + vcol(4 * run), VSTR, w);
        } else {
          store_vt_4x8(vs + (8 * dc) * VSTR + vcol(4 * run), VSTR, v[u]);
        }
      }
    }
  }
};

// Both parts for one tile (used where K and V of the same tile move together).
template <int D, int BN, int NT, bool ROPE>
struct TileStage {
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = BN + 8;
  static constexpr int KBUF = BN * KSTR;
  KStage<D, BN, NT, ROPE> k;
  VStage<D, BN, NT> v;

  __device__ __forceinline__ void load(const AttnParams& p, const __bf16* kb, const __bf16* vb,
                                       int k0, int key_end, int tid) {
    k.load(p, kb, k0, key_end, tid);
    k.load_tables(p, tid);
    v.load(p, vb, k0, key_end, tid);
  }
  __device__ __forceinline__ void store(__bf16* slot, int tid) {
    k.store(slot, tid);
    v.store(slot + KBUF, tid);
  }
};

}  // namespace attnfuse
