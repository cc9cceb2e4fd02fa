// Cooperative K/V tile staging: global -> registers -> (RoPE) -> LDS.
//
// A tile is BN consecutive keys of one kv-head.  K goes to LDS row-major
// ([BN][D + 8], rotated when ROPE), V goes transposed ([D][BN + 8], key
// columns permuted by vcol()).  load() only issues the global loads, so a
// kernel can call it one tile ahead and hide their latency behind the
// current tile's MFMA work; store() then rotates and writes LDS.
#pragma once

#include "common.h"

namespace attnfuse {

template <int D, int BN, int NT, bool ROPE>
struct TileStage {
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = BN + 8;
  static constexpr int KBUF = BN * KSTR;
  static constexpr int KUNITS = BN * (D / 16);       // (key, chunk pair d / d + D/2)
  static constexpr int KU = (KUNITS + NT - 1) / NT;
  static constexpr int VUNITS = (BN / 4) * (D / 8);  // (4-key run, 8-wide d chunk)
  static constexpr int VU = (VUNITS + NT - 1) / NT;

  uint4 klo[KU], khi[KU];
  F8 cs[KU], sn[KU];
  uint4 v[VU][4];

  // Keys k0 .. k0+BN-1 (rows past key_end - 1 are clamped to key_end - 1;
  // they are masked by the caller).
  __device__ __forceinline__ void load(const AttnParams& p, const __bf16* kb, const __bf16* vb,
                                       int k0, int key_end, int tid) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * NT;
      if (KUNITS % NT == 0 || unit < KUNITS) {
        const int j = unit / (D / 16), c = unit % (D / 16);
        const int kj = min(k0 + j, key_end - 1);
        const __bf16* src = kb + (long long)kj * p.ksn + 8 * c;
        klo[u] = ld16(src);
        khi[u] = ld16(src + D / 2);
        if (ROPE) {
          const long long row = (long long)(p.k_pos0 + kj) * (D / 2) + 8 * c;
          cs[u] = ld_f8(p.rcos + row);
          sn[u] = ld_f8(p.rsin + row);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = tid + u * NT;
      if (VUNITS % NT == 0 || unit < VUNITS) {
        const int run = unit / (D / 8), dc = unit % (D / 8);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int kj = min(k0 + 4 * run + b, key_end - 1);
          v[u][b] = ld16(vb + (long long)kj * p.vsn + 8 * dc);
        }
      }
    }
  }

  __device__ __forceinline__ void store(__bf16* slot, int tid) {
    __bf16* ks = slot;
    __bf16* vs = slot + KBUF;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int unit = tid + u * NT;
      if (KUNITS % NT == 0 || unit < KUNITS) {
        const int j = unit / (D / 16), c = unit % (D / 16);
        uint4 lo = klo[u], hi = khi[u];
        if (ROPE) rope_rotate_bf16x8(lo, hi, cs[u], sn[u]);
        st16(ks + j * KSTR + 8 * c, lo);
        st16(ks + j * KSTR + D / 2 + 8 * c, hi);
      }
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int unit = tid + u * NT;
      if (VUNITS % NT == 0 || unit < VUNITS) {
        const int run = unit / (D / 8), dc = unit % (D / 8);
        store_vt_4x8(vs + (8 * dc) * VSTR + vcol(4 * run), VSTR, v[u]);
      }
    }
  }
};

}  // namespace attnfuse
