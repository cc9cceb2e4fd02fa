// C ABI of the fused attention library: descriptor validation, variant
// dispatch and launch.  Everything here runs on the host; validation touches
// no device memory and makes no HIP call, so every error return happens
// before any GPU work is enqueued.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attnfuse.h"
#include "launch.h"

using attnfuse::AttnParams;
using attnfuse::kBandInf;

namespace {

constexpr long long kMaxLen = 1LL << 30;
constexpr long long kMaxRowStride = 1LL << 24;  // Q / K / V row stride limit of the bf16 prefill (elements)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape, dtype, stride, position and mask checks shared by fwd and decode.
int validate_common(const attnfuse_variant_desc* d) {
  if (!d || d->struct_size != sizeof(attnfuse_variant_desc)) return ATTNFUSE_ERR_INVALID;
  if (d->dtype != ATTNFUSE_BF16 && d->dtype != ATTNFUSE_FP32) return ATTNFUSE_ERR_INVALID;
  if (d->norm == ATTNFUSE_NORM_RELU) return ATTNFUSE_ERR_UNSUPPORTED;
  if (d->norm != ATTNFUSE_NORM_SOFTMAX) return ATTNFUSE_ERR_INVALID;
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->Nq < 0 || d->Nk < 0 || d->D < 1)
    return ATTNFUSE_ERR_INVALID;
  if (d->Hq % d->Hkv) return ATTNFUSE_ERR_INVALID;
  if (d->D % 2) return ATTNFUSE_ERR_INVALID;
  if (d->D != 64 && d->D != 128) return ATTNFUSE_ERR_UNSUPPORTED;
  if (d->Nq >= kMaxLen || d->Nk >= kMaxLen) return ATTNFUSE_ERR_UNSUPPORTED;
  const int vec = d->dtype == ATTNFUSE_BF16 ? 8 : 4;  // elements per 16-byte access
  const int64_t* strides[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
  for (const int64_t* s : strides)
    for (int a = 0; a < 3; ++a) {
      if (s[a] < 0) return ATTNFUSE_ERR_INVALID;
      if (s[a] % vec) return ATTNFUSE_ERR_UNSUPPORTED;
    }
  if (!(d->scale >= 0.f) || !isfinite(d->scale)) return ATTNFUSE_ERR_INVALID;
  if (d->q_pos0 < 0 || d->k_pos0 < 0 || d->q_pos0 + d->Nq >= kMaxLen ||
      d->k_pos0 + d->Nk >= kMaxLen)
    return ATTNFUSE_ERR_INVALID;
  if (d->causal != 0 && d->causal != 1) return ATTNFUSE_ERR_INVALID;
  if (d->kv_fp8 != 0 && d->kv_fp8 != 1) return ATTNFUSE_ERR_INVALID;
  if (d->kv_fp8 && (!(d->k_scale > 0.f) || !isfinite(d->k_scale) || !(d->v_scale > 0.f) ||
                    !isfinite(d->v_scale)))
    return ATTNFUSE_ERR_INVALID;
  if (d->q_fp8 != 0 && d->q_fp8 != 1) return ATTNFUSE_ERR_INVALID;
  if (d->q_fp8 && (!(d->q_scale > 0.f) || !isfinite(d->q_scale))) return ATTNFUSE_ERR_INVALID;
  if (d->window < 0) return ATTNFUSE_ERR_INVALID;
  if (d->rope) {
    if (!(d->rope_theta > 0.0)) return ATTNFUSE_ERR_INVALID;
    const int64_t need = (d->q_pos0 + d->Nq > d->k_pos0 + d->Nk) ? d->q_pos0 + d->Nq
                                                                   : d->k_pos0 + d->Nk;
    if (d->rope_table_len < need || d->rope_table_len < 1) return ATTNFUSE_ERR_INVALID;
  }
  if (d->bias)
    for (int a = 0; a < 4; ++a)
      if (d->bias_stride[a] < 0) return ATTNFUSE_ERR_INVALID;
  if (d->bs_row_ptr) {
    if (d->bs_block_m < 1 || d->bs_block_n < 1 || d->bs_nnz < 0 || d->bs_head_stride < 0)
      return ATTNFUSE_ERR_INVALID;
    if (d->bs_nnz > 0 && !d->bs_col_idx) return ATTNFUSE_ERR_INVALID;
    const int64_t nqb = (d->Nq + d->bs_block_m - 1) / d->bs_block_m;
    if (d->bs_head_stride > 0 && d->bs_head_stride < nqb + 1) return ATTNFUSE_ERR_INVALID;
  }
  return ATTNFUSE_OK;
}

// RoPE tables each entry point reads: fp32 cos / sin for the fp32 prefill
// and the pre-rotation pass; fp16 pairs for the bf16 prefill (Q and K) and
// for decode.
bool fp32_tables_ok(const attnfuse_variant_desc* d) {
  return !d->rope || (d->rope_cos && d->rope_sin && aligned16(d->rope_cos) && aligned16(d->rope_sin));
}
bool f16_table_ok(const attnfuse_variant_desc* d) {
  return !d->rope || (d->rope_cs_f16 && aligned16(d->rope_cs_f16));
}

// Fill the kernel parameters that fwd and decode share.
AttnParams base_params(const void* q, const void* k, const void* v, void* out,
                       const attnfuse_variant_desc* d) {
  AttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = out;
  p.B = d->B;
  p.Hq = d->Hq;
  p.Hkv = d->Hkv;
  p.Nq = d->Nq;
  p.Nk = d->Nk;
  p.G = d->Hq / d->Hkv;
  p.qsb = d->q_stride[0]; p.qsh = d->q_stride[1]; p.qsn = d->q_stride[2];
  p.ksb = d->k_stride[0]; p.ksh = d->k_stride[1]; p.ksn = d->k_stride[2];
  p.vsb = d->v_stride[0]; p.vsh = d->v_stride[1]; p.vsn = d->v_stride[2];
  p.osb = d->o_stride[0]; p.osh = d->o_stride[1]; p.osn = d->o_stride[2];
  const double scale = d->scale > 0.f ? (double)d->scale : 1.0 / sqrt((double)d->D);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  p.v_scale = 1.f;
  p.rcos = d->rope ? d->rope_cos : nullptr;
  p.rsin = d->rope ? d->rope_sin : nullptr;
  p.rcs = d->rope ? d->rope_cs_f16 : nullptr;
  p.rope_len = d->rope ? (int)(d->rope_table_len < kMaxLen ? d->rope_table_len : kMaxLen) : 0;
  p.rope_log2_theta = d->rope ? (float)log2(d->rope_theta) : 0.f;
  p.q_pos0 = (int)d->q_pos0;
  p.k_pos0 = (int)d->k_pos0;
  // Band in position space: lo <= p_k - p_q <= hi; then shifted to index space.
  long long lo = -kBandInf, hi = kBandInf;
  if (d->causal) hi = 0;
  if (d->window > 0) {
    lo = -(long long)(d->window - 1);
    if (!d->causal) hi = d->window - 1;
  }
  p.has_band = (d->causal || d->window > 0) ? 1 : 0;
  const long long dpos = d->k_pos0 - d->q_pos0;
  auto clampb = [](long long x) {
    return (int)(x < -kBandInf ? -kBandInf : (x > kBandInf ? kBandInf : x));
  };
  p.band_lo = lo <= -kBandInf ? -kBandInf : clampb(lo - dpos);
  p.band_hi = hi >= kBandInf ? kBandInf : clampb(hi - dpos);
  p.alibi = d->alibi_slopes;
  p.bias = d->bias;
  p.bsb = d->bias_stride[0]; p.bsh = d->bias_stride[1];
  p.bsi = d->bias_stride[2]; p.bsj = d->bias_stride[3];
  p.row_ptr = d->bs_row_ptr;
  p.col_idx = d->bs_col_idx;
  p.bm = d->bs_block_m;
  p.bn = d->bs_block_n;
  p.bs_head_stride = d->bs_head_stride;
  p.bs_nnz = d->bs_nnz;
  p.lse = d->lse;
  p.chain = 1;
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTNFUSE_OK : ATTNFUSE_ERR_HIP; }

int largest_pow2_divisor(int g, int cap) {
  int hp = 1;
  while (hp * 2 <= cap && g % (hp * 2) == 0) hp *= 2;
  return hp;
}

// Causal dense attention: workgroup j of a unit runs query block
// n_qblk - 1 - j and then block j as one stream of key tiles, so half as
// many workgroups pay the start-up and drain of a block (without a window
// every workgroup also streams about n_qblk + 1 key tiles).  Needs the
// eight-wave schedule without an additive bias (ALiBi slopes are fine) and
// key tiles for every block (band_hi >= 0 for the first, the last block's
// band starting inside the keys).  Whether it pays depends on how the grid
// fills the CUs (one eight-wave workgroup per CU at a time): a time model
// in key tiles, with a fixed start-up and drain per workgroup, compares
// rounds of pairs against the unpaired blocks spread over the CUs (e.g.
// the GPT-2-small shape B4 H12 N4096 D64: 384 pairs are one and a half
// rounds, 15% slower than 768 single blocks; the Llama-3-8B shape: 256
// pairs, one round, faster).  Sets p.pair (and the longest-first block
// order the pairing uses) and returns the grid.
long long pair_blocks(AttnParams& p, const attnfuse_variant_desc* d, int rows, bool eight_waves,
                      bool sparse, long long grid) {
  constexpr long long kCUs = 256;     // MI355X compute units
  constexpr long long kFixed = 4;     // start-up + drain of a workgroup, in key tiles
  const long long n = p.n_qblk;
  const long long last_lo = (n - 1) * rows + p.band_lo;
  if (!eight_waves || sparse || d->bias != nullptr || !d->causal || d->Nk <= 0 || p.band_hi < 0 ||
      last_lo > d->Nk - 1 || n < 2)
    return grid;
  // Key tiles of query block j (the kernel's band range).
  auto tiles = [&](long long j) -> long long {
    const long long r0 = j * rows, rlast = std::min(r0 + rows, (long long)d->Nq) - 1;
    const long long lo = std::max(0LL, r0 + std::max((long long)p.band_lo, -(long long)kBandInf));
    const long long hi = std::min((long long)d->Nk - 1, rlast + p.band_hi);
    return hi >= lo ? hi / 64 - lo / 64 + 1 : 0;
  };
  long long sum = 0, longest = 0, longest_pair = 0;
  for (long long j = 0; j < n; ++j) {
    const long long t = tiles(j);
    sum += t;
    longest = std::max(longest, t);
    if (j < n - 1 - j) longest_pair = std::max(longest_pair, t + tiles(n - 1 - j));
  }
  const long long units = p.n_units, pairs = units * ((n + 1) / 2);
  const long long t_single = std::max((units * (sum + n * kFixed) + kCUs - 1) / kCUs, longest + kFixed);
  const long long t_paired = (pairs + kCUs - 1) / kCUs * (longest_pair + kFixed + 1);
  if (t_paired >= t_single) return grid;
  p.pair = 1;
  p.longest_first = 1;
  return pairs;
}

// Block-sparse chains: on the two- and four-wave kernels (few waves per
// SIMD, start-up and drain not hidden by a partner wave) a workgroup runs
// `chain` consecutive query blocks of its head as one stream of key tiles,
// when its rows are one CSR block row and there is no additive bias.  The
// library's choice: as many blocks per chain as the single blocks would take
// rounds of the CUs (workgroups per CU from the kernel's LDS), at most 8.
// E.g. the BigBird workload (B2 H16 N4096, 64-row blocks, two waves, the
// shallow schedule's 40 KB of LDS): 2048 blocks on 1024 workgroup slots,
// chains of 2.  Sets p.chain and the
// grid; returns a status (a requested chain where none can run is
// unsupported).
int chain_blocks(AttnParams& p, const attnfuse_variant_desc* d, int NW, int rows, bool sparse,
                 bool rope, long long& grid) {
  constexpr long long kCUs = 256;             // MI355X compute units
  constexpr long long kLdsPerCU = 160 * 1024;  // bytes
  const bool can = sparse && NW < 8 && d->bias == nullptr && d->bs_block_m == rows;
  // (A block mask with no keys launches the dense kernel: nothing to chain.)
  if (d->tile_chain > 1 && !can && !(d->bs_row_ptr && !sparse)) return ATTNFUSE_ERR_UNSUPPORTED;
  if (!can || d->tile_chain == 1) return ATTNFUSE_OK;
  long long c = d->tile_chain;
  if (c == 0) {
    const long long lds = attnfuse::fwd_bf16_lds_bytes(d->D, NW, rope, sparse, d->bias != nullptr);
    const long long slots = kCUs * std::max(1LL, kLdsPerCU / lds);
    c = std::min(8LL, grid / slots);
  }
  c = std::min(c, (long long)p.n_qblk);
  if (c <= 1) return ATTNFUSE_OK;
  p.chain = (int)c;
  grid = (long long)p.n_units * ((p.n_qblk + c - 1) / c);
  return ATTNFUSE_OK;
}

// Launch choice of attnfuse_fwd.
struct FwdPlan {
  int kind = ATTNFUSE_PLAN_NONE;
  int NW = 0, hp = 0, rows = 0;  // waves and q-heads per workgroup, query rows per block
  long long grid = 0;
};

// Validation and launch choice of attnfuse_fwd (kernel, tile, grid), shared
// with attnfuse_fwd_plan.  With have_ptrs false the data pointers are not
// examined.
int plan_fwd(const void* q, const void* k, const void* v, const void* out,
             const attnfuse_variant_desc* desc, bool have_ptrs, AttnParams& p, FwdPlan& f) {
  f = FwdPlan{};
  int st = validate_common(desc);
  if (st != ATTNFUSE_OK) return st;
  const attnfuse_variant_desc* d = desc;
  if (d->tile_chain < 0) return ATTNFUSE_ERR_INVALID;
  // fp8 inputs: Q, K and V together, with neither RoPE nor an additive bias.
  const bool fp8 = d->kv_fp8 || d->q_fp8;
  if (fp8) {
    if (!d->kv_fp8 || !d->q_fp8 || d->dtype != ATTNFUSE_BF16 || d->rope || d->bias)
      return ATTNFUSE_ERR_UNSUPPORTED;
    const int64_t* in_strides[3] = {d->q_stride, d->k_stride, d->v_stride};
    for (const int64_t* st : in_strides)
      for (int a = 0; a < 3; ++a)
        if (st[a] % 16) return ATTNFUSE_ERR_UNSUPPORTED;
    if (d->tile_waves != 0 && d->tile_waves != 8) return ATTNFUSE_ERR_UNSUPPORTED;
  }
  // Q / out may be NULL only when there are no queries, K / V only when there
  // are no keys (empty tensors).
  if (have_ptrs && ((d->Nq > 0 && (!q || !out)) || (d->Nk > 0 && (!k || !v))))
    return ATTNFUSE_ERR_INVALID;
  // fp32 kernels read the fp32 tables; bf16 kernels rotate Q and K with the
  // fp16 pairs.
  if (d->dtype == ATTNFUSE_FP32 && !fp32_tables_ok(d)) return ATTNFUSE_ERR_INVALID;
  if (d->dtype == ATTNFUSE_BF16 && !f16_table_ok(d)) return ATTNFUSE_ERR_INVALID;
  if (have_ptrs && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)))
    return ATTNFUSE_ERR_UNSUPPORTED;
  const bool sparse = d->bs_row_ptr != nullptr;
  const bool bf16 = d->dtype == ATTNFUSE_BF16;
  // The bf16 kernel addresses a 64-key tile with 32-bit offsets.
  if (bf16 && (d->q_stride[2] >= kMaxRowStride || d->k_stride[2] >= kMaxRowStride ||
               d->v_stride[2] >= kMaxRowStride))
    return ATTNFUSE_ERR_UNSUPPORTED;
  if (sparse) {
    if (bf16 && (d->bs_block_m % 64 || d->bs_block_n % 64)) return ATTNFUSE_ERR_UNSUPPORTED;
    if (!bf16 && (d->bs_block_m % 64 || d->bs_block_n % 32)) return ATTNFUSE_ERR_UNSUPPORTED;
  }
  if (d->Nq == 0) return ATTNFUSE_OK;  // plan: nothing to launch
  p = base_params(q, k, v, const_cast<void*>(out), d);
  if (d->Nk == 0) p.row_ptr = nullptr;  // nothing to visit: every row is empty
  const bool use_sparse = p.row_ptr != nullptr;
  p.longest_first = (d->causal && d->window == 0 && !use_sparse) ? 1 : 0;

  if (!bf16) {
    p.n_qblk = (d->Nq + 63) / 64;
    const long long grid = (long long)d->B * d->Hq * p.n_qblk;
    if (grid >= (1LL << 31)) return ATTNFUSE_ERR_UNSUPPORTED;
    if (d->tile_chain > 1) return ATTNFUSE_ERR_UNSUPPORTED;
    f = FwdPlan{ATTNFUSE_PLAN_FP32, 1, 1, 64, grid};
    return ATTNFUSE_OK;
  }

  if (fp8) {
    // Eight waves (the fp8 schedule), as many q-heads of a group as fit.
    int hp = largest_pow2_divisor(p.G, 8);
    if (d->tile_heads != 0) {
      const int h2 = d->tile_heads;
      if (!(h2 == 1 || h2 == 2 || h2 == 4 || h2 == 8) || p.G % h2) return ATTNFUSE_ERR_UNSUPPORTED;
      hp = h2;
    }
    if (use_sparse) {
      if (d->bs_head_stride > 0) {
        if (d->tile_heads > 1) return ATTNFUSE_ERR_UNSUPPORTED;
        hp = 1;
      }
      if (d->bs_block_m % (32 * (8 / hp))) return ATTNFUSE_ERR_UNSUPPORTED;
    }
    p.hp = hp;
    p.n_units = d->B * d->Hkv * (p.G / hp);
    p.n_qblk = (d->Nq + 32 * (8 / hp) - 1) / (32 * (8 / hp));
    long long grid = (long long)p.n_units * p.n_qblk;
    if (grid >= (1LL << 31)) return ATTNFUSE_ERR_UNSUPPORTED;
    grid = pair_blocks(p, d, 32 * (8 / hp), true, use_sparse, grid);
    if (d->tile_chain > 1) return ATTNFUSE_ERR_UNSUPPORTED;
    // Products of codes: both dequantisation scales join the score scale.
    const double sc = d->scale > 0.f ? (double)d->scale : 1.0 / sqrt((double)d->D);
    p.scale_log2 = (float)(sc * 1.4426950408889634 * (double)d->q_scale * (double)d->k_scale);
    p.v_scale = d->v_scale;
    f = FwdPlan{ATTNFUSE_PLAN_FP8, 8, hp, 32 * (8 / hp), grid};
    return ATTNFUSE_OK;
  }

  // bf16 MFMA kernel: choose waves per workgroup (NW) and q-heads per
  // workgroup (hp); the workgroup covers 32 * NW / hp query rows.
  int NW = 8;
  int hp = largest_pow2_divisor(p.G, 8);
  if (use_sparse) {
    if (d->bs_head_stride > 0) hp = 1;  // per-head masks: one head per workgroup
    // The workgroup's rows must lie inside one CSR block row.
    bool found = false;
    for (int nw = 8; nw >= 2 && !found; nw /= 2) {
      const int h2 = hp < nw ? hp : nw;
      if (d->bs_block_m % (32 * (nw / h2)) == 0) {
        NW = nw;
        hp = h2;
        found = true;
      }
    }
    if (!found) return ATTNFUSE_ERR_UNSUPPORTED;
  }
  const bool rope = d->rope != 0;
  const bool scoremod = d->alibi_slopes != nullptr || d->bias != nullptr;
  if (!use_sparse) {
    // Tile table, from the tile sweep on MI355X (GPT-2-small grid, B=4 H=12
    // D=64 N=512..4096 over seven variants, and the Llama-3-8B shape): eight
    // waves with as many q-heads of a group as fit, unless that under-fills
    // the 256 CUs: halve the waves while the grid has fewer than 128
    // workgroups (or a workgroup would hold more row blocks than there are
    // rows); a score modifier (ALiBi, bias) takes four waves when eight
    // would leave fewer than 256 workgroups.
    auto grid_of = [&](int nw) {
      const int h2 = hp < nw ? hp : nw;
      const long long rows = 32LL * (nw / h2);
      return (long long)d->B * d->Hkv * (p.G / h2) * ((d->Nq + rows - 1) / rows);
    };
    const int rb_need = (d->Nq + 31) / 32;
    while (NW > 2 && NW > hp && (NW / hp) / 2 >= rb_need) NW /= 2;
    while (NW > 2 && grid_of(NW) < 128) NW /= 2;
    if (scoremod && NW == 8 && grid_of(8) < 256) NW = 4;
    // D = 64 with one q-head per workgroup (the GPT-2-small geometry): under
    // a band (causal or a window) four waves (128-row blocks, two workgroups
    // and so two waves per SIMD per CU) beat eight (256-row blocks, less of
    // whose band is visible): a window by 10-40%, causal by 2-16% (N 1k-4k),
    // unless the eight-wave blocks pair (causal N=8192: 444 us paired
    // against 452 us on four waves).  Dense launches keep eight waves.
    if (d->D == 64 && NW == 8 && hp == 1 && (d->causal || d->window > 0)) {
      AttnParams pp = p;
      pp.n_units = d->B * d->Hkv * p.G;
      pp.n_qblk = (d->Nq + 255) / 256;
      const long long g8 = (long long)pp.n_units * pp.n_qblk;
      if (pair_blocks(pp, d, 256, true, false, g8) == g8) NW = 4;
    }
    // Dense D = 64, one q-head per workgroup: eight waves run rounds of 256
    // workgroups, four waves rounds of 512 (two per CU) at about 1.08 times
    // the eight-wave time per round, a last round of at most 256 at about
    // 0.65; four waves when that is clearly shorter (a grid of one and a half
    // eight-wave rounds, e.g. B4 H12 N2048: 8-12% faster on four waves).
    if (d->D == 64 && NW == 8 && hp == 1 && !d->causal && d->window == 0 && !scoremod) {
      const long long g8 = grid_of(8), g4 = grid_of(4);
      const double cost8 = (double)((g8 + 255) / 256);
      const long long rem4 = g4 % 512;
      const double cost4 = (double)(g4 / 512) * 1.08 + (rem4 == 0 ? 0.0 : rem4 <= 256 ? 0.65 : 1.08);
      if (cost4 < 0.95 * cost8) NW = 4;
    }
    if (hp > NW) hp = NW;
  }
  if (!attnfuse::fwd_bf16_supported(d->D, NW, rope, scoremod, use_sparse)) {
    NW /= 2;  // fewer waves, twice the registers each
    if (hp > NW) hp = NW;
  }
  if (d->tile_waves != 0 || d->tile_heads != 0) {  // caller's tile choice
    const int nw = d->tile_waves != 0 ? d->tile_waves : NW;
    int h2 = d->tile_heads != 0 ? d->tile_heads : (hp < nw ? hp : nw);
    const bool pow2 = (nw == 2 || nw == 4 || nw == 8) && (h2 == 1 || h2 == 2 || h2 == 4 || h2 == 8);
    if (!pow2 || h2 > nw || p.G % h2 != 0) return ATTNFUSE_ERR_UNSUPPORTED;
    if (use_sparse && (d->bs_block_m % (32 * (nw / h2)) != 0 || (d->bs_head_stride > 0 && h2 != 1)))
      return ATTNFUSE_ERR_UNSUPPORTED;
    if (!attnfuse::fwd_bf16_supported(d->D, nw, rope, scoremod, use_sparse))
      return ATTNFUSE_ERR_UNSUPPORTED;
    NW = nw;
    hp = h2;
  }
  p.hp = hp;
  const int RB = NW / hp;
  p.n_units = d->B * d->Hkv * (p.G / hp);
  p.n_qblk = (d->Nq + 32 * RB - 1) / (32 * RB);
  long long grid = (long long)p.n_units * p.n_qblk;
  if (grid >= (1LL << 31)) return ATTNFUSE_ERR_UNSUPPORTED;
  grid = pair_blocks(p, d, 32 * RB, NW == 8, use_sparse, grid);
  st = chain_blocks(p, d, NW, 32 * RB, use_sparse, rope, grid);
  if (st != ATTNFUSE_OK) return st;
  f = FwdPlan{ATTNFUSE_PLAN_BF16, NW, hp, 32 * RB, grid};
  return ATTNFUSE_OK;
}

}  // namespace

extern "C" {

const char* attnfuse_status_string(int status) {
  switch (status) {
    case ATTNFUSE_OK: return "ok";
    case ATTNFUSE_ERR_INVALID: return "invalid argument or descriptor";
    case ATTNFUSE_ERR_UNSUPPORTED: return "unsupported variant or shape";
    case ATTNFUSE_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTNFUSE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int attnfuse_fwd(const void* q, const void* k, const void* v, void* out,
                 const attnfuse_variant_desc* desc, void* stream) {
  AttnParams p;
  FwdPlan f;
  const int st = plan_fwd(q, k, v, out, desc, true, p, f);
  if (st != ATTNFUSE_OK || f.kind == ATTNFUSE_PLAN_NONE) return st;
  const attnfuse_variant_desc* d = desc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned g = (unsigned)f.grid;
  const bool use_sparse = p.row_ptr != nullptr;
  const bool scoremod = d->alibi_slopes != nullptr || d->bias != nullptr;
  if (f.kind == ATTNFUSE_PLAN_FP32) return hip_status(attnfuse::launch_fwd_fp32(p, d->D, g, s));
  if (f.kind == ATTNFUSE_PLAN_FP8) {
    const bool alibi = d->alibi_slopes != nullptr;
    return hip_status(d->D == 128 ? attnfuse::launch_fwd_fp8<128>(p, alibi, use_sparse, g, s)
                                  : attnfuse::launch_fwd_fp8<64>(p, alibi, use_sparse, g, s));
  }
  const bool rope = d->rope != 0;
  hipError_t e;
  if (d->D == 128) {
    if (f.NW == 8) e = attnfuse::launch_fwd_bf16<128, 8>(p, rope, scoremod, use_sparse, g, s);
    else if (f.NW == 4) e = attnfuse::launch_fwd_bf16<128, 4>(p, rope, scoremod, use_sparse, g, s);
    else e = attnfuse::launch_fwd_bf16<128, 2>(p, rope, scoremod, use_sparse, g, s);
  } else {
    if (f.NW == 8) e = attnfuse::launch_fwd_bf16<64, 8>(p, rope, scoremod, use_sparse, g, s);
    else if (f.NW == 4) e = attnfuse::launch_fwd_bf16<64, 4>(p, rope, scoremod, use_sparse, g, s);
    else e = attnfuse::launch_fwd_bf16<64, 2>(p, rope, scoremod, use_sparse, g, s);
  }
  return hip_status(e);
}

int attnfuse_fwd_plan(const attnfuse_variant_desc* desc, attnfuse_fwd_plan_info* info) {
  if (!info) return ATTNFUSE_ERR_INVALID;
  AttnParams p;
  FwdPlan f;
  const int st = plan_fwd(nullptr, nullptr, nullptr, nullptr, desc, false, p, f);
  if (st != ATTNFUSE_OK) return st;
  *info = attnfuse_fwd_plan_info{};
  info->kernel = f.kind;
  if (f.kind != ATTNFUSE_PLAN_NONE) {
    info->waves = f.NW;
    info->heads = f.hp;
    info->rows = f.rows;
    info->query_blocks = p.n_qblk;
    info->paired = p.pair;
    info->workgroups = f.grid;
    info->chain = p.chain;
  }
  return ATTNFUSE_OK;
}

size_t attnfuse_decode_workspace_size(const attnfuse_variant_desc* desc, int32_t num_splits) {
  if (validate_common(desc) != ATTNFUSE_OK || num_splits < 1 || num_splits > 4096) return 0;
  return (size_t)desc->B * desc->Hq * num_splits * (desc->D + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Split-KV decode on a partials buffer `workspace` of `workspace_bytes`.
int decode_impl(const void* q, const void* k_cache, const void* v_cache, void* out,
                const attnfuse_variant_desc* desc, int32_t num_splits, void* workspace,
                size_t workspace_bytes, void* stream) {
  int st = validate_common(desc);
  if (st != ATTNFUSE_OK) return st;
  const attnfuse_variant_desc* d = desc;
  if (!q || !k_cache || !v_cache || !out) return ATTNFUSE_ERR_INVALID;
  if (d->Nq != 1 || num_splits < 1 || num_splits > 4096) return ATTNFUSE_ERR_INVALID;
  if (!f16_table_ok(d)) return ATTNFUSE_ERR_INVALID;
  if (d->dtype != ATTNFUSE_BF16 || d->bias || d->bs_row_ptr || d->q_fp8) return ATTNFUSE_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return ATTNFUSE_ERR_UNSUPPORTED;
  const size_t need = attnfuse_decode_workspace_size(d, num_splits);
  if (!workspace || workspace_bytes < need) return ATTNFUSE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTNFUSE_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  AttnParams p = base_params(q, k_cache, v_cache, out, d);
  p.splits = num_splits;
  p.chunk = (d->Nk + num_splits - 1) / num_splits;
  if (p.chunk < 1) p.chunk = 1;
  p.n_hgrp = (p.G + 31) / 32;
  p.ws = reinterpret_cast<float*>(workspace);
  if (d->kv_fp8) {  // rows = scale * code: the key scale joins the score scale
    p.scale_log2 *= d->k_scale;
    p.v_scale = d->v_scale;
  }
  const long long U = (long long)d->B * d->Hkv * p.n_hgrp;
  const long long grid = 8 * U * ((num_splits + 7) / 8);
  if (grid >= (1LL << 31) || (long long)d->B * d->Hq * (d->D / 32) >= (1LL << 31))
    return ATTNFUSE_ERR_UNSUPPORTED;
  hipError_t e = attnfuse::launch_decode_split(p, d->D, d->rope != 0, d->kv_fp8 != 0,
                                               (unsigned)grid, s);
  if (e != hipSuccess) return ATTNFUSE_ERR_HIP;
  return hip_status(attnfuse::launch_decode_combine(p, d->D, s));
}

constexpr size_t kScratchBytes = ATTNFUSE_DECODE_NOALLOC_MAX_BYTES;

}  // namespace

namespace attnfuse {
// Partials buffer of attnfuse_decode_noalloc: one static array per GPU (the
// code object's copy on that device), never allocated at run time.  In host
// code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
__device__ __align__(256) unsigned char scratch[kScratchBytes];
}  // namespace attnfuse

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(attnfuse::scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attnfuse_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                    const attnfuse_variant_desc* desc, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, out, desc, num_splits, workspace, workspace_bytes, stream);
}

int attnfuse_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out,
                            const attnfuse_variant_desc* desc, int32_t num_splits, void* stream) {
  int st = validate_common(desc);
  if (st != ATTNFUSE_OK) return st;
  if (num_splits < 1 || num_splits > 4096) return ATTNFUSE_ERR_INVALID;
  if (attnfuse_decode_workspace_size(desc, num_splits) > kScratchBytes) return ATTNFUSE_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return ATTNFUSE_ERR_HIP;
  return decode_impl(q, k_cache, v_cache, out, desc, num_splits, ws, kScratchBytes, stream);
}

namespace {
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
// Workspace of the backward: delta [B, Hq, Nq] fp32, then with RoPE the
// rotated copies Q' [B, Hq, Nq, D] and K' [B, Hkv, Nk, D] in bf16.
size_t bwd_delta_bytes(const attnfuse_variant_desc* d) {
  return round256((size_t)d->B * d->Hq * d->Nq * sizeof(float));
}
// The rotated copies are only read when there are both queries and keys.
bool bwd_rotates(const attnfuse_variant_desc* d) { return d->rope && d->Nq > 0 && d->Nk > 0; }
size_t bwd_qrot_bytes(const attnfuse_variant_desc* d) {
  return bwd_rotates(d) ? round256((size_t)d->B * d->Hq * d->Nq * d->D * 2) : 0;
}
size_t bwd_krot_bytes(const attnfuse_variant_desc* d) {
  return bwd_rotates(d) ? round256((size_t)d->B * d->Hkv * d->Nk * d->D * 2) : 0;
}

// Under a causal or windowed band the dK/dV work of the key blocks differs by
// up to Nk/128 times; when the grid is too small to even that out over the
// 256 CUs, each (kv-head, key block) is split over two workgroups (each
// taking half of its (q-head, query tile) steps) that write fp32 partial
// sums, which a last pass adds up.
int bwd_kv_parts(const attnfuse_variant_desc* d) {
  const long long gk = (long long)d->B * d->Hkv * ((d->Nk + 127) / 128);
  return ((d->causal || d->window > 0) && d->Nq > 0 && gk > 0 && gk <= 512) ? 2 : 1;
}
size_t bwd_part_bytes(const attnfuse_variant_desc* d) {
  const int parts = bwd_kv_parts(d);
  return parts > 1 ? round256((size_t)parts * 2 * d->B * d->Hkv * d->Nk * d->D * sizeof(float)) : 0;
}
}  // namespace

size_t attnfuse_bwd_workspace_size(const attnfuse_variant_desc* desc) {
  if (validate_common(desc) != ATTNFUSE_OK) return 0;
  return bwd_delta_bytes(desc) + bwd_qrot_bytes(desc) + bwd_krot_bytes(desc) + bwd_part_bytes(desc);
}

int attnfuse_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, const attnfuse_variant_desc* desc,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_common(desc);
  if (st != ATTNFUSE_OK) return st;
  const attnfuse_variant_desc* d = desc;
  if (d->dtype != ATTNFUSE_BF16 || d->kv_fp8 || d->q_fp8) return ATTNFUSE_ERR_UNSUPPORTED;
  if (d->bs_row_ptr && (d->bs_block_m % 64 || d->bs_block_n % 64)) return ATTNFUSE_ERR_UNSUPPORTED;
  // The gradient kernels address a tile's rows by 32-bit offsets from the
  // tile's first row.
  if (d->q_stride[2] >= kMaxRowStride || d->k_stride[2] >= kMaxRowStride ||
      d->v_stride[2] >= kMaxRowStride || d->o_stride[2] >= kMaxRowStride)
    return ATTNFUSE_ERR_UNSUPPORTED;
  if (d->Nq > 0 && (!q || !out || !dout || !lse || !dq)) return ATTNFUSE_ERR_INVALID;
  if (d->Nk > 0 && (!k || !v || !dk || !dv)) return ATTNFUSE_ERR_INVALID;
  if (!fp32_tables_ok(d)) return ATTNFUSE_ERR_INVALID;
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTNFUSE_ERR_UNSUPPORTED;
  if (d->Nq == 0 && d->Nk == 0) return ATTNFUSE_OK;
  const size_t need = attnfuse_bwd_workspace_size(d);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return ATTNFUSE_ERR_WORKSPACE;
  AttnParams p = base_params(q, k, v, const_cast<void*>(out), d);
  if (d->Nk == 0) p.row_ptr = nullptr;  // no keys: nothing to visit
  p.lse = const_cast<float*>(lse);
  attnfuse::BwdParams g{};
  g.dout = static_cast<const __bf16*>(dout);
  g.delta = static_cast<float*>(workspace);
  g.dq = static_cast<__bf16*>(dq);
  g.dk = static_cast<__bf16*>(dk);
  g.dv = static_cast<__bf16*>(dv);
  char* ws = static_cast<char*>(workspace);
  g.kv_parts = bwd_kv_parts(d);
  g.kv_part = g.kv_parts > 1 ? reinterpret_cast<float*>(ws + bwd_delta_bytes(d) + bwd_qrot_bytes(d) +
                                                        bwd_krot_bytes(d))
                             : nullptr;
  if (bwd_rotates(d)) {
    g.qrot = reinterpret_cast<__bf16*>(ws + bwd_delta_bytes(d));
    g.krot = reinterpret_cast<__bf16*>(ws + bwd_delta_bytes(d) + bwd_qrot_bytes(d));
    g.qr = g.qrot;
    g.kr = g.krot;
    g.qr_sb = (long long)d->Hq * d->Nq * d->D;
    g.qr_sh = (long long)d->Nq * d->D;
    g.kr_sb = (long long)d->Hkv * d->Nk * d->D;
    g.kr_sh = (long long)d->Nk * d->D;
    g.qr_sn = g.kr_sn = d->D;
  } else {
    g.qr = static_cast<const __bf16*>(q);
    g.kr = static_cast<const __bf16*>(k);
    g.qr_sb = d->q_stride[0]; g.qr_sh = d->q_stride[1]; g.qr_sn = d->q_stride[2];
    g.kr_sb = d->k_stride[0]; g.kr_sh = d->k_stride[1]; g.kr_sn = d->k_stride[2];
  }
  const long long gq = (long long)d->B * d->Hq * ((d->Nq + 63) / 64);
  const long long gk = (long long)d->B * d->Hkv * ((d->Nk + 127) / 128) * g.kv_parts;
  // The rotation and row-reduction passes use at most one 256-thread block
  // per 16 rows (D = 128 row reduction).
  const long long row_blocks = (long long)d->B * (d->Hq > d->Hkv ? d->Hq : d->Hkv) *
                               (d->Nq > d->Nk ? d->Nq : d->Nk) / 16 + 1;
  if (gq >= (1LL << 31) || gk >= (1LL << 31) || row_blocks >= (1LL << 31))
    return ATTNFUSE_ERR_UNSUPPORTED;
  return hip_status(attnfuse::launch_bwd(p, g, d->D, reinterpret_cast<hipStream_t>(stream)));
}

int attnfuse_rope_table(double theta, int32_t D, int64_t len, float* cos_out, float* sin_out,
                        uint32_t* cs_f16_out, uint32_t* cs_bf16_out, void* stream) {
  if (!(theta > 0.0) || !isfinite(theta) || D < 2 || D > 1024 || D % 2 || len < 1 ||
      len >= kMaxLen || (!cos_out && !sin_out && !cs_f16_out && !cs_bf16_out))
    return ATTNFUSE_ERR_INVALID;
  return hip_status(attnfuse::launch_rope_table(theta, D, len, cos_out, sin_out, cs_f16_out,
                                                cs_bf16_out, reinterpret_cast<hipStream_t>(stream)));
}

int attnfuse_prerotate(const void* x, void* x_rot, const attnfuse_variant_desc* desc,
                       int32_t which, void* stream) {
  int st = validate_common(desc);
  if (st != ATTNFUSE_OK) return st;
  const attnfuse_variant_desc* d = desc;
  if (!x || !x_rot || !d->rope || (which != 0 && which != 1)) return ATTNFUSE_ERR_INVALID;
  if (d->kv_fp8 || d->q_fp8) return ATTNFUSE_ERR_UNSUPPORTED;
  if (!fp32_tables_ok(d)) return ATTNFUSE_ERR_INVALID;
  const int H = which == 0 ? d->Hq : d->Hkv;
  const int N = which == 0 ? d->Nq : d->Nk;
  const int64_t* str = which == 0 ? d->q_stride : d->k_stride;
  const int pos0 = (int)(which == 0 ? d->q_pos0 : d->k_pos0);
  if (N == 0) return ATTNFUSE_OK;
  const bool vec_ok = aligned16(x) && aligned16(x_rot);
  return hip_status(attnfuse::launch_prerotate(
      x, x_rot, d->dtype == ATTNFUSE_BF16, vec_ok, d->D, d->B, H, N, str[0], str[1], str[2],
      pos0, d->rope_cos, d->rope_sin, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
