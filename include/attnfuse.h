/*
 * attnfuse.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * Operation (AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU
 * Kernels, arXiv 2609.13612):
 *
 *     out = softmax(mask(bias(RoPE(Q) . RoPE(K)^T * scale))) . V
 *
 * computed exactly (online softmax, "2 Background / FlashAttention and online
 * softmax") in one fused kernel per call.  The variant descriptor carries one
 * field group per building block of "3.1 The Researcher Interface":
 * scaled_dot_product (scale), rope (cos/sin table), causal, sliding_window,
 * full (no mask field set), block_sparse (CSR BlockMask, "4.3 Block-Sparse
 * Attention"), alibi (slopes), additive_bias (bias tensor), softmax (norm).
 * relu_attention is named on the pages but never defined there; its enum
 * value is reserved and rejected with ATTNFUSE_ERR_UNSUPPORTED.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Tensors are [B, H, N, D] with D contiguous (stride 1); the b, h, n strides
 *    are given in elements.  Q is [B, Hq, Nq, D]; K and V are [B, Hkv, Nk, D];
 *    the output has Q's shape with its own strides.  Hq must be a multiple of
 *    Hkv; q-head h reads kv-head h / (Hq / Hkv) (grouped-query attention).
 *  * dtype ATTNFUSE_BF16: Q, K, V, out are bf16; products accumulate in fp32.
 *    dtype ATTNFUSE_FP32: everything is fp32 (no bf16 rounding anywhere).
 *  * Positions: query row i sits at q_pos0 + i, key row j at k_pos0 + j.
 *    They drive RoPE angles, the causal / window masks and ALiBi distances.
 *  * Every pointer argument is caller-owned DEVICE memory (except `desc`,
 *    which is host memory read during the call only).  The library
 *    allocates nothing, keeps no pointer after returning, and holds no mutable
 *    global state, so calls from several host threads are safe.  (The one
 *    exception is attnfuse_decode_noalloc, which writes a static per-GPU
 *    buffer of the library instead of a caller workspace; see there.)
 *  * `stream` is a hipStream_t (NULL = the default stream).  All GPU work is
 *    enqueued asynchronously on it; the caller keeps buffers alive until the
 *    stream has completed the work.  No call synchronises.
 *  * Errors: argument validation happens on the host before any GPU work and
 *    returns ATTNFUSE_ERR_INVALID (malformed arguments) or
 *    ATTNFUSE_ERR_UNSUPPORTED (well formed but not implemented) with nothing
 *    enqueued.  A failed kernel launch returns ATTNFUSE_ERR_HIP.  No C++
 *    exception crosses this interface.
 */
#ifndef ATTNFUSE_H_
#define ATTNFUSE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attnfuse_status {
  ATTNFUSE_OK = 0,
  ATTNFUSE_ERR_INVALID = -1,     /* malformed descriptor or argument          */
  ATTNFUSE_ERR_UNSUPPORTED = -2, /* well formed, but no kernel implements it  */
  ATTNFUSE_ERR_WORKSPACE = -3,   /* decode / backward workspace missing or too small */
  ATTNFUSE_ERR_HIP = -4          /* a HIP runtime call or launch failed        */
} attnfuse_status;

typedef enum attnfuse_dtype {
  ATTNFUSE_BF16 = 0,
  ATTNFUSE_FP32 = 1
} attnfuse_dtype;

typedef enum attnfuse_norm {
  ATTNFUSE_NORM_SOFTMAX = 0,
  ATTNFUSE_NORM_RELU = 1 /* reserved: rejected with ATTNFUSE_ERR_UNSUPPORTED */
} attnfuse_norm;

/* Variant descriptor: one field group per building block.  Zero-initialise,
 * set struct_size = sizeof(attnfuse_variant_desc), then fill what is used. */
typedef struct attnfuse_variant_desc {
  uint32_t struct_size;   /* must equal sizeof(attnfuse_variant_desc)               */
  int32_t dtype;          /* attnfuse_dtype                                          */
  int32_t B, Hq, Hkv;     /* batch, query heads, key/value heads (Hq % Hkv == 0)     */
  int32_t Nq, Nk, D;      /* query rows, key rows, head dim (D in {64, 128})         */
  int64_t q_stride[3];    /* element strides of Q over (b, h, n); d stride is 1      */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];

  /* scaled_dot_product: scores are <q', k'> * scale; scale 0 means 1/sqrt(D). */
  float scale;
  int32_t norm;           /* attnfuse_norm                                           */

  /* rope ("4.1 Fused RoPE", NeoX half-split pairs (r, r + D/2)).  rope != 0
   * applies the rotation in-kernel to Q (once) and to every K tile.  The
   * tables hold cos / sin of position * theta^(-2r/D), row-major
   * [rope_table_len][D/2], 16-byte aligned:
   *   rope_cos / rope_sin: fp32.  Read by attnfuse_fwd with dtype
   *     ATTNFUSE_FP32 and by attnfuse_prerotate.
   *   rope_cs_f16: one 32-bit word per entry holding the fp16 pair (cos in
   *     bits 0-15, sin in bits 16-31; rounding at most 2^-12, well below the
   *     bf16 rounding of the rotated vectors).  Read by attnfuse_fwd with
   *     dtype ATTNFUSE_BF16 (the Q and K rotations, fp32 arithmetic on the
   *     exact bf16 values) and by attnfuse_decode.
   *   rope_cs_bf16: the same pairs rounded to bf16, as attnfuse_rope_table
   *     writes them.  No entry point reads it (the field keeps the
   *     descriptor's layout); it may be NULL.
   * Build them with attnfuse_rope_table.  Every position used
   * (q_pos0 + Nq - 1, k_pos0 + Nk - 1) must be below rope_table_len.
   * rope_theta records the base the tables were built with.  A table an
   * entry point does not read may be NULL. */
  int32_t rope;
  double rope_theta;
  const float* rope_cos;
  const float* rope_sin;
  const uint32_t* rope_cs_f16;
  const uint32_t* rope_cs_bf16;
  int64_t rope_table_len;

  int64_t q_pos0, k_pos0; /* positions of query row 0 and key row 0 (>= 0)          */

  /* causal: keep p_k <= p_q.  sliding_window: window > 0 keeps
   * 0 <= p_q - p_k < window when causal, |p_q - p_k| < window otherwise. */
  int32_t causal;
  int32_t window;

  /* alibi: adds alibi_slopes[h] * (p_k - p_q) to the score of q-head h.
   * NULL = off.  fp32 [Hq]. */
  const float* alibi_slopes;

  /* additive_bias: adds bias[b, h, i, j] (fp32) to the score.  Strides are in
   * elements over (b, h, i, j); a stride of 0 broadcasts that axis.  NULL = off.
   * Supported by attnfuse_fwd only. */
  const float* bias;
  int64_t bias_stride[4];

  /* block_sparse (CSR BlockMask): query row i may see key j only when key
   * block j / bs_block_n is listed in CSR row i / bs_block_m.  bs_row_ptr
   * holds ceil(Nq / bs_block_m) + 1 offsets into bs_col_idx (bs_nnz
   * entries); with bs_head_stride > 0, q-head h uses the row_ptr block that
   * starts at bs_row_ptr + h * bs_head_stride (one mask per head), with 0 one
   * mask serves every head.  The same mask serves every batch index.  Offsets
   * are clamped to [0, bs_nnz] and columns outside the key range are skipped,
   * so a malformed mask gives wrong numbers but no out-of-bounds access.
   * bf16: bs_block_m % 64 == 0 and bs_block_n % 64 == 0.
   * fp32: bs_block_m % 64 == 0 and bs_block_n % 32 == 0.
   * NULL bs_row_ptr = dense.  Supported by attnfuse_fwd only. */
  const int32_t* bs_row_ptr;
  const int32_t* bs_col_idx;
  int32_t bs_block_m, bs_block_n;
  int64_t bs_head_stride;
  int64_t bs_nnz;

  /* Saved row statistic ("4.4 Backward Pass": L = m + log l, natural log):
   * optional fp32 output [B, Hq, Nq], contiguous.  Rows with no visible key
   * get -inf (and an all-zero output row).  NULL = not written. */
  float* lse;

  /* Tile choice of attnfuse_fwd's bf16 prefill kernel ("3.2 From DSL to
   * Kernel", the Tile pass): tile_waves = waves per workgroup (2, 4 or 8),
   * tile_heads = q-heads of a GQA group per workgroup (1, 2, 4 or 8, dividing
   * Hq / Hkv, at most tile_waves); the workgroup covers 32 * tile_waves /
   * tile_heads query rows against 64-key tiles.  0 = the library's dispatch
   * table (from a tile sweep on MI355X).  A choice the kernels cannot run
   * (a block mask whose bs_block_m is not a multiple of the workgroup's rows,
   * per-head masks with tile_heads > 1, or a variant without an instance at
   * that size) returns ATTNFUSE_ERR_UNSUPPORTED.  Ignored by the other entry
   * points and by fp32. */
  int32_t tile_waves;
  int32_t tile_heads;

  /* KV cache in fp8 (attnfuse_decode only): kv_fp8 = 1 means k_cache and
   * v_cache hold OCP FP8 E4M3 codes (1 byte each: bias 7, largest 448, no
   * infinities) and the cached rows are k_scale * code and v_scale * code
   * (per-tensor dequantisation scales, finite and > 0); K/V strides then
   * count bytes and keep the 8-element alignment of the bf16 layout.  q and
   * out stay bf16.  0 = K/V have the dtype above.  attnfuse_fwd takes
   * kv_fp8 = 1 only together with q_fp8 = 1 (below); the other entry points
   * return ATTNFUSE_ERR_UNSUPPORTED when kv_fp8 is set. */
  int32_t kv_fp8;
  float k_scale;
  float v_scale;

  /* fp8 prefill inputs (attnfuse_fwd; "9.1 Limitations and Future
   * Directions" names fp8 as future work): q_fp8 = 1 together with kv_fp8 = 1
   * means q, k and v all hold OCP FP8 E4M3 codes, the rows being
   * q_scale * code, k_scale * code and v_scale * code (per-tensor
   * dequantisation scales, finite and > 0).  Q and K then meet on the fp8
   * matrix core (products of codes, fp32 accumulate; the scales multiply the
   * fp32 score) and P V runs in bf16 on V codes converted exactly, so the
   * result matches attention on the dequantised values to the bf16 bar.
   * Strides count bytes and must be multiples of 16, base pointers 16-byte
   * aligned; out stays bf16 (dtype ATTNFUSE_BF16).  Supports causal, window,
   * alibi and block_sparse (bs_block_m a multiple of the workgroup's 32 * 8 /
   * tile_heads rows); rope and additive_bias return ATTNFUSE_ERR_UNSUPPORTED
   * (rotated or biased values are not fp8 codes; rotate before quantising),
   * and so do tile_waves other than 0 or 8.  q_fp8 = 1 without kv_fp8 = 1,
   * or on any other entry point, returns ATTNFUSE_ERR_UNSUPPORTED.
   * 0 = q has desc->dtype. */
  int32_t q_fp8;
  float q_scale;

  /* Block-sparse chains (attnfuse_fwd's bf16 prefill with a block mask on
   * the two- and four-wave kernels, without additive_bias, when a
   * workgroup's rows are one CSR block row): tile_chain = consecutive query
   * blocks of one head per workgroup, streamed as one list of key tiles so
   * that a workgroup's start-up and drain are paid once per chain ("4.3
   * Block-Sparse Attention": the work stays proportional to the active
   * blocks).  0 = the library's choice (chains when the single blocks would
   * take several rounds of the CUs); 1 = one block per workgroup.  Larger
   * values than the unit's query blocks act as that count.  Negative values
   * return ATTNFUSE_ERR_INVALID; a value above 1 where no chain can run
   * returns ATTNFUSE_ERR_UNSUPPORTED.  Ignored by the other entry points. */
  int32_t tile_chain;
} attnfuse_variant_desc;

/* Fused attention forward: out = attention(q, k, v) under `desc`.
 * q, k, v, out: device pointers laid out as described above (dtype from
 * desc->dtype); k and v may be NULL when desc->Nk == 0 (every output row is
 * then zero and its lse -inf), q and out when desc->Nq == 0 (nothing to do).
 * Returns an attnfuse_status. */
int attnfuse_fwd(const void* q, const void* k, const void* v, void* out,
                 const attnfuse_variant_desc* desc, void* stream);

/* Which kernel attnfuse_fwd launches for a descriptor, and how ("3.2 From
 * DSL to Kernel": one fused kernel per variant, its tile chosen per shape).
 * kernel: ATTNFUSE_PLAN_NONE (Nq == 0: nothing is launched), _FP32, _BF16
 * (the MFMA kernel) or _FP8.  waves and heads: waves and q-heads per
 * workgroup; rows: query rows of one head per query block; query_blocks:
 * blocks per (batch, kv-head, head group) unit; paired: 1 when every
 * workgroup of a causal dense launch runs two query blocks, block
 * query_blocks - 1 - j and block j, so that all workgroups stream about the
 * same number of key tiles; workgroups: the grid; chain: query blocks per
 * workgroup of a block-sparse launch (tile_chain above), else 1.  Validates `desc` exactly
 * as attnfuse_fwd does, except for the data pointers, which are not
 * examined; returns the status attnfuse_fwd would return for valid
 * pointers.  `info` is host memory owned by the caller; on an error it is
 * left unchanged. */
#define ATTNFUSE_PLAN_NONE 0
#define ATTNFUSE_PLAN_FP32 1
#define ATTNFUSE_PLAN_BF16 2
#define ATTNFUSE_PLAN_FP8 3
typedef struct attnfuse_fwd_plan_info {
  int32_t kernel;
  int32_t waves;
  int32_t heads;
  int32_t rows;
  int32_t query_blocks;
  int32_t paired;
  int64_t workgroups;
  int32_t chain;
} attnfuse_fwd_plan_info;

int attnfuse_fwd_plan(const attnfuse_variant_desc* desc, attnfuse_fwd_plan_info* info);

/* Bytes of workspace attnfuse_decode needs for `desc` and `num_splits`
 * (B * Hq * num_splits * (D + 2) * 4).  Returns 0 for an invalid descriptor. */
size_t attnfuse_decode_workspace_size(const attnfuse_variant_desc* desc, int32_t num_splits);

/* Split-KV single-query decode ("4.2 Flash Decoding").  desc->Nq must be 1;
 * k_cache / v_cache are [B, Hkv, Nk, D] with key j at position k_pos0 + j.
 * Phase 1 splits the Nk keys into num_splits chunks of ceil(Nk / num_splits)
 * keys (trailing chunks may be short or empty), and writes one partial
 * (m, l, acc[D]) per (b, q-head, chunk) into `workspace`; phase 2 merges the
 * partials by log-sum-exp into `out` (and desc->lse when set).  Both kernels
 * run on `stream`.  Supports rope, causal, window, alibi; bias and
 * block_sparse return ATTNFUSE_ERR_UNSUPPORTED; kv_fp8 reads an fp8 cache.
 * workspace is caller-owned
 * device memory of at least attnfuse_decode_workspace_size bytes (else
 * ATTNFUSE_ERR_WORKSPACE); its contents on entry do not matter.
 * 1 <= num_splits <= 4096. */
int attnfuse_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                    const attnfuse_variant_desc* desc, int32_t num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Largest partials buffer attnfuse_decode_noalloc can use (8 MiB). */
#define ATTNFUSE_DECODE_NOALLOC_MAX_BYTES ((size_t)8 << 20)

/* attnfuse_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same two kernels and results as attnfuse_decode with the same
 * arguments, but the partials go to a static buffer of
 * ATTNFUSE_DECODE_NOALLOC_MAX_BYTES that the library holds on each GPU it
 * runs on (until the process ends) instead of a caller workspace.  The call
 * itself allocates nothing; the first call on a device looks up that
 * device's buffer address once.  A call whose partials would exceed the
 * buffer (attnfuse_decode_workspace_size(desc, num_splits) >
 * ATTNFUSE_DECODE_NOALLOC_MAX_BYTES, e.g. B * Hq * num_splits > 16,131 at
 * D = 128) returns ATTNFUSE_ERR_WORKSPACE with nothing enqueued; other errors
 * as attnfuse_decode.  Every call on one GPU shares that GPU's buffer: calls
 * that may overlap in time on one GPU (different streams, or different host
 * threads without ordering) race on it and must be serialised by the
 * caller; calls on one stream are ordered and safe.  The buffer's contents
 * on entry do not matter (phase 1 writes every partial phase 2 reads). */
int attnfuse_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out,
                            const attnfuse_variant_desc* desc, int32_t num_splits, void* stream);

/* RoPE tables ("4.1 Fused RoPE": a precomputed cos / sin table):
 * cos_out[p][r] = cos(p * theta^(-2r/D)), sin_out likewise, for
 * 0 <= p < len and 0 <= r < D/2, with the angle formed in fp64 and the results
 * rounded to fp32; cs_f16_out[p][r] packs the same two values rounded to
 * fp16 (cos in bits 0-15, sin in bits 16-31), cs_bf16_out[p][r] packs them
 * rounded (from fp32, to nearest even) to bf16.  cos_out, sin_out: device
 * buffers of len * D/2 floats; cs_f16_out, cs_bf16_out: len * D/2 uint32.
 * Any output may be NULL (at least one must be given).  D even,
 * 2 <= D <= 1024, 1 <= len < 2^30, theta > 0 and finite. */
int attnfuse_rope_table(double theta, int32_t D, int64_t len, float* cos_out, float* sin_out,
                        uint32_t* cs_f16_out, uint32_t* cs_bf16_out, void* stream);

/* Pre-rotation pass (the "apply RoPE in a separate kernel" baseline of
 * "1 Introduction" and "5.3 The Rotation Calculus"): writes RoPE(x) to x_rot.
 * which = 0 rotates a Q-shaped tensor ([B, Hq, Nq, D], q_stride, positions
 * q_pos0 + i); which = 1 a K-shaped one ([B, Hkv, Nk, D], k_stride,
 * positions k_pos0 + j).  x_rot uses the same strides as x.  Uses desc's
 * dtype, D and rope tables (desc->rope must be non-zero). */
int attnfuse_prerotate(const void* x, void* x_rot, const attnfuse_variant_desc* desc,
                       int32_t which, void* stream);

/* Bytes of workspace attnfuse_bwd needs, each part rounded up to 256:
 *   B * Hq * Nq floats (the row reductions delta = rowsum(dO * O));
 *   with rope (and Nq, Nk > 0): the rotated copies RoPE(q) [B, Hq, Nq, D] and
 *     RoPE(k) [B, Hkv, Nk, D] in bf16, which the gradient passes read;
 *   with causal or window > 0 when B * Hkv * ceil(Nk / 128) <= 512: two fp32
 *     partial sums of dK and dV, [2][2][B * Hkv * Nk][D] (each key block's
 *     work is split over two workgroups to even out the band's imbalance).
 * Returns 0 for an invalid descriptor. */
size_t attnfuse_bwd_workspace_size(const attnfuse_variant_desc* desc);

/* Attention backward ("4.4 Backward Pass": the FlashAttention-2 split into a
 * row-reduction pass, a key/value-gradient pass and a query-gradient pass,
 * no atomics): the gradients of sum(out * dout) with respect to q, k and v,
 * for the forward attnfuse_fwd computes with the same desc.
 *   q, k, v, out: the forward's inputs and output (bf16, desc's strides);
 *   dout: gradient of the output, [B, Hq, Nq, D] with out's strides (o_stride);
 *   lse: the forward's saved statistic [B, Hq, Nq] fp32 (natural log; rows
 *        with no visible key hold -inf and get zero gradients);
 *   dq: written with q's strides; dk, dv: written with k's and v's strides
 *       (with GQA each kv-head's gradient sums over its q-heads);
 *   workspace: caller-owned device memory of at least
 *       attnfuse_bwd_workspace_size bytes, 16-byte aligned (else
 *       ATTNFUSE_ERR_WORKSPACE); its contents on entry do not matter.
 * Supports bf16 with rope (fp32 cos / sin tables required), causal, window,
 * alibi, additive_bias (a constant of the forward: no bias gradient) and
 * block_sparse (both gradient passes visit only listed blocks; bs_block_m
 * and bs_block_n multiples of 64, else ATTNFUSE_ERR_UNSUPPORTED); fp32
 * returns ATTNFUSE_ERR_UNSUPPORTED, and so do row strides (q_stride[2],
 * k_stride[2], v_stride[2], o_stride[2]) of 2^24 elements or more.
 * All pointers 16-byte aligned.  Runs three to six kernels on `stream` (with
 * rope the two rotations first; with split key blocks a final reduction).  */
int attnfuse_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, const attnfuse_variant_desc* desc,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* attnfuse_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTNFUSE_H_ */
