/*
 * attnfuse_microbench.h -- machine-peak probes shipped with the fused
 * attention library (libattnfuse.so), used to put the attention kernels'
 * measured throughput next to what the chip sustains on the same box.
 *
 * They are not part of the attention computation.  The roofline they serve is
 * the one of "5.3 The Rotation Calculus" (AttnFuse: A Composable DSL for
 * Compiling Attentions to Fused GPU Kernels): compute throughput against
 * memory bandwidth.
 *
 * Conventions: every pointer is caller-owned device memory; `stream` is a
 * hipStream_t (NULL = default stream); work is enqueued asynchronously and the
 * caller times it (e.g. with events on the same stream).  The first wave of
 * the first workgroup writes two counters to stamps[0..1]: elapsed shader-clock
 * cycles (s_memtime) and elapsed ticks of the constant 100 MHz counter
 * (s_memrealtime) over its own run, so stamps[0] / stamps[1] * 100 MHz is the
 * shader clock while the probe ran.  Invalid arguments return
 * ATTNFUSE_MB_ERR_INVALID with nothing enqueued; a failed launch returns
 * ATTNFUSE_MB_ERR_HIP.
 */
#ifndef ATTNFUSE_MICROBENCH_H_
#define ATTNFUSE_MICROBENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTNFUSE_MB_OK = 0,
  ATTNFUSE_MB_ERR_INVALID = -1,
  ATTNFUSE_MB_ERR_HIP = -4
};

/* Matrix-core loop: `workgroups` workgroups of 256 threads (four waves); each
 * wave issues 4 * iters v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on four
 * independent accumulators.  Total work: workgroups * 4 * 4 * iters * 32768
 * FLOP.  sink: workgroups * 256 floats (written, values meaningless);
 * stamps: 2 uint64.  1 <= workgroups <= 2^20, 1 <= iters <= 2^24. */
int attnfuse_mb_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, unsigned long long* stamps,
                          void* stream);

/* The same matrix-core loop on caller-given operands: `operands` holds
 * workgroups * 256 * 64 bytes of device memory (16-byte aligned), four
 * bf16x8 values per thread (a0, b0, a1, b1); consecutive MFMAs alternate
 * them (a0 b0, a1 b1, a0 b1, a1 b0), so with random values the matrix
 * core's inputs change every instruction.  Same work, sink and stamps as
 * attnfuse_mb_mfma_bf16. */
int attnfuse_mb_mfma_bf16_ops(int32_t workgroups, int32_t iters, const void* operands, float* sink,
                              unsigned long long* stamps, void* stream);

/* Streaming read of `bytes` bytes at `src` (16-byte aligned, bytes a multiple
 * of 16) by `workgroups` workgroups of 256 threads, 16-byte loads, grid-stride
 * with four loads in flight per thread.  sink: workgroups * 256 floats;
 * stamps: 2 uint64.  1 <= workgroups <= 2^20. */
int attnfuse_mb_hbm_read(const void* src, size_t bytes, int32_t workgroups, float* sink,
                         unsigned long long* stamps, void* stream);

/* Host cost of one call ("3.3 Runtime Dispatch" keeps it under a microsecond
 * on the pages' system): issues `calls` calls back to back from C, with no
 * synchronisation, and writes the mean host time per call (ns) to
 * *ns_per_call.  which = 0: attnfuse_fwd(q, k, v, out, desc, stream);
 * which = 1: attnfuse_decode(q, k, v, out, desc, num_splits, workspace,
 * workspace_bytes, stream); which = 2: a launch of an empty kernel that takes
 * the same kernel-argument block as the attention kernels (HIP's own launch
 * cost; the tensor arguments are ignored); which = 3: attnfuse_fwd on a copy
 * of *desc with Nq = 0, which runs the whole argument validation and returns
 * before any launch (the library's own host cost).  The calls enqueue real work on
 * `stream`: keep `calls` small enough for the queue not to fill (a full queue
 * makes the host wait for the GPU).  Returns the first failing call's status
 * (the entry point's own codes) or ATTNFUSE_MB_OK; 1 <= calls <= 2^20. */
int attnfuse_mb_host_cost(int32_t which, const void* q, const void* k, const void* v, void* out,
                          const struct attnfuse_variant_desc* desc, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, int32_t calls, double* ns_per_call, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNFUSE_MICROBENCH_H_ */
