/*
 * pa_probe.h -- measurement kernels of libpa_probe.so (not part of the
 * paged-attention ABI in pa.h; a benchmark links them to report what the device
 * it runs on reaches beside the published figures).  Same conventions as pa.h:
 * device pointers, asynchronous on `stream`, host-side validation returning a
 * pa_status before anything is enqueued, nothing allocated.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Device ceilings, for the rooflines of the entry points of pa.h: the pages
 * call decode bandwidth-bound and prefill compute-bound ([T4 engine];
 * [Pico-vLLM] "H200 comparison"), and these two kernels measure the
 * corresponding limits of the device they run on.  Measurement only.
 *
 * pa_probe_stream_read: reads `bytes` (a positive multiple of 16) of device
 * memory at buf once, with 16-byte non-temporal loads from `grid` workgroups
 * of 256 threads, and writes the 32-bit wrap-around sum of the buffer's
 * 32-bit words seen by workgroup w to sums[w] (sums: uint32 [grid], device
 * memory); the grand total equals the sum of all words of the buffer mod 2^32.
 *
 * pa_probe_gather_read: reads `bytes` of device memory at buf once as 4 KiB
 * tiles (the size of one (block, KV head) tile of a paged pool at head_dim 128)
 * in a scrambled order, each wave of 64 lanes loading 4 tiles with all of its
 * loads in flight before it adds them: the access pattern of a paged K/V read
 * without its arithmetic.  bytes must be a positive multiple of 4096 whose
 * tile count is a power of two.  Workgroup w (of
 * pa_probe_gather_read_groups(bytes)) writes to sums[w] the 32-bit
 * wrap-around sum of the words it read; the grand total equals the sum of all
 * words of the buffer mod 2^32.  pa_probe_gather_read_groups returns 0 for
 * bytes <= 0.
 *
 * pa_probe_mfma_bf16: `grid` workgroups of 4 waves each run `iters` rounds of
 * four independent 16x16x32 bf16 matrix products per wave (16384 flop each);
 * wave v of workgroup w writes out[4*w + v] = 128 * iters exactly (out: fp32
 * [4*grid], device memory).  flop = grid * 4 * iters * 4 * 16384.
 *
 * pa_probe_issue_mix: `grid` workgroups of 4 waves each run `iters` rounds of
 * (mode 1) sixteen 16x16x32 bf16 matrix products per wave on 8 independent
 * accumulators, (mode 2) thirty-two exp2 + FMA steps per lane on 16
 * independent chains, or (mode 3) both in the same wave.  A grid of c x (the
 * CU count) places c waves on each SIMD; the launch times of the three modes
 * show whether a SIMD overlaps matrix products with that ALU work (the mix of
 * a softmax beside the products of an attention step).  Thread t of the grid
 * writes a deterministic, finite value to out[t] (out: fp32 [256 * grid],
 * device memory).
 *
 * PA_ERR_NULL for a NULL pointer, PA_ERR_SHAPE for non-positive sizes, a mode
 * outside 1..3 or a byte count not a multiple of 16 (of 4096 with a
 * power-of-two tile count for the gather).
 */
pa_status pa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sums, int32_t grid,
                               pa_stream_t stream);
int64_t pa_probe_gather_read_groups(int64_t bytes);
pa_status pa_probe_gather_read(const void* buf, int64_t bytes, uint32_t* sums, pa_stream_t stream);
pa_status pa_probe_mfma_bf16(int32_t iters, float* out, int32_t grid, pa_stream_t stream);
pa_status pa_probe_issue_mix(int32_t mode, int32_t iters, float* out, int32_t grid, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
