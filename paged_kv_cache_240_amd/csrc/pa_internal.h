// Internal launchers of libpa (C++ linkage, not part of the ABI).  Arguments
// are already validated by the entry points in pa_api.cpp; each launcher only
// picks the kernel instance and grid, enqueues it and reports the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

hipError_t launch_cache_store(void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, const int32_t* positions,
                              const float* cos_sin, int T, int Hq, int Hkv, int D,
                              hipStream_t stream);

// Split-K partial kernel (partition_size > 0) or single pass (partition_size == 0,
// o_part/lse unused, out written).
hipError_t launch_decode(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                         int max_blocks, int max_context_len, float scale, int partition_size,
                         hipStream_t stream);

// The decode step with the store folded into the decode kernel: RoPE of q
// and of the new k, the new token's K/V row stored at position L-1, attention;
// with partition_size > 0 the partials are then reduced by the combine launch
// (with_combine) or left in o_part / lse.
hipError_t launch_decode_step(void* out, float* o_part, float* lse, const void* q,
                              const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const float* cos_sin, int B, int Hq, int Hkv, int D, int max_blocks,
                              int max_context_len, float scale, int partition_size,
                              bool with_combine, hipStream_t stream);

// Multi-query (speculative verification) partial kernel or single pass: q/out
// are [B][NQ][Hq][D]; the partials are reduced by launch_decode_combine over
// NQ * Hq rows per sequence.
hipError_t launch_decode_multi(void* out, float* o_part, float* lse, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int B,
                               int NQ, int Hq, int Hkv, int D, int max_blocks, int max_context_len,
                               float scale, int partition_size, hipStream_t stream);

hipError_t launch_decode_combine(void* out, const float* o_part, const float* lse,
                                 const int32_t* context_lens, int B, int Hq, int D,
                                 int num_partitions, int partition_size, hipStream_t stream);

// Whole-block copies src pools -> dst pools for n (src, dst) id pairs.
hipError_t launch_block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                             const int32_t* src_ids, const int32_t* dst_ids, int n,
                             int64_t bytes_per_block, hipStream_t stream);

hipError_t launch_rmsnorm(void* out, void* residual, const void* x, const void* weight, int T,
                          int H, float eps, hipStream_t stream);

hipError_t launch_swiglu(void* out, const void* gate_up, int64_t T, int I, hipStream_t stream);

// The current device's address of the library's own split-K workspace of
// PA_DECODE_NOALLOC_SCRATCH_BYTES (pa_decode_noalloc), looked up on its first
// use on that device; NULL if the lookup fails.
void* decode_scratch();

// Workgroups of the chunked-prefill launch (its grid is one-dimensional).
int64_t prefill_workgroups(int B, int Hq, int Hkv, int max_query_len);
hipError_t launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int B, int Hq, int Hkv, int D,
                          int max_blocks, int max_query_len, float scale, hipStream_t stream);

// Device ceilings (measurement only): a streaming read of `bytes` (a multiple
// of 16) writing one 32-bit sum per workgroup to sums[grid]; and `iters`
// rounds of four bf16 MFMA chains per wave, one float per wave to out[grid*4].
hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sums, int grid,
                                    hipStream_t stream);
hipError_t launch_probe_mfma_bf16(int iters, float* out, int grid, hipStream_t stream);
hipError_t launch_probe_issue_mix(int mode, int iters, float* out, int grid, hipStream_t stream);
// A one-pass gather of `bytes` (a power-of-two count of 4 KiB tiles) in
// scrambled 4 KiB tiles, one 32-bit sum per workgroup to
// sums[probe_gather_read_groups(bytes)].
int64_t probe_gather_read_groups(int64_t bytes);
hipError_t launch_probe_gather_read(const void* buf, int64_t bytes, uint32_t* sums,
                                    hipStream_t stream);

// Shared-prefix decode: the group prefixes' partials (chunked-prefill kernel,
// group mode: rows of up to group_prefix_row_blocks(max_group_size, G) row
// blocks per (group, partition, KV head); part_tokens a multiple of 32), the
// suffix partitions of each sequence from starts[b], and their log-sum-exp
// reduce.  Workspace rows hold num_slots partials: suffix partitions from slot
// 0, prefix partitions from slot0.
int64_t group_prefix_row_blocks(int max_group_size, int G);
hipError_t launch_group_prefix(float* o_part, float* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* group_start, const int32_t* prefix_lens, int groups,
                               int max_group_size, int max_prefix, int part_tokens, int slot0,
                               int num_slots, int Hq, int Hkv, int D, int max_blocks, float scale,
                               hipStream_t stream);
hipError_t launch_decode_suffix(float* o_part, float* lse, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* starts, int B, int Hq,
                                int Hkv, int D, int max_blocks, int max_context_len, float scale,
                                int partition_size, int num_slots, hipStream_t stream);
// The same decode in one partition launch of the decode kernel: items of one
// 16-row tile -- 16 / G sequences of a group over one partition of their
// shared prefix (slots slot0 + i), or one sequence's G heads over a partition
// of its tokens after the prefix (slots 0..) -- each reading its K/V once.
// Partitions of at most 512 tokens (one chunk); the same reduce follows.
hipError_t launch_cascade_decode(float* o_part, float* lse, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* group_start,
                                 const int32_t* prefix_lens, int B, int num_groups,
                                 int max_group_size, int max_prefix, int prefix_part,
                                 int max_suffix, int suffix_part, int slot0, int num_slots,
                                 int Hq, int Hkv, int D, int max_blocks, float scale,
                                 hipStream_t stream);
hipError_t launch_decode_combine_cascade(void* out, const float* o_part, const float* lse,
                                         const int32_t* context_lens, const int32_t* starts, int B,
                                         int Hq, int D, int num_slots, int partition_size,
                                         int slot0, int prefix_tokens, hipStream_t stream);

}  // namespace pa
