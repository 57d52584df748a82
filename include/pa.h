/*
 * pa.h - C ABI of libpa, paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow four public pages on paged attention:
 *   [Pico-vLLM]  "Pico-vLLM" write-up (zingnex forum): §1 model layer (RoPE,
 *                GQA, in-place rotate_half), §2 kernel layer (paged prefill
 *                kernel, paged decode kernel, fused RoPE + KV-cache store,
 *                Flash-Attention-style tiling), H200 comparison (Flash Decode).
 *   [mini-llm]   "mini-llm-engine" post (liangqianxing): §3.1 Paged KV Cache
 *                (16-token physical blocks, per-sequence logical->physical
 *                block table), §3.3 Chunked Prefill, §3.4 Prefix Caching
 *                (blocks shared by several sequences, ref_count > 1).
 *   [nano-vllm]  "nano-vllm" commentary (ai-stack), FAQ Q2 (KV cache stored
 *                in non-contiguous fixed-size blocks through a table).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to dense row-major data, except where
 *     a comment says "host".  bf16 tensors hold IEEE bfloat16 bit patterns.
 *   - The caller owns all memory.  The library allocates nothing, keeps no
 *     state between calls (apart from caching the device's properties) and
 *     never synchronises: work is enqueued on `stream` and the call returns.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns an error status and leaves every buffer untouched.  No
 *     C++ exception crosses this interface.
 *   - Device-side preconditions are NOT checked (reading device memory would
 *     need a synchronisation); violating one is undefined behaviour:
 *       * every block-table entry a call reads is in [0, num_blocks);
 *       * the non-negative slots of one pa_cache_store call are distinct;
 *       * no store targets a block that several sequences share (a shared
 *         block is copied before it is written, [mini-llm] §3.4);
 *       * 0 <= context_lens[b] <= max_context_len <= max_blocks * block_size;
 *       * positions[i] < max_pos for every token with slot_mapping[i] >= 0.
 *   - Cache layout: k_cache and v_cache are bf16 [num_blocks][Hkv][block_size][D];
 *     the 16 x D tile of one (block, KV head) is contiguous.  Token t of
 *     sequence b lives in block block_tables[b][t / block_size], row
 *     t % block_size ([mini-llm] §3.1, [nano-vllm] FAQ Q2).
 *   - GQA: query head h reads KV head h / (Hq / Hkv) ([Pico-vLLM] §1).
 *   - Supported shapes: block_size 16; head_dim 64 or 128; Hq % Hkv == 0 with
 *     Hq / Hkv between 1 and 8.  Others return PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t.  NULL is the default (null) stream. */
typedef void* pa_stream_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or inconsistent */
  PA_ERR_UNSUPPORTED = 3,  /* consistent, but a shape this library does not implement */
  PA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required */
  PA_ERR_HIP = 5,          /* the HIP runtime reported an error while enqueueing */
  PA_ERR_MEMORY = 6,       /* a pool is neither device memory nor device-accessible pinned host memory */
  PA_ERR_CAPACITY = 7      /* block manager: not enough free blocks (or output space); nothing changed */
} pa_status;

/* Static, human-readable name of a status code.  Never NULL. */
const char* pa_status_str(pa_status s);

/*
 * Fused rotate-half RoPE + KV-cache store ([Pico-vLLM] §2: position encoding
 * fused with the cache write; §1: rotate_half computed in place; [mini-llm]
 * §3.1: the slot of a token is a row of a physical block).
 *
 * For every token i in [0, T) with slot s = slot_mapping[i] >= 0 and position
 * p = positions[i]:
 *   k_cache[s / bs][g][s % bs][:] = bf16(rope(k[i][g][:], p))  for every KV head g
 *   v_cache[s / bs][g][s % bs][:] = v[i][g][:]  (bits copied)  for every KV head g
 *   q[i][h][:]                    = bf16(rope(q[i][h][:], p))  for every query head h (in place)
 * A token with a negative slot is padding: nothing is written for it (its q,
 * k and v rows may be read, and q is left unchanged).
 * rope pairs element j with element j + D/2 (j < D/2):
 *   y[j]       = fl(fl(x[j] * c[j]) - fl(x[j + D/2] * s[j]))
 *   y[j + D/2] = fl(fl(x[j + D/2] * c[j]) + fl(x[j] * s[j]))
 * with c = cos_sin[p][0 .. D/2), s = cos_sin[p][D/2 .. D), every operation
 * one fp32 IEEE operation rounded to nearest even (no fused multiply-add), and
 * the result rounded to bf16 (nearest even).
 *
 * q            bf16 [T][Hq][D], rotated in place; may be NULL (then only k is rotated).
 * k, v         bf16 [T][Hkv][D].
 * k_cache, v_cache  bf16 [num_blocks][Hkv][block_size][D].
 * slot_mapping int32 [T]; positions int32 [T].
 * cos_sin      fp32 [max_pos][D]: cos of the D/2 angles, then their sin.
 * T == 0 is a no-op that returns PA_OK.
 */
pa_status pa_cache_store(void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                         const int32_t* slot_mapping, const int32_t* positions,
                         const float* cos_sin, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int64_t num_blocks, int32_t max_pos,
                         pa_stream_t stream);

/*
 * Bytes of workspace pa_decode needs for split-K decoding with this
 * partition size: fp32 partial outputs [B][Hq][P][D] followed by fp32
 * log-sum-exps [B][Hq][P], P = ceil(max_context_len / partition_size).
 * partition_size 0 (single pass) needs none; -1 sizes the library's own
 * choice (pa_decode_partition_size).  Returns 0 for invalid arguments.
 */
size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * The partition size pa_decode uses when asked to choose (partition_size
 * -1): 0 (single pass) when the B * Hkv (sequence, KV head) pairs alone give
 * every compute unit a workgroup, or when max_context_len is at most 128;
 * otherwise the smallest of 128, 256 and 512 tokens whose grid,
 * B * Hkv * ceil(max_context_len / P), stays within two workgroups per compute
 * unit with at most 64 partitions per sequence; failing that 512, doubled while
 * a sequence would need more than 64 partitions.  Host-only; reads the
 * device's compute-unit count once.
 */
int32_t pa_decode_partition_size(int32_t B, int32_t Hkv, int32_t max_context_len);

/*
 * Paged GQA decode ([Pico-vLLM] §2 decode kernel with Flash-Attention-style
 * tiling; Flash Decode in the H200 comparison; [mini-llm] §3.1):
 *   out[b][h][:] = sum_{t < L_b} softmax_t(scale * q[b][h] . K_b[t][g]) V_b[t][g],
 *   g = h / (Hq / Hkv), L_b = context_lens[b]; L_b == 0 gives zeros.
 * The new token's K/V must already be in the cache (pa_cache_store) and q
 * already rotated.  One workgroup serves all query heads of one KV head, so
 * each K/V byte is read once per step.  Accumulation is fp32; out is rounded
 * to bf16 (nearest even).
 *
 * out, q          bf16 [B][Hq][D]; out may not alias q.
 * block_tables    int32 [B][max_blocks]; entries past ceil(L_b/16) may be
 *                 loaded (inside the row) but are never used as block ids.
 * context_lens    int32 [B].
 * max_context_len host-known bound on context_lens (sizes the grid; no
 *                 device-to-host read).
 * partition_size  0: one pass over each sequence; > 0: split-K (Flash
 *                 Decode) with partitions of that many tokens (a multiple of
 *                 16), combined by a log-sum-exp reduce; -1: library's choice.
 * workspace       device memory of at least pa_decode_workspace_bytes(...)
 *                 bytes when split-K is used (may be NULL otherwise).
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * The two stages of split-K decode, for callers that place or exchange the
 * partials themselves (e.g. partials computed on several devices for
 * disjoint token ranges and combined on one).  pa_decode with
 * partition_size > 0 is exactly pa_decode_partitions followed by
 * pa_decode_combine on the same workspace.
 *
 * pa_decode_partitions: partition p of sequence b covers tokens
 * [p*P, min((p+1)*P, L_b)).  For every non-empty partition it writes
 *   o_part[b][h][p][:] = sum_t e^(s_t - m) V[t] / sum_t e^(s_t - m)   (fp32)
 *   lse[b][h][p]       = log2(sum_t 2^(s_t*log2(e)))                  (fp32, base 2)
 * with s_t = scale * q[b][h] . K[t][g].  Partitions with p*P >= L_b are not
 * written.  o_part is [B][Hq][num_partitions][D] and lse is
 * [B][Hq][num_partitions], num_partitions = ceil(max_context_len / P).
 *
 * pa_decode_combine: for every (b, h) with L_b > 0 and n = ceil(L_b / P),
 *   M = max_{p<n} lse_p, w_p = 2^(lse_p - M),
 *   out[b][h][:] = bf16(sum_p w_p o_part_p / sum_p w_p);
 * L_b == 0 gives zeros.
 */
pa_status pa_decode_partitions(float* o_part, float* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t block_size, int32_t max_blocks,
                               int32_t max_context_len, float scale, int32_t partition_size,
                               pa_stream_t stream);

pa_status pa_decode_combine(void* out, const float* o_part, const float* lse,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t D,
                            int32_t max_context_len, int32_t partition_size, pa_stream_t stream);

/*
 * Causal paged chunked prefill ([Pico-vLLM] §2 prefill kernel; [mini-llm]
 * §3.3 Chunked Prefill).  Sequence b owns query rows
 * [query_start_loc[b], query_start_loc[b+1]) (C_b rows) and has
 * L_b = context_lens[b] cached tokens, its chunk's own keys included (store
 * the chunk with pa_cache_store first).  Row i of the chunk sits at position
 * L_b - C_b + i and attends keys t <= L_b - C_b + i:
 *   out[r][h][:] = sum_t softmax_t(scale * q[r][h] . K_b[t][g]) V_b[t][g].
 * QK^T and PV run on bf16 matrix cores with fp32 accumulation; out is
 * rounded to bf16 (nearest even).
 *
 * out, q           bf16 [T][Hq][D] packed by sequence; out may not alias q.
 * query_start_loc  int32 [B+1], non-decreasing, query_start_loc[B] == T,
 *                  C_b <= L_b.
 * max_query_len    host-known bound on C_b (sizes the grid).
 */
pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                     int32_t D, int32_t block_size, int32_t max_blocks, int32_t max_query_len,
                     float scale, pa_stream_t stream);

/*
 * Multi-query paged decode for speculative-decoding verification ([mini-llm]
 * §3.6: the target model checks the K draft tokens in one pass, equivalent to
 * one prefill).  Sequence b brings NQ consecutive queries (the last accepted
 * token and NQ - 1 drafts), all already stored in the cache with
 * pa_cache_store; query i sits at position L_b - NQ + i and attends keys
 * t <= L_b - NQ + i:
 *   out[b][i][h][:] = sum_t softmax_t(scale * q[b][i][h] . K_b[t][g]) V_b[t][g].
 * This is pa_prefill with C_b = NQ for every sequence, computed the way
 * pa_decode is: one workgroup per (sequence, KV head, partition) serves its
 * NQ * G (query, head) rows, so each K/V byte is read once; split-K partials
 * are combined by the same log-sum-exp reduce.
 *
 * out, q          bf16 [B][NQ][Hq][D]; out may not alias q.
 * NQ              1 <= NQ and NQ * (Hq / Hkv) <= 32, else PA_ERR_UNSUPPORTED
 *                 (NQ = 1 is pa_decode).
 * context_lens    int32 [B]; L_b >= NQ is a device-side precondition
 *                 (a query whose position would be negative sees no key and
 *                 gets zeros); L_b == 0 gives zeros.
 * partition_size  as for pa_decode, except that -1 (library choice) takes
 *                 1024 where pa_decode_partition_size gives 512, the rows of a
 *                 (sequence, KV head) fill two 16-row tiles (NQ * Hq / Hkv > 16)
 *                 and B * Hkv * ceil(max_context_len / 1024) is at least the
 *                 device's CU count: partitions of 513 to 1024 tokens run as one
 *                 chunk of 8 waves per workgroup.
 * other arguments as for pa_decode; the workspace holds fp32 partials
 * [B][NQ][Hq][P][D] followed by log-sum-exps [B][NQ][Hq][P]
 * (pa_decode_multi_workspace_bytes resolves -1 the same way).
 */
size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t NQ, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t max_context_len, int32_t partition_size);

pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t NQ, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                          int32_t max_blocks, int32_t max_context_len, float scale,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          pa_stream_t stream);

/*
 * The decode step with the store folded into the decode kernel ([Pico-vLLM]
 * §2: fused RoPE + KV-cache store and the paged decode kernel; "H200
 * comparison": Flash Decode's split and reduce; [mini-llm] §3.1: the new
 * token's row in its 16-token block).  For every sequence b with
 * L_b = context_lens[b] > 0 the new token sits at position L_b - 1:
 *   1. its k (rotated) and v are written to row (L_b-1) % 16 of block
 *      block_tables[b][(L_b-1) / 16] of every KV head, as pa_cache_store with
 *      slot = that row and position = L_b - 1 would write them;
 *   2. out[b] = pa_decode of the rotated q over the L_b tokens, new one
 *      included, with the same partition size and the same reduce.
 * The results (out and the pools) are bit-identical to pa_cache_store
 * followed by pa_decode; the step takes two launches (one with a single
 * pass) instead of three.  q is only read (the separate store rotates it in
 * place; this call does not).  L_b = 0: out[b] is zero and nothing is written.
 *
 * q, k, v          bf16 [B][Hq][D], [B][Hkv][D], [B][Hkv][D]: the new token,
 *                  not rotated.
 * cos_sin          fp32 [max_pos][D] as for pa_cache_store; max_pos must be at
 *                  least max_context_len, else PA_ERR_SHAPE.
 * other arguments  as for pa_decode, the workspace included
 *                  (pa_decode_workspace_bytes).
 * Device-side preconditions as for pa_decode, plus: the new token's block is
 * owned by its sequence alone (ref_count 1: copy-on-write first) and L_b - 1
 * < max_pos.
 */
pa_status pa_decode_step(void* out, const void* q, const void* k, const void* v, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                         const float* cos_sin, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t max_blocks, int32_t max_context_len,
                         int32_t max_pos, float scale, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, pa_stream_t stream);

/*
 * The first stage of pa_decode_step with partition_size > 0: the store of the
 * new token folded into pa_decode_partitions.  It writes the new K/V rows
 * exactly as pa_decode_step does and o_part / lse exactly as
 * pa_decode_partitions would after pa_cache_store; pa_decode_combine then
 * gives pa_decode_step's out.  Arguments as for pa_decode_step and
 * pa_decode_partitions.
 */
pa_status pa_decode_step_partitions(float* o_part, float* lse, const void* q, const void* k,
                                    const void* v, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    const float* cos_sin, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t block_size, int32_t max_blocks,
                                    int32_t max_context_len, int32_t max_pos, float scale,
                                    int32_t partition_size, pa_stream_t stream);

/*
 * Decode with shared prefixes read once ([mini-llm] §3.4: full blocks shared
 * by several sequences, ref_count > 1; [Pico-vLLM] §3: requests sharing a
 * system prompt).  The same result as pa_decode (up to rounding order), but
 * the keys of a prefix shared by a group of sequences are read once for
 * several sequences: each sequence's own split-K partitions cover only its
 * tokens after the prefix, and one log-sum-exp reduce merges them with the
 * prefix partials.  Two ways, the library's choice:
 *   - one partition launch: work items of one 16-row tile of (sequence, head)
 *     rows, 16 / G sequences of a group over one 512-token partition of their
 *     prefix or one sequence's heads over one partition of its suffix; taken when
 *     there is a prefix, the suffix partitions are at most 512 tokens and the
 *     prefix items number at most one per CU;
 *   - otherwise the group's queries (every sequence and head, 96 rows per
 *     workgroup) attend each partition of the prefix (512 tokens, 128 to 1024
 *     when the grid or the workspace slots need it) together on the matrix
 *     cores, then the suffix partitions, then the reduce.
 * It pays when many sequences share a long prefix (measured: 2.1x pa_decode
 * for 128 sequences sharing 4096 tokens); for a few sequences on a prefix that
 * stays in the last-level cache, pa_decode is faster.
 *
 * group_start     int32 [num_groups + 1], device memory: group i is sequences
 *                 group_start[i] .. group_start[i+1]-1 (contiguous, ascending,
 *                 disjoint).  May be NULL when num_groups == 0.
 * prefix_lens     int32 [B], device memory: the shared-prefix tokens of each
 *                 sequence, a multiple of 16 (whole blocks), equal within a
 *                 group, at most max_prefix and at most L_b; 0 for a sequence
 *                 in no group (it is then decoded as by pa_decode).
 * max_group_size  bound on group sizes (sizes the grid); max_prefix bound on
 *                 prefix_lens, a multiple of 16, at most max_context_len.
 * max_suffix_len  bound on L_b - prefix_lens[b] (sizes the suffix grid), at
 *                 most max_context_len.
 * partition_size  suffix partitions: > 0 (a multiple of 16) or -1 (library's
 *                 choice: pa_decode's rule applied to max_suffix_len, at least
 *                 64; the workspace query then assumes 64).
 * workspace       pa_decode_shared_prefix_workspace_bytes(...) bytes of
 *                 device memory: fp32 partials [B][Hq][slots][D] and
 *                 log-sum-exps [B][Hq][slots], slots = ceil(max_suffix_len /
 *                 P) + ceil(max_prefix / Pg) with Pg the prefix partition
 *                 (the query assumes Pg = 128, an upper bound); a call whose
 *                 slots cannot fit 64 with any Pg is PA_ERR_UNSUPPORTED.
 * Device-side preconditions as for pa_decode, plus: within a group the first
 * prefix_lens/16 block-table entries are identical (the prefix is read
 * through the group's first sequence's table).
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                               int32_t max_suffix_len, int32_t max_prefix,
                                               int32_t partition_size);

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens, int32_t B,
                                  int32_t num_groups, int32_t max_group_size, int32_t max_prefix,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                  int32_t max_blocks, int32_t max_context_len, int32_t max_suffix_len,
                                  float scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, pa_stream_t stream);

/*
 * Copy-on-write block copies inside one pair of pools ([mini-llm] §3.4: a
 * block shared by several sequences, ref_count > 1, is copied to a freshly
 * allocated block before one of them writes it).  For every i < n, the whole
 * [Hkv][block_size][D] tile of block src_blocks[i] is copied, bit for bit, to
 * block dst_blocks[i], in k_cache and in v_cache.
 *
 * k_cache, v_cache         bf16 [num_blocks][Hkv][block_size][D], device memory.
 * src_blocks, dst_blocks   int32 [n], device memory (or device-accessible
 *                          pinned host memory); may be NULL when n == 0.
 * Device-side preconditions: every id is in [0, num_blocks); the destination
 * ids are distinct and none is also a source (copies run in no fixed order).
 * PA_ERR_MEMORY if a pointer is neither device memory nor device-accessible
 * pinned host memory (pageable memory is refused before any launch).
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t n, int32_t Hkv, int32_t D,
                         int32_t block_size, int64_t num_blocks, pa_stream_t stream);

/*
 * Block moves between two pairs of pools: swap-out to and swap-in from host
 * memory ([mini-llm] §3.5: a preempted sequence's blocks go to CPU memory and
 * come back into newly allocated device blocks instead of being recomputed).
 * For every i < n:  dst_k[dst_blocks[i]] = src_k[src_blocks[i]] and the same
 * for V, whole [Hkv][block_size][D] tiles, bit for bit.
 *
 * dst_k, dst_v, src_k, src_v  bf16 pools [*][Hkv][block_size][D]; each either
 *                             device memory or pinned host memory the device
 *                             can access (e.g. hipHostMalloc): a kernel moves
 *                             the data over PCIe, so device-to-host,
 *                             host-to-device and device-to-device all work.
 * src_blocks, dst_blocks      int32 [n], device or pinned host memory; may be
 *                             NULL when n == 0.
 * Device-side preconditions: ids in range of their pools; destination ids
 * distinct; the source and destination tiles do not overlap.
 */
pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t n,
                         int32_t Hkv, int32_t D, int32_t block_size, pa_stream_t stream);

/*
 * Fused RMSNorm + residual add ([Pico-vLLM] §2 kernel layer; Qwen2.5's
 * RMSNorm), per row t of H values:
 *   r'        = bf16(x[t] + residual[t])   written back over residual[t]
 *   out[t][j] = bf16(weight[j] * r'[j] / sqrt(mean_j(r'[j]^2) + eps))
 * in fp32 with one final rounding (nearest even).  residual NULL: plain
 * RMSNorm of x (r' = x, nothing written back).
 * out, x, residual bf16 [T][H]; weight bf16 [H]; H a multiple of 8, at most
 * 16384, else PA_ERR_UNSUPPORTED.  out may alias neither x nor residual.
 */
pa_status pa_rmsnorm_residual(void* out, void* residual, const void* x, const void* weight,
                              int32_t T, int32_t H, float eps, pa_stream_t stream);

/*
 * Fused SwiGLU ([Pico-vLLM] §2 kernel layer; Qwen2.5's MLP activation), per
 * row t: gate = gate_up[t][0 .. I), up = gate_up[t][I .. 2I),
 *   out[t][j] = bf16(gate[j] / (1 + e^(-gate[j])) * up[j])
 * in fp32 (hardware exp2 and reciprocal: a few fp32 ulps before the one
 * rounding to bf16, nearest even); results down to the subnormals are kept
 * for large negative gates.
 * out bf16 [T][I]; gate_up bf16 [T][2I]; I a multiple of 8 and at most 2^26,
 * T at most 2^31 - 1, else PA_ERR_UNSUPPORTED.
 */
pa_status pa_swiglu(void* out, const void* gate_up, int64_t T, int32_t I, pa_stream_t stream);

/*
 * For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: pa_decode with its split-K
 * workspace in a file-scope device array of the library (one per GPU, held
 * until the process ends) instead of a caller buffer.  Same arguments,
 * semantics, results (bit for bit) and errors as pa_decode, minus workspace.
 * Allocates nothing, on the host or the device.
 *
 * Limit: the workspace pa_decode would need, pa_decode_workspace_bytes(B, Hq,
 * Hkv, D, max_context_len, P) for the partition size used, must be at most
 * PA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. 64 sequences x 12 query heads
 * with 20 partitions at D = 128), else PA_ERR_WORKSPACE and nothing is
 * enqueued.  All calls on one GPU share its array: calls that overlap on one
 * GPU (other streams or threads) race and must not be issued.  The array's
 * device address is looked up on the first call on each GPU; PA_ERR_HIP if
 * that fails.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t max_blocks, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_stream_t stream);

/*
 * Host block manager ([mini-llm] §3.1 physical blocks with ref counts, O(1)
 * free list, per-sequence logical->physical table; §3.4 full blocks shared by
 * content hash, copy-on-write; §3.5 swap-out / swap-in; [Pico-vLLM] §3 LRU
 * eviction of cached blocks with lazy deletion).  Host memory only; it
 * produces the block tables and slot mappings the kernels consume and the
 * block pairs pa_copy_blocks / pa_swap_blocks move.  Not thread-safe: one
 * caller at a time per manager.  Block size 16.
 *
 * Policy: a full block's hash chains the previous block's hash with its 16
 * tokens (a hit is confirmed by comparing the tokens); hashes are registered
 * by pa_bm_commit once the tokens' K/V are written; prefix reuse stops at the
 * first miss and always leaves at least one prompt token to compute; a
 * released hashed block stays cached (evictable) until an allocation finds no
 * never-cached free block, then the least recently released one is reused.
 * Errors leave the manager unchanged.
 */
typedef struct pa_block_manager pa_block_manager;

/* NULL on invalid sizes (num_blocks <= 0, num_host_blocks < 0, block_size != 16)
   or when out of host memory. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);

/* Free + evictable cached blocks; cached (released, hashed) blocks; free host slots;
   a block's ref count (-1 for a bad id). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* m);
int32_t pa_bm_num_cached_blocks(const pa_block_manager* m);
int32_t pa_bm_num_free_host_blocks(const pa_block_manager* m);
int32_t pa_bm_block_ref(const pa_block_manager* m, int32_t block);

/* New sequence with a prompt of n_tokens token ids (host array).  Reuses cached
   blocks of the longest identical full-block prefix (ref_count + 1) and allocates
   the rest; *n_cached_tokens = prompt tokens whose K/V are already in the cache
   (a multiple of 16, < n_tokens).  PA_ERR_CAPACITY if blocks run out. */
pa_status pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                             int32_t n_tokens, int32_t* n_cached_tokens);

/* The first n_computed_tokens of the sequence have their K/V written: register the
   hashes of its full blocks in that range (first writer of a content wins). */
pa_status pa_bm_commit(pa_block_manager* m, int64_t seq_id, int32_t n_computed_tokens);

/* Reserve the slot of the sequence's next token (decode): a new block when the last
   is full; if the last block is shared (after pa_bm_fork), the sequence first moves
   to a fresh block and *cow_src / *cow_dst name the copy to run (else both -1). */
pa_status pa_bm_append_token(pa_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot,
                             int32_t* cow_src, int32_t* cow_dst);

/* Child shares every block of the parent (ref_count + 1 each). */
pa_status pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id);

/* Release every block (or host slot) of the sequence. */
pa_status pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id);

/* Tokens held by the sequence (-1 if unknown). */
int32_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id);

/* The sequence's block table into out[capacity]; *n_blocks = its length (set even
   when capacity is too small, which returns PA_ERR_CAPACITY). */
pa_status pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* out,
                            int32_t capacity, int32_t* n_blocks);

/* slot_mapping[i] = slot of token start + i, i < n (tokens must be reserved). */
pa_status pa_bm_slots(const pa_block_manager* m, int64_t seq_id, int32_t start, int32_t n,
                      int32_t* slot_mapping);

/* Swap-out: the sequence's device blocks get host slots (pairs written to
   device_blocks[i] -> host_blocks[i], *n of them) and are released.  Swap-in:
   new device blocks for its host slots (host_blocks[i] -> device_blocks[i]);
   the slots are released.  Run the pairs with pa_swap_blocks. */
pa_status pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int32_t* device_blocks,
                         int32_t* host_blocks, int32_t capacity, int32_t* n);
pa_status pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int32_t* host_blocks,
                        int32_t* device_blocks, int32_t capacity, int32_t* n);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
