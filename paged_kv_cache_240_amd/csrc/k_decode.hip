// Paged GQA decode for gfx950: one workgroup per (sequence, KV head,
// partition) serving all G query heads of that KV head, so every K/V byte of
// the step is read from HBM once.
//
// Operation (Pico-vLLM write-up, §2: paged decode kernel in the manner of
// Flash Attention; H200 comparison: Flash Decode; §1: GQA; mini-llm-engine
// post, §3.1: K/V in 16-token physical blocks reached through a per-sequence
// block table): out[b,h] = softmax(scale * q[b,h] K_b^T) V_b over the L_b
// cached tokens of sequence b, K_b/V_b the rows of KV head h / G.
//
// Workgroup = 4 independent waves; the tokens of a partition (split-K) or of
// the whole sequence (single pass) are walked in chunks of 4*WB blocks, wave w
// taking blocks w, w+4, ..., w+4(WB-1) of each chunk (WB = 8 blocks per wave
// for partitions of more than 256 tokens and for single passes; 4 and 2 for
// partitions of up to 256 and 128 tokens, whose ring then holds every block
// of the wave at once).  Both products run on
// v_mfma_f32_16x16x32_bf16 with the G query heads padded to 16:
//   QK   S^T = K Q^T per block: the key tile is the A operand as it lies in
//        memory (lane = key, 16 contiguous bytes of its row per k-step), the
//        query rows the B operand.  A lane ends up with 4 consecutive keys of
//        one head; rows past the range become -inf by a select.
//   P    after the WB blocks of a chunk, the running max per head (in-lane max,
//        then two cross-row swaps: a head's 32 keys of a block pair live in
//        4 lanes), p = 2^((s - m) * scale * log2 e), rounded to bf16 in place:
//        the 8 p of a lane for two blocks are exactly its A operand of PV.
//   PV   O = P V per block pair (32 keys): lane (n, g) loads rows 4g..4g+3 of
//        each block, D/16 consecutive dims from n*D/16; v_perm pairs the rows
//        per dim, which makes the B operand of the output tile holding dims
//        n*D/16 + s.  A ninth product against a ones operand accumulates the
//        normaliser l from the same rounded p the outputs use.
// Rows past the range are redirected to row 0 of their block when V is
// loaded, so NaN in unused slots never meets a zero probability.
// K and V blocks stream through a ring of DEPTH register buffers in the
// order K0..K(WB-1), V0..V(WB-1), K0' ... so loads run DEPTH blocks ahead of
// the arithmetic across phase and chunk boundaries; with at most 4 blocks per
// wave the ring holds all 2*WB, so no V load waits for a K block to arrive.  Loads past the last block of
// the range re-read the last valid block (an L2 hit) instead of branching.
// The waves never synchronise until the end, where their (max, sum, output)
// triples are combined through LDS.  The output is the normalised bf16 row
// (single pass) or an fp32 partial plus its base-2 log-sum-exp (split-K),
// reduced by combine_kernel (Flash Decode's reduce).

#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_DEPTH_ONE
#define PA_DECODE_DEPTH_ONE 8
#endif

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kWaveBlocks = 8;                           // blocks per wave per chunk (streaming)
constexpr int kChunkBlocks = kWaves * kWaveBlocks;       // 32
constexpr int kChunkTokens = kChunkBlocks * kBlockSize;  // 512

// Blocks per wave for a split-K launch whose partitions hold at most
// `partition_size` tokens and fit one chunk.
constexpr int wave_blocks_for(int partition_size) {
  return partition_size <= kWaves * 2 * kBlockSize ? 2 : partition_size <= kWaves * 4 * kBlockSize ? 4 : 8;
}
constexpr int kDepth = 4;     // blocks in flight per wave when chunks repeat (ring slots must cycle per chunk)
constexpr int kDepthOne = PA_DECODE_DEPTH_ONE;  // ... when the range is a single chunk
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // two bf16 1.0

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma_bf16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 2^x on v_exp_f32 directly: results below the fp32 normal range may flush to
// zero, which only touches probabilities already under 2^-126 of the maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Log-sum-exp combine of split-K partials (Flash Decode's reduce) for one
// query row of a sequence of L tokens, by one wave (lane = 0..63); a row is a
// query head (or, for multi-query decode, a (query, head) pair).  Every load
// is issued before L is used: lane j < num_parts reads lse[j] and each lane
// reads one 16-byte piece of every partial it may need (indices clamped into
// the workspace); partitions past ceil(L / P) were never written and are
// removed by selects, not arithmetic, so stale workspace contents (NaN
// included) cannot leak.  Then: M = max lse,
// out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
// CASC (shared-prefix decode): the row's valid slots are its
// ceil((L - start) / part_tokens) suffix partitions, from slot 0, and the
// ceil(start / prefix_tokens) prefix partitions, from slot slot0.
template <int D, int MAXP, bool CASC = false>
__device__ __forceinline__ void combine_row(uint16_t* __restrict__ out, const float* __restrict__ o_part,
                                            const float* __restrict__ lse, int L, int64_t row,
                                            int num_parts, int part_tokens, int lane, int start = 0,
                                            int slot0 = 0, int prefix_tokens = 1) {
  constexpr int PIECES = D / 4;     // float4 pieces of one partial row
  constexpr int PPI = 64 / PIECES;  // partials covered by one wave-wide step
  constexpr int NSTEP = MAXP / PPI;
  const int piece = lane % PIECES, sub = lane / PIECES;
  const float* ls = lse + row * num_parts;
  const float* src = o_part + row * num_parts * D + piece * 4;
  const float my_lse = ls[min(lane, num_parts - 1)];
  float4 t[NSTEP];
  float tl[NSTEP];
#pragma unroll
  for (int k = 0; k < NSTEP; ++k) {
    const int i = min(sub + PPI * k, num_parts - 1);
    t[k] = *reinterpret_cast<const float4*>(src + (int64_t)i * D);
    tl[k] = ls[i];
  }
  uint16_t* o = out + row * D + piece * 4;
  if (L <= 0) {
    if (sub == 0) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const int n = CASC ? (L - start + part_tokens - 1) / part_tokens : (L + part_tokens - 1) / part_tokens;
  const int n_pre = CASC ? (start + prefix_tokens - 1) / prefix_tokens : 0;
  auto valid = [&](int i) { return i < n || (CASC && i >= slot0 && i < slot0 + n_pre); };
  const float M = wave_max(valid(lane) ? my_lse : -INFINITY);
  if (M == -INFINITY) {  // no partition saw a key of this row (multi-query rows before the cache)
    if (sub == 0) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const float W = wave_sum(valid(lane) ? exp2f(my_lse - M) : 0.f);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < NSTEP; ++k) {
    const bool in = valid(sub + PPI * k);
    const float w = in ? exp2f(tl[k] - M) : 0.f;
    acc.x += in ? w * t[k].x : 0.f; acc.y += in ? w * t[k].y : 0.f;
    acc.z += in ? w * t[k].z : 0.f; acc.w += in ? w * t[k].w : 0.f;
  }
  if constexpr (PPI >= 4) {
    acc.x += swap16(acc.x); acc.y += swap16(acc.y); acc.z += swap16(acc.z); acc.w += swap16(acc.w);
  }
  acc.x += swap32(acc.x); acc.y += swap32(acc.y); acc.z += swap32(acc.z); acc.w += swap32(acc.w);
  if (sub == 0) {
    const float inv = 1.f / W;
    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv),
                                              pack_bf16x2(acc.z * inv, acc.w * inv));
  }
}

// The same reduce for more than 64 partitions: loops over the partitions.
template <int D>
__device__ __forceinline__ void combine_row_many(uint16_t* __restrict__ out, const float* __restrict__ o_part,
                                                 const float* __restrict__ lse, int L, int64_t row,
                                                 int num_parts, int part_tokens, int lane) {
  constexpr int PIECES = D / 4;
  constexpr int PPI = 64 / PIECES;
  const int piece = lane % PIECES, sub = lane / PIECES;
  uint16_t* o = out + row * D + piece * 4;
  if (L <= 0) {
    if (sub == 0) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const int n = (L + part_tokens - 1) / part_tokens;
  const float* ls = lse + row * num_parts;
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, ls[i]);
  M = wave_max(M);
  if (M == -INFINITY) {  // no partition saw a key of this row
    if (sub == 0) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  float W = 0.f;
  for (int i = lane; i < n; i += 64) W += exp2f(ls[i] - M);
  W = wave_sum(W);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = o_part + row * num_parts * D + piece * 4;
#pragma unroll 8
  for (int i = sub; i < n; i += PPI) {
    const float w = exp2f(ls[i] - M);
    const float4 t = *reinterpret_cast<const float4*>(src + (int64_t)i * D);
    acc.x = fmaf(w, t.x, acc.x); acc.y = fmaf(w, t.y, acc.y);
    acc.z = fmaf(w, t.z, acc.z); acc.w = fmaf(w, t.w, acc.w);
  }
  if constexpr (PPI >= 4) {
    acc.x += swap16(acc.x); acc.y += swap16(acc.y); acc.z += swap16(acc.z); acc.w += swap16(acc.w);
  }
  acc.x += swap32(acc.x); acc.y += swap32(acc.y); acc.z += swap32(acc.z); acc.w += swap32(acc.w);
  if (sub == 0) {
    const float inv = 1.f / W;
    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv),
                                              pack_bf16x2(acc.z * inv, acc.w * inv));
  }
}

// Inputs of the fused decode step (FUSED kernels only): the new token of
// every sequence, not yet rotated, and the rotation table.
struct StepArgs {
  const uint16_t* k_new;  // bf16 [B][Hkv][D]
  const uint16_t* v_new;  // bf16 [B][Hkv][D]
  const float* cos_sin;   // fp32 [max_pos][D]: cos | sin of each position
};

// Shared-prefix decode in one launch (CASC): grid item x is either 16 / G
// sequences of a group over prefix partition pp of the group's shared prefix
// (rows: those sequences times the G heads, one 16-row tile; keys read through
// the group's first sequence's table; partials in slot slot0 + pp) or one
// sequence's G heads over partition sp of its tokens after its prefix
// (partials in slot sp).  Every row sees every key of its item's range.
struct CascItems {
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int n_pre;       // prefix items: groups * max_sub * pre_parts (first in the grid)
  int max_sub;     // prefix items per group and partition
  int pre_parts;   // prefix partitions per group
  int pre_tokens;  // prefix partition size
  int suf_parts;   // suffix partitions per sequence
  int suf_tokens;  // suffix partition size
  int slot0;       // first prefix slot
};

// Rotate-half RoPE of 8 consecutive dims j..j+7 of the first half (a) and
// their partners j+D/2.. (b): lo = a cos - b sin, hi = b cos + a sin, each
// product and each sum rounded to fp32 on its own (no fused multiply-add),
// then rounded to bf16 to nearest even: the operation order of the fused
// RoPE + store kernel, so both produce the same bits.
__device__ __forceinline__ void rope_rotate8(const uint4 a, const uint4 b, const float (&c)[8],
                                             const float (&sn)[8], uint4& lo, uint4& hi) {
#pragma clang fp contract(off)
  float fa[8], fb[8], l[8], h[8];
  unpack_bf16x8(a, fa);
  unpack_bf16x8(b, fb);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ac = fa[e] * c[e];
    const float bs = fb[e] * sn[e];
    const float bc = fb[e] * c[e];
    const float as = fa[e] * sn[e];
    l[e] = ac - bs;
    h[e] = bc + as;
  }
  lo = pack_bf16x8(l);
  hi = pack_bf16x8(h);
}

// Fused step, V of the new token's block or of a block past the range (which
// re-reads it): rows from r_new on take the new row (row r_new itself, and the
// rows past the range, which only meet p = 0 and would otherwise read row 0 --
// the new row's stale slot when r_new is 0).  A lane holds rows 4*quad ..
// 4*quad+3, HALF dwords each.
template <int SLOT, int HALF>
__device__ __forceinline__ void substitute_v_rows(uint32_t (&slot)[SLOT], const uint32_t* vrow,
                                                  int lane, int r_new) {
  const int quad = lane >> 4;
  uint32_t v[HALF];
#pragma unroll
  for (int w = 0; w < HALF; ++w) v[w] = vrow[w * 64 + lane];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int w = 0; w < HALF; ++w)
      slot[r * HALF + w] = 4 * quad + r >= r_new ? v[w] : slot[r * HALF + w];
}

// ONE: the range is a single chunk (split-K with partitions of at most
// 4*WB blocks), so the ring need not cycle and can be deeper; no refills past it.
// WB: blocks per wave per chunk (8, or 4 / 2 for short partitions).
// FUSED: the decode step's store folded in (see launch_decode_step): q and
// the new k arrive unrotated, and the new token's K/V row is written to the
// cache and used from registers.
template <int D, int G, bool SPLIT, bool ONE, bool FUSED, int WB = kWaveBlocks, bool CASC = false>
__global__ void __launch_bounds__(256, 2)  // 2 waves per SIMD: 8 streaming waves per CU
decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
              const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
              const int32_t* __restrict__ context_lens, int Hkv, int max_blocks,
              float scale_log2, int part_tokens, int num_parts, uint16_t* __restrict__ out,
              float* __restrict__ o_part, float* __restrict__ lse, const StepArgs st,
              const int32_t* __restrict__ starts, const CascItems ci) {
  static_assert(G >= 1 && G <= 8, "query heads per KV head: 1..8");
  static_assert(!CASC || (SPLIT && ONE && !FUSED), "shared-prefix items are single-chunk partitions");
  constexpr int NSEQ = CASC ? 16 / G : 1;  // sequences per workgroup
  constexpr int RM = NSEQ * G;             // rows: (sequence, head) pairs, at most 16
  static_assert(WB == 2 || WB == 4 || WB == 8, "blocks per wave: 2, 4 or 8");
  static_assert(ONE || WB == kWaveBlocks, "a cycling ring takes 8 blocks per wave");
  constexpr int CHUNK_BLOCKS = kWaves * WB;
  constexpr int CHUNK_TOKENS = CHUNK_BLOCKS * kBlockSize;
  constexpr int KS = D / 32;    // QK k-steps over the head dimension
  constexpr int DPL = D / 16;   // PV: dims per lane = output tiles of 16 columns
  constexpr int HALF = DPL / 2; // dwords of one V row piece
  constexpr int SLOT = 4 * KS;  // dwords per lane of a K block (16 bytes per k-step)
  static_assert(SLOT == 4 * HALF, "K and V blocks must occupy the same ring slot");
  constexpr int STEPS = 2 * WB;  // K0..K(WB-1) then V0..V(WB-1)
  constexpr int DEPTH = ONE ? (2 * WB < kDepthOne ? 2 * WB : kDepthOne) : kDepth;
  static_assert(DEPTH % 2 == 0 && (ONE || STEPS % DEPTH == 0), "ring slots must repeat per chunk");

  __shared__ __align__(16) float red[kWaves][RM][D];  // per-wave outputs, dim n*DPL+s at s*16+n
  __shared__ float st_m[kWaves][RM], st_l[kWaves][RM];
  // fused step: the new V row's pieces, one copy per wave (lane-major), and
  // the owner wave's new K row, parked between the prologue and their use
  __shared__ uint32_t new_v[FUSED ? kWaves * HALF * 64 : 1];
  __shared__ uint32_t new_k[FUSED ? SLOT * 64 : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar table reads
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int hq0 = g * G;
  // Rows r < R are (sequence seq0 + r / G, head hq0 + r % G); keys through the
  // table row of sequence b_tab; partials go to slot `slot`.  Without CASC: the
  // G heads of sequence b, partition p.
  int R = G, b_tab = b, slot = p, L, start = 0;
  int64_t seq0 = b;
  if constexpr (CASC) {
    int it = p;
    if (it < ci.n_pre) {
      const int pp = it % ci.pre_parts;
      it /= ci.pre_parts;
      const int gi = it / ci.max_sub, sg = it % ci.max_sub;
      const int q0 = ci.group_start[gi], q1 = ci.group_start[gi + 1];
      const int first = q0 + sg * NSEQ;
      if (first >= q1) return;
      const int pre = ci.prefix_lens[q0];
      start = pp * ci.pre_tokens;  // the item's range: [start, min(start + tokens, pre))
      if (start >= pre) return;
      L = min(start + ci.pre_tokens, pre);
      R = min(NSEQ, q1 - first) * G;
      seq0 = first;
      b_tab = q0;
      slot = ci.slot0 + pp;
    } else {
      it -= ci.n_pre;
      const int sp = it % ci.suf_parts, bb = it / ci.suf_parts;
      const int Lb = context_lens[bb];
      start = ci.prefix_lens[bb] + sp * ci.suf_tokens;
      if (start >= Lb) return;  // empty partition: not written, not combined
      L = min(start + ci.suf_tokens, Lb);
      seq0 = bb;
      b_tab = bb;
      slot = sp;
    }
  } else {
    L = context_lens[b];
    // split-K with starts: sequence b's partitions cover [starts[b], L) (a
    // shared prefix before it is attended elsewhere); starts[b] is whole blocks
    start = (SPLIT && starts != nullptr) ? starts[b] : 0;
  }
  const int32_t* bt_row = block_tables + (int64_t)b_tab * max_blocks;
  // The first chunk's table entries are requested before L is known (indices
  // clamped into the table; an entry past the sequence is never dereferenced:
  // it is replaced by the range's first block once L arrives), so the first
  // K/V loads wait for one round trip instead of two.
  const int lb0 = CASC ? start / kBlockSize : SPLIT ? (start + p * part_tokens) / kBlockSize : 0;
  const int lb_spec = lb0 + wave + kWaves * (threadIdx.x & (WB - 1));
  const int ent_spec = bt_row[min(lb_spec, max_blocks - 1)];
  const int ent_first = bt_row[min(lb0, max_blocks - 1)];  // lb0 may lie past a short suffix
  const int col = lane & 15, quad = lane >> 4;  // MFMA lane roles
  // B operand of QK: query row of head `col` (zero beyond G), 8 dims per
  // k-step; padding lanes read head 0 and discard it (a select, not a branch)
  uint4 qraw[KS];
  {
    const int rr = min(col, R - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ks] = *reinterpret_cast<const uint4*>(q + ((seq0 + rr / G) * Hq + hq0 + rr % G) * D +
                                                 ks * 32 + quad * 8);
  }
  // every start-up load is in flight before the emptiness test below
  asm volatile("" ::"v"(ent_spec), "s"(ent_first), "s"(L));

  int t_begin = 0, t_end = L;
  if (CASC) {
    t_begin = start;
  } else if (SPLIT) {
    t_begin = start + p * part_tokens;
    if (t_begin >= L) return;  // empty partition: not written, not combined
    t_end = min(t_begin + part_tokens, L);
  } else if (L <= 0) {
    for (int e = threadIdx.x; e < G * D / 2; e += blockDim.x)
      reinterpret_cast<uint32_t*>(out + ((int64_t)b * Hq + hq0) * D)[e] = 0u;
    return;
  }

  // Fused step: the new token sits at position L-1, row r_new of logical block
  // nb_new, the last block of the last range (own_wg).  The one wave whose
  // blocks include it (owner) rotates its k, writes the K/V row to the cache
  // and substitutes the K row into that block.  Every wave of own_wg
  // substitutes the V row into that block and into the blocks past the range,
  // which re-read it and send their rows to its row 0: the new row's stale
  // slot when r_new is 0.  The loads and the cos/sin row are requested here,
  // before the ring fill, and consumed after it.
  const int nb_new = (L - 1) / kBlockSize, r_new = (L - 1) % kBlockSize;
  const int lb_new = nb_new - lb0;  // in this range
  const bool own_wg = FUSED && (!SPLIT || p == (L - 1 - start) / part_tokens);
  const bool owner = own_wg && wave == lb_new % kWaves;
  const int c_new = lb_new / CHUNK_BLOCKS, i_new = (lb_new % CHUNK_BLOCKS) / kWaves;
  float cs_c[KS / 2][8], cs_s[KS / 2][8];
  uint4 kraw[KS];
  uint32_t vraw[HALF];
  int ent_new = 0;
  if constexpr (FUSED) {
    const float* cs = st.cos_sin + (int64_t)(L - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      const int j = ks * 32 + quad * 8;
      const float4 c0 = *reinterpret_cast<const float4*>(cs + j);
      const float4 c1 = *reinterpret_cast<const float4*>(cs + j + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(cs + D / 2 + j);
      const float4 s1 = *reinterpret_cast<const float4*>(cs + D / 2 + j + 4);
      cs_c[ks][0] = c0.x; cs_c[ks][1] = c0.y; cs_c[ks][2] = c0.z; cs_c[ks][3] = c0.w;
      cs_c[ks][4] = c1.x; cs_c[ks][5] = c1.y; cs_c[ks][6] = c1.z; cs_c[ks][7] = c1.w;
      cs_s[ks][0] = s0.x; cs_s[ks][1] = s0.y; cs_s[ks][2] = s0.z; cs_s[ks][3] = s0.w;
      cs_s[ks][4] = s1.x; cs_s[ks][5] = s1.y; cs_s[ks][6] = s1.z; cs_s[ks][7] = s1.w;
    }
    if (owner) {
      const uint16_t* kn = st.k_new + ((int64_t)b * Hkv + g) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kraw[ks] = *reinterpret_cast<const uint4*>(kn + ks * 32 + quad * 8);
      ent_new = bt_row[nb_new];
    }
    if (own_wg) {
      const uint16_t* vn = st.v_new + ((int64_t)b * Hkv + g) * D + col * DPL;
      if constexpr (HALF == 4) {
        const uint4 t = *reinterpret_cast<const uint4*>(vn);
        vraw[0] = t.x; vraw[1] = t.y; vraw[2] = t.z; vraw[3] = t.w;
      } else {
        const uint2 t = *reinterpret_cast<const uint2*>(vn);
        vraw[0] = t.x; vraw[1] = t.y;
      }
    }
  }

  floatx4_t o[DPL];  // O[head 4*quad+e][dim col*DPL+s] in o[s][e]
  floatx4_t lacc = {0.f, 0.f, 0.f, 0.f};  // l of head 4*quad+e (every column the same)
#pragma unroll
  for (int s = 0; s < DPL; ++s) o[s] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // raw-score max of head `col` (same in the 4 lanes of a head)

  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;
  const int nchunks = ONE ? 1 : (t_end - t_begin + CHUNK_TOKENS - 1) / CHUNK_TOKENS;
  const int last_lb = (t_end - 1) / kBlockSize;  // last logical block of the range
  const int lane_k = col * D + quad * 8;         // element offsets inside a block tile
  const int lane_v = col * DPL;
  const uint4 ones = make_uint4(kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2);

  // Block-table entries of this wave's 8 blocks of chunk c: one vector load,
  // lane j (mod 8) fetching the entry of block j; blocks past the range take
  // the last valid entry.  Fetched a chunk ahead and read with readlane, so a
  // ring refill never waits on the table.
  auto fetch_entries = [&](int c) -> int {
    const int lb = (t_begin + c * CHUNK_TOKENS) / kBlockSize + wave + kWaves * (lane & (WB - 1));
    return bt_row[min(lb, last_lb)];
  };
  // Ring step `step` (0..7 K blocks, 8..15 V blocks) of the chunk whose
  // entries are `ent`; `left` = rows of that block inside the range.
  auto load_step = [&](uint32_t (&slot)[SLOT], int ent, int step, int left) {
    const int i = step & (WB - 1);
    const int64_t base = (int64_t)__builtin_amdgcn_readlane(ent, i) * blk_stride + head_off;
    if (step < WB) {
      const uint16_t* src = k_cache + base + lane_k;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 t = load_stream16(src + ks * 32);
        slot[4 * ks] = t.x; slot[4 * ks + 1] = t.y; slot[4 * ks + 2] = t.z; slot[4 * ks + 3] = t.w;
      }
    } else {
      const uint16_t* src = v_cache + base + lane_v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * quad + r < left ? 4 * quad + r : 0;  // past the range: row 0 (finite)
        if constexpr (HALF == 4) {
          const uint4 t = load_stream16(src + row * D);
          slot[4 * r] = t.x; slot[4 * r + 1] = t.y; slot[4 * r + 2] = t.z; slot[4 * r + 3] = t.w;
        } else {
          const uint2 t = load_stream8(src + row * D);
          slot[2 * r] = t.x; slot[2 * r + 1] = t.y;
        }
      }
    }
  };
  auto rows_left = [&](int nt, int step) { return nt - (wave + kWaves * (step & (WB - 1))) * kBlockSize; };

  int ent_cur = lb_spec <= last_lb ? ent_spec : ent_first;  // == fetch_entries(0)
  int ent_nxt = ONE ? 0 : fetch_entries(nchunks > 1 ? 1 : 0);
  const int nt0 = min(CHUNK_TOKENS, t_end - t_begin);
  uint32_t ring[DEPTH][SLOT];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) load_step(ring[s], ent_cur, s, rows_left(nt0, s));

  uint4 qb[KS];
  if constexpr (FUSED) {
    uint4 qr[KS], kr[KS];
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      rope_rotate8(qraw[ks], qraw[ks + KS / 2], cs_c[ks], cs_s[ks], qr[ks], qr[ks + KS / 2]);
      if (owner) rope_rotate8(kraw[ks], kraw[ks + KS / 2], cs_c[ks], cs_s[ks], kr[ks], kr[ks + KS / 2]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = col < R ? qr[ks] : make_uint4(0u, 0u, 0u, 0u);
    if (own_wg) {
#pragma unroll
      for (int w = 0; w < HALF; ++w) new_v[(wave * HALF + w) * 64 + lane] = vraw[w];
    }
    if (owner) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        new_k[(4 * ks) * 64 + lane] = kr[ks].x;
        new_k[(4 * ks + 1) * 64 + lane] = kr[ks].y;
        new_k[(4 * ks + 2) * 64 + lane] = kr[ks].z;
        new_k[(4 * ks + 3) * 64 + lane] = kr[ks].w;
      }
      // the row for later steps (no load of this launch reads it back); the
      // pools are written only here, through the one row of the new token
      const int64_t row_off = (int64_t)ent_new * blk_stride + head_off + r_new * D;
      uint16_t* kw = const_cast<uint16_t*>(k_cache) + row_off;
      uint16_t* vw = const_cast<uint16_t*>(v_cache) + row_off;
      if (col == 0)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<uint4*>(kw + ks * 32 + quad * 8) = kr[ks];
      if (quad == 0) {
        if constexpr (HALF == 4)
          *reinterpret_cast<uint4*>(vw + col * DPL) = make_uint4(vraw[0], vraw[1], vraw[2], vraw[3]);
        else
          *reinterpret_cast<uint2*>(vw + col * DPL) = make_uint2(vraw[0], vraw[1]);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = col < R ? qraw[ks] : make_uint4(0u, 0u, 0u, 0u);
  }

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = t_begin + c * CHUNK_TOKENS;
    const int nt = min(CHUNK_TOKENS, t_end - c0);  // valid tokens of the chunk
    const int nt_next = min(CHUNK_TOKENS, t_end - c0 - CHUNK_TOKENS);
    floatx4_t st[WB];  // raw scores: keys 4*quad+e of block i, head col
    uint4 pa[WB / 2];  // bf16 probabilities: A operand of block pair j

    static_for<STEPS>([&](auto step_c) {
      constexpr int step = decltype(step_c)::value;
      uint32_t(&cur)[SLOT] = ring[step % DEPTH];
      constexpr int i = step & (WB - 1);

      if constexpr (step < WB) {
        // ---- QK on block i: S^T (16 keys x 16 heads) ---------------------------
        const int left = rows_left(nt, step);
        if constexpr (FUSED) {
          if (owner && c == c_new && i == i_new) {
#pragma unroll
            for (int d = 0; d < SLOT; ++d) cur[d] = col == r_new ? new_k[d * 64 + lane] : cur[d];
          }
        }
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = mfma_bf16(make_uint4(cur[4 * ks], cur[4 * ks + 1], cur[4 * ks + 2], cur[4 * ks + 3]),
                          qb[ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) st[i][e] = 4 * quad + e < left ? acc[e] : -INFINITY;
        // refill the slot just consumed
        constexpr int ns = step + DEPTH;
        if constexpr (ns < STEPS) load_step(cur, ent_cur, ns, rows_left(nt, ns));
        else if constexpr (!ONE) load_step(cur, ent_nxt, ns - STEPS, rows_left(nt_next, ns - STEPS));
      } else {
        if constexpr (step == WB) {
          // ---- P: online softmax over this wave's 8 blocks -------------------------
          // scores are finite or a masked -inf, so the NaN-propagating max is exact
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < WB; ++j)
            mx = maxn(maxn(mx, maxn(st[j][0], st[j][1])), maxn(st[j][2], st[j][3]));
          mx = maxn_swap32(maxn_swap16(mx));
          const float m_new = fmaxf(m_run, mx);
          // no key of this head in range yet: m stays -inf and every p is 0
          const float ref = m_new == -INFINITY ? 0.f : m_new * scale_log2;
          const float alpha = fast_exp2(m_run * scale_log2 - ref);
          m_run = m_new;
#pragma unroll
          for (int j = 0; j < WB / 2; ++j) {
            const floatx4_t& sa = st[2 * j];
            const floatx4_t& sb = st[2 * j + 1];
            pa[j].x = cvt_bf16x2(fast_exp2(fmaf(sa[0], scale_log2, -ref)), fast_exp2(fmaf(sa[1], scale_log2, -ref)));
            pa[j].y = cvt_bf16x2(fast_exp2(fmaf(sa[2], scale_log2, -ref)), fast_exp2(fmaf(sa[3], scale_log2, -ref)));
            pa[j].z = cvt_bf16x2(fast_exp2(fmaf(sb[0], scale_log2, -ref)), fast_exp2(fmaf(sb[1], scale_log2, -ref)));
            pa[j].w = cvt_bf16x2(fast_exp2(fmaf(sb[2], scale_log2, -ref)), fast_exp2(fmaf(sb[3], scale_log2, -ref)));
          }
          // rescale the accumulators: lane (col, quad) holds heads 4*quad+e
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), e));
            const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 4 + e));
            a[e] = quad == 0 ? lo : hi;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lacc[e] *= a[e];
#pragma unroll
            for (int s = 0; s < DPL; ++s) o[s][e] *= a[e];
          }
        }
        if constexpr (i % 2 == 1) {
          // ---- PV on blocks i-1, i: 32 keys ---------------------------------------
          uint32_t(&va)[SLOT] = ring[(step - 1) % DEPTH];
          uint32_t(&vb)[SLOT] = cur;
          if constexpr (FUSED) {
            // blocks i-1, i of this chunk, at or past the new block; two
            // separate tests on fixed slots: a merged call on a selected slot
            // address would force the whole ring into memory
            const int lb_i = c * CHUNK_BLOCKS + wave + kWaves * i;  // block i in the range
            if (own_wg && lb_i - kWaves >= lb_new)
              substitute_v_rows<SLOT, HALF>(va, new_v + wave * HALF * 64, lane, r_new);
            __builtin_amdgcn_sched_barrier(0);
            if (own_wg && lb_i >= lb_new)
              substitute_v_rows<SLOT, HALF>(vb, new_v + wave * HALF * 64, lane, r_new);
          }
          const uint4 pj = pa[i / 2];
#pragma unroll
          for (int s = 0; s < DPL; ++s) {
            const int w = s / 2;
            uint4 bv;
            if (s % 2 == 0) {
              bv.x = interleave_lo(va[w], va[HALF + w]);
              bv.y = interleave_lo(va[2 * HALF + w], va[3 * HALF + w]);
              bv.z = interleave_lo(vb[w], vb[HALF + w]);
              bv.w = interleave_lo(vb[2 * HALF + w], vb[3 * HALF + w]);
            } else {
              bv.x = interleave_hi(va[w], va[HALF + w]);
              bv.y = interleave_hi(va[2 * HALF + w], va[3 * HALF + w]);
              bv.z = interleave_hi(vb[w], vb[HALF + w]);
              bv.w = interleave_hi(vb[2 * HALF + w], vb[3 * HALF + w]);
            }
            o[s] = mfma_bf16(pj, bv, o[s]);
          }
          lacc = mfma_bf16(pj, ones, lacc);
          // refill both slots of the pair
          constexpr int na = step - 1 + DEPTH, nb = step + DEPTH;
          if constexpr (nb < STEPS) {
            load_step(va, ent_cur, na, rows_left(nt, na));
            load_step(vb, ent_cur, nb, rows_left(nt, nb));
          } else if constexpr (!ONE) {
            load_step(va, ent_nxt, na - STEPS, rows_left(nt_next, na - STEPS));
            load_step(vb, ent_nxt, nb - STEPS, rows_left(nt_next, nb - STEPS));
          }
        }
      }
      // keep each step's loads here: hoisting later steps' loads would hold
      // every block of the chunk in registers at once
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!ONE) {
      ent_cur = ent_nxt;
      ent_nxt = fetch_entries(c + 2 < nchunks ? c + 2 : nchunks - 1);
    }
  }

  // ---- combine the waves through LDS, write ------------------------------------
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (4 * quad + e < R) {
#pragma unroll
      for (int s = 0; s < DPL; ++s) red[wave][4 * quad + e][s * 16 + col] = o[s][e];
      if (col == 0) st_l[wave][4 * quad + e] = lacc[e];
    }
  if (quad == 0 && col < R) st_m[wave][col] = m_run * scale_log2;
  __syncthreads();
  for (int e = threadIdx.x; e < R * D / 4; e += blockDim.x) {
    const int h = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;  // dims d4..d4+3: lane n = d4 / DPL, tiles s0..s0+3
    const int n = d4 / DPL, s0 = d4 % DPL;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w][h]);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = st_m[w][h] == -INFINITY ? 0.f : fast_exp2(st_m[w][h] - M);
      const float* r = &red[w][h][s0 * 16 + n];
      sum.x += wt * r[0]; sum.y += wt * r[16]; sum.z += wt * r[32]; sum.w += wt * r[48];
      lsum += wt * st_l[w][h];
    }
    const float inv = 1.f / lsum;
    const int64_t row = (seq0 + h / G) * Hq + hq0 + h % G;
    if (SPLIT) {
      *reinterpret_cast<float4*>(o_part + (row * num_parts + slot) * D + d4) =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
      if (d4 == 0) lse[row * num_parts + slot] = M + log2f(lsum);
    } else {
      uint2 ov;
      ov.x = pack_bf16x2(sum.x * inv, sum.y * inv);
      ov.y = pack_bf16x2(sum.z * inv, sum.w * inv);
      *reinterpret_cast<uint2*>(out + row * D + d4) = ov;
    }
  }
}

// One wave per (query row, sequence).
template <int D, int MAXP>
__global__ void __launch_bounds__(64)
combine_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
               const float* __restrict__ lse, const int32_t* __restrict__ context_lens, int Hq,
               int num_parts, int part_tokens) {
  const int h = blockIdx.x, b = blockIdx.y;
  combine_row<D, MAXP>(out, o_part, lse, context_lens[b], (int64_t)b * Hq + h, num_parts,
                       part_tokens, threadIdx.x);
}

// Shared-prefix decode: suffix and prefix partials of each row.
template <int D, int MAXP>
__global__ void __launch_bounds__(64)
combine_cascade_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
                       const float* __restrict__ lse, const int32_t* __restrict__ context_lens,
                       const int32_t* __restrict__ starts, int Hq, int num_slots, int part_tokens,
                       int slot0, int prefix_tokens) {
  const int h = blockIdx.x, b = blockIdx.y;
  combine_row<D, MAXP, true>(out, o_part, lse, context_lens[b], (int64_t)b * Hq + h, num_slots,
                             part_tokens, threadIdx.x, starts[b], slot0, prefix_tokens);
}

template <int D>
__global__ void __launch_bounds__(64)
combine_many_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
                    const float* __restrict__ lse, const int32_t* __restrict__ context_lens, int Hq,
                    int num_parts, int part_tokens) {
  const int h = blockIdx.x, b = blockIdx.y;
  combine_row_many<D>(out, o_part, lse, context_lens[b], (int64_t)b * Hq + h, num_parts,
                      part_tokens, threadIdx.x);
}

template <int D, int G, bool FUSED>
hipError_t launch_dg(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                     int B, int Hkv, int max_blocks, int max_context_len, float scale,
                     int partition_size, const StepArgs& st, const int32_t* starts,
                     hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  auto* oo = static_cast<uint16_t*>(out);
  if (partition_size > 0) {
    const int np = (max_context_len + partition_size - 1) / partition_size;
#define PA_ONE(WBB)                                                                           \
  hipLaunchKernelGGL((decode_kernel<D, G, true, true, FUSED, WBB>), dim3(np, Hkv, B), dim3(256), 0, \
                     stream, qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, scale_log2,   \
                     partition_size, np, oo, o_part, lse, st, starts, CascItems{})
    if (partition_size <= kChunkTokens) {
      switch (wave_blocks_for(partition_size)) {
        case 2: PA_ONE(2); break;
        case 4: PA_ONE(4); break;
        default: PA_ONE(8); break;
      }
    } else
      hipLaunchKernelGGL((decode_kernel<D, G, true, false, FUSED>), dim3(np, Hkv, B), dim3(256), 0,
                         stream, qq, kc, vc, block_tables, context_lens, Hkv, max_blocks,
                         scale_log2, partition_size, np, oo, o_part, lse, st, starts, CascItems{});
  } else {
    hipLaunchKernelGGL((decode_kernel<D, G, false, false, FUSED>), dim3(1, Hkv, B), dim3(256), 0,
                       stream, qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, scale_log2,
                       0, 1, oo, o_part, lse, st, nullptr, CascItems{});
  }
#undef PA_ONE
  return hipGetLastError();
}

template <int D, bool FUSED>
hipError_t launch_d(int G, void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* bt, const int32_t* cl, int B, int Hkv,
                    int mb, int mcl, float scale, int ps, const StepArgs& sa, const int32_t* starts,
                    hipStream_t st) {
#define PA_DG(GG) return launch_dg<D, GG, FUSED>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, sa, starts, st)
  switch (G) {
    case 1: PA_DG(1);
    case 2: PA_DG(2);
    case 3: PA_DG(3);
    case 4: PA_DG(4);
    case 5: PA_DG(5);
    case 6: PA_DG(6);
    case 7: PA_DG(7);
    case 8: PA_DG(8);
  }
#undef PA_DG
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                         int max_blocks, int max_context_len, float scale, int partition_size,
                         hipStream_t stream) {
  const int G = Hq / Hkv;
  const StepArgs none{};
  if (D == 128)
    return launch_d<128, false>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens,
                                B, Hkv, max_blocks, max_context_len, scale, partition_size, none,
                                nullptr, stream);
  return launch_d<64, false>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens, B,
                             Hkv, max_blocks, max_context_len, scale, partition_size, none, nullptr,
                             stream);
}

// The decode step with the store folded into the decode kernel: RoPE of q and
// of the new k, the new token's K/V row written at position L-1 of each
// sequence's table, attention over the L tokens; split-K partials are then
// reduced by the combine launch, as for pa_decode.
hipError_t launch_decode_step(void* out, float* o_part, float* lse, const void* q,
                              const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const float* cos_sin, int B, int Hq, int Hkv, int D, int max_blocks,
                              int max_context_len, float scale, int partition_size,
                              bool with_combine, hipStream_t stream) {
  const int G = Hq / Hkv;
  const StepArgs sa{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), cos_sin};
  const hipError_t e =
      D == 128 ? launch_d<128, true>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens,
                                     B, Hkv, max_blocks, max_context_len, scale, partition_size, sa, nullptr, stream)
               : launch_d<64, true>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens,
                                    B, Hkv, max_blocks, max_context_len, scale, partition_size, sa, nullptr, stream);
  if (e != hipSuccess || partition_size <= 0 || !with_combine) return e;
  const int np = (max_context_len + partition_size - 1) / partition_size;
  return launch_decode_combine(out, o_part, lse, context_lens, B, Hkv * G, D, np, partition_size, stream);
}

// Shared-prefix decode in one partition launch (CASC items above).
hipError_t launch_cascade_decode(float* o_part, float* lse, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* group_start,
                                 const int32_t* prefix_lens, int B, int num_groups,
                                 int max_group_size, int max_prefix, int prefix_part,
                                 int max_suffix, int suffix_part, int slot0, int num_slots,
                                 int Hq, int Hkv, int D, int max_blocks, float scale,
                                 hipStream_t stream) {
  const int G = Hq / Hkv;
  if (G < 1 || G > 8 || prefix_part <= 0 || prefix_part > kChunkTokens || suffix_part <= 0 ||
      suffix_part > kChunkTokens)
    return hipErrorInvalidValue;
  const int nseq = 16 / G;
  CascItems ci{};
  ci.group_start = group_start;
  ci.prefix_lens = prefix_lens;
  ci.max_sub = (std::max(max_group_size, 1) + nseq - 1) / nseq;
  ci.pre_parts = std::max((max_prefix + prefix_part - 1) / prefix_part, 1);
  ci.pre_tokens = prefix_part;
  ci.n_pre = (num_groups > 0 && max_prefix > 0) ? num_groups * ci.max_sub * ci.pre_parts : 0;
  ci.suf_parts = std::max((std::max(max_suffix, 1) + suffix_part - 1) / suffix_part, 1);
  ci.suf_tokens = suffix_part;
  ci.slot0 = slot0;
  const int64_t items = (int64_t)ci.n_pre + (int64_t)B * ci.suf_parts;
  if (items <= 0) return hipSuccess;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)items, Hkv, 1);
  const float sl = scale * 1.4426950408889634f;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  const StepArgs none{};
  const int wb = wave_blocks_for(std::max(prefix_part, suffix_part));
#define PA_CASC1(DD, GG, WBB)                                                                       \
  hipLaunchKernelGGL((decode_kernel<DD, GG, true, true, false, WBB, true>), grid, dim3(256), 0, stream, \
                     qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, sl, 0, num_slots,       \
                     nullptr, o_part, lse, none, nullptr, ci)
#define PA_CASC(DD, GG)                      \
  do {                                       \
    if (wb == 2) PA_CASC1(DD, GG, 2);        \
    else if (wb == 4) PA_CASC1(DD, GG, 4);   \
    else PA_CASC1(DD, GG, 8);                \
  } while (0)
#define PA_CASC_G(DD)                  \
  switch (G) {                         \
    case 1: PA_CASC(DD, 1); break;     \
    case 2: PA_CASC(DD, 2); break;     \
    case 3: PA_CASC(DD, 3); break;     \
    case 4: PA_CASC(DD, 4); break;     \
    case 5: PA_CASC(DD, 5); break;     \
    case 6: PA_CASC(DD, 6); break;     \
    case 7: PA_CASC(DD, 7); break;     \
    case 8: PA_CASC(DD, 8); break;     \
    default: return hipErrorInvalidValue; \
  }
  if (D == 128) { PA_CASC_G(128) } else { PA_CASC_G(64) }
#undef PA_CASC_G
#undef PA_CASC
#undef PA_CASC1
  return hipGetLastError();
}

// Split-K partitions of each sequence's suffix [starts[b], L_b).
hipError_t launch_decode_suffix(float* o_part, float* lse, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* starts, int B, int Hq,
                                int Hkv, int D, int max_blocks, int max_context_len, float scale,
                                int partition_size, int num_slots, hipStream_t stream) {
  // the partials' row stride is num_slots, so the kernel's num_parts is num_slots
  const int G = Hq / Hkv;
  const StepArgs none{};
  const float scale_log2 = scale * 1.4426950408889634f;
  const int np = (max_context_len + partition_size - 1) / partition_size;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
#define PA_SUF1(DD, GG, WBB)                                                                        \
  hipLaunchKernelGGL((decode_kernel<DD, GG, true, true, false, WBB>), dim3(np, Hkv, B), dim3(256), 0, \
                     stream, qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, scale_log2,    \
                     partition_size, num_slots, nullptr, o_part, lse, none, starts, CascItems{})
#define PA_SUF(DD, GG)                                                                             \
  do {                                                                                             \
    if (partition_size <= kChunkTokens) {                                                          \
      const int wb = wave_blocks_for(partition_size);                                              \
      if (wb == 2) PA_SUF1(DD, GG, 2);                                                             \
      else if (wb == 4) PA_SUF1(DD, GG, 4);                                                        \
      else PA_SUF1(DD, GG, 8);                                                                     \
    } else                                                                                         \
      hipLaunchKernelGGL((decode_kernel<DD, GG, true, false, false>), dim3(np, Hkv, B), dim3(256), 0, \
                         stream, qq, kc, vc, block_tables, context_lens, Hkv, max_blocks,           \
                         scale_log2, partition_size, num_slots, nullptr, o_part, lse, none, starts, CascItems{}); \
  } while (0)
#define PA_SUF_G(DD)                 \
  switch (G) {                       \
    case 1: PA_SUF(DD, 1); break;    \
    case 2: PA_SUF(DD, 2); break;    \
    case 3: PA_SUF(DD, 3); break;    \
    case 4: PA_SUF(DD, 4); break;    \
    case 5: PA_SUF(DD, 5); break;    \
    case 6: PA_SUF(DD, 6); break;    \
    case 7: PA_SUF(DD, 7); break;    \
    case 8: PA_SUF(DD, 8); break;    \
    default: return hipErrorInvalidValue; \
  }
  if (D == 128) { PA_SUF_G(128) } else { PA_SUF_G(64) }
#undef PA_SUF_G
#undef PA_SUF
#undef PA_SUF1
  return hipGetLastError();
}

hipError_t launch_decode_combine_cascade(void* out, const float* o_part, const float* lse,
                                         const int32_t* context_lens, const int32_t* starts, int B,
                                         int Hq, int D, int num_slots, int partition_size,
                                         int slot0, int prefix_tokens, hipStream_t stream) {
  auto* oo = static_cast<uint16_t*>(out);
  const dim3 grid(Hq, B), block(64);
#define PA_CC(DD, MP)                                                                          \
  hipLaunchKernelGGL((combine_cascade_kernel<DD, MP>), grid, block, 0, stream, oo, o_part, lse,  \
                     context_lens, starts, Hq, num_slots, partition_size, slot0, prefix_tokens)
  if (num_slots > 64) return hipErrorInvalidValue;
  if (D == 128) {
    if (num_slots <= 16) PA_CC(128, 16);
    else if (num_slots <= 32) PA_CC(128, 32);
    else PA_CC(128, 64);
  } else {
    if (num_slots <= 16) PA_CC(64, 16);
    else if (num_slots <= 32) PA_CC(64, 32);
    else PA_CC(64, 64);
  }
#undef PA_CC
  return hipGetLastError();
}

hipError_t launch_decode_combine(void* out, const float* o_part, const float* lse,
                                 const int32_t* context_lens, int B, int Hq, int D,
                                 int num_partitions, int partition_size, hipStream_t stream) {
  auto* oo = static_cast<uint16_t*>(out);
  const dim3 grid(Hq, B), block(64);
#define PA_COMBINE(DD, MP)                                                                    \
  hipLaunchKernelGGL((combine_kernel<DD, MP>), grid, block, 0, stream, oo, o_part, lse,       \
                     context_lens, Hq, num_partitions, partition_size)
  if (D == 128) {
    if (num_partitions <= 16) PA_COMBINE(128, 16);
    else if (num_partitions <= 32) PA_COMBINE(128, 32);
    else if (num_partitions <= 64) PA_COMBINE(128, 64);
    else hipLaunchKernelGGL(combine_many_kernel<128>, grid, block, 0, stream, oo, o_part, lse,
                            context_lens, Hq, num_partitions, partition_size);
  } else {
    if (num_partitions <= 16) PA_COMBINE(64, 16);
    else if (num_partitions <= 32) PA_COMBINE(64, 32);
    else if (num_partitions <= 64) PA_COMBINE(64, 64);
    else hipLaunchKernelGGL(combine_many_kernel<64>, grid, block, 0, stream, oo, o_part, lse,
                            context_lens, Hq, num_partitions, partition_size);
  }
#undef PA_COMBINE
  return hipGetLastError();
}

}  // namespace pa
