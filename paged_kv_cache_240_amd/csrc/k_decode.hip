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
// the whole sequence (single pass) are walked in chunks of 32 blocks, wave w
// taking blocks w, w+4, ..., w+28 of each chunk.  Both products run on
// v_mfma_f32_16x16x32_bf16 with the G query heads padded to 16:
//   QK   S^T = K Q^T per block: the key tile is the A operand as it lies in
//        memory (lane = key, 16 contiguous bytes of its row per k-step), the
//        query rows the B operand.  A lane ends up with 4 consecutive keys of
//        one head; rows past the range become -inf by a select.
//   P    after the 8 blocks of a chunk, the running max per head (in-lane max,
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
// order K0..K7, V0..V7, K0' ... so loads run DEPTH blocks ahead of the
// arithmetic across phase and chunk boundaries.  Loads past the last block of
// the range re-read the last valid block (an L2 hit) instead of branching.
// The waves never synchronise until the end, where their (max, sum, output)
// triples are combined through LDS.  The output is the normalised bf16 row
// (single pass) or an fp32 partial plus its base-2 log-sum-exp (split-K),
// reduced by combine_kernel (Flash Decode's reduce).

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_DEPTH_ONE
#define PA_DECODE_DEPTH_ONE 8
#endif

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kWaveBlocks = 8;                           // blocks per wave per chunk
constexpr int kChunkBlocks = kWaves * kWaveBlocks;       // 32
constexpr int kChunkTokens = kChunkBlocks * kBlockSize;  // 512
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

// ONE: the range is a single chunk (split-K with partitions of at most 512
// tokens), so the ring need not cycle and can be deeper; no refills past it.
template <int D, int G, bool SPLIT, bool ONE>
__global__ void __launch_bounds__(256, 2)  // 2 waves per SIMD: 8 streaming waves per CU
decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
              const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
              const int32_t* __restrict__ context_lens, int Hkv, int max_blocks,
              float scale_log2, int part_tokens, int num_parts, uint16_t* __restrict__ out,
              float* __restrict__ o_part, float* __restrict__ lse) {
  static_assert(G >= 1 && G <= 8, "query heads per KV head: 1..8");
  constexpr int KS = D / 32;    // QK k-steps over the head dimension
  constexpr int DPL = D / 16;   // PV: dims per lane = output tiles of 16 columns
  constexpr int HALF = DPL / 2; // dwords of one V row piece
  constexpr int SLOT = 4 * KS;  // dwords per lane of a K block (16 bytes per k-step)
  static_assert(SLOT == 4 * HALF, "K and V blocks must occupy the same ring slot");
  constexpr int STEPS = 2 * kWaveBlocks;  // K0..K7 then V0..V7
  constexpr int DEPTH = ONE ? kDepthOne : kDepth;
  static_assert(DEPTH % 2 == 0 && (ONE || STEPS % DEPTH == 0), "ring slots must repeat per chunk");

  __shared__ __align__(16) float red[kWaves][G][D];  // per-wave outputs, dim n*DPL+s at s*16+n
  __shared__ float st_m[kWaves][G], st_l[kWaves][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar table reads
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int hq0 = g * G;
  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int L = context_lens[b];
  // The first chunk's table entries are requested before L is known (indices
  // clamped into the table; an entry past the sequence is never dereferenced:
  // it is replaced by the range's first block once L arrives), so the first
  // K/V loads wait for one round trip instead of two.
  const int lb0 = SPLIT ? p * part_tokens / kBlockSize : 0;
  const int lb_spec = lb0 + wave + kWaves * (threadIdx.x & 7);
  const int ent_spec = bt_row[min(lb_spec, max_blocks - 1)];
  const int ent_first = bt_row[lb0];
  const int col = lane & 15, quad = lane >> 4;  // MFMA lane roles
  // B operand of QK: query row of head `col` (zero beyond G), 8 dims per
  // k-step; padding lanes read head 0 and discard it (a select, not a branch)
  uint4 qraw[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qraw[ks] = *reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + hq0 + min(col, G - 1)) * D +
                                               ks * 32 + quad * 8);
  // every start-up load is in flight before the emptiness test below
  asm volatile("" ::"v"(ent_spec), "s"(ent_first), "s"(L));

  int t_begin = 0, t_end = L;
  if (SPLIT) {
    t_begin = p * part_tokens;
    if (t_begin >= L) return;  // empty partition: not written, not combined
    t_end = min(t_begin + part_tokens, L);
  } else if (L <= 0) {
    for (int e = threadIdx.x; e < G * D / 2; e += blockDim.x)
      reinterpret_cast<uint32_t*>(out + ((int64_t)b * Hq + hq0) * D)[e] = 0u;
    return;
  }

  uint4 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = col < G ? qraw[ks] : make_uint4(0u, 0u, 0u, 0u);

  floatx4_t o[DPL];  // O[head 4*quad+e][dim col*DPL+s] in o[s][e]
  floatx4_t lacc = {0.f, 0.f, 0.f, 0.f};  // l of head 4*quad+e (every column the same)
#pragma unroll
  for (int s = 0; s < DPL; ++s) o[s] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // raw-score max of head `col` (same in the 4 lanes of a head)

  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;
  const int nchunks = ONE ? 1 : (t_end - t_begin + kChunkTokens - 1) / kChunkTokens;
  const int last_lb = (t_end - 1) / kBlockSize;  // last logical block of the range
  const int lane_k = col * D + quad * 8;         // element offsets inside a block tile
  const int lane_v = col * DPL;
  const uint4 ones = make_uint4(kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2);

  // Block-table entries of this wave's 8 blocks of chunk c: one vector load,
  // lane j (mod 8) fetching the entry of block j; blocks past the range take
  // the last valid entry.  Fetched a chunk ahead and read with readlane, so a
  // ring refill never waits on the table.
  auto fetch_entries = [&](int c) -> int {
    const int lb = (t_begin + c * kChunkTokens) / kBlockSize + wave + kWaves * (lane & 7);
    return bt_row[min(lb, last_lb)];
  };
  // Ring step `step` (0..7 K blocks, 8..15 V blocks) of the chunk whose
  // entries are `ent`; `left` = rows of that block inside the range.
  auto load_step = [&](uint32_t (&slot)[SLOT], int ent, int step, int left) {
    const int i = step & (kWaveBlocks - 1);
    const int64_t base = (int64_t)__builtin_amdgcn_readlane(ent, i) * blk_stride + head_off;
    if (step < kWaveBlocks) {
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
  auto rows_left = [&](int nt, int step) { return nt - (wave + kWaves * (step & 7)) * kBlockSize; };

  int ent_cur = lb_spec <= last_lb ? ent_spec : ent_first;  // == fetch_entries(0)
  int ent_nxt = ONE ? 0 : fetch_entries(nchunks > 1 ? 1 : 0);
  const int nt0 = min(kChunkTokens, t_end - t_begin);
  uint32_t ring[DEPTH][SLOT];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) load_step(ring[s], ent_cur, s, rows_left(nt0, s));

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = t_begin + c * kChunkTokens;
    const int nt = min(kChunkTokens, t_end - c0);  // valid tokens of the chunk
    const int nt_next = min(kChunkTokens, t_end - c0 - kChunkTokens);
    floatx4_t st[kWaveBlocks];  // raw scores: keys 4*quad+e of block i, head col
    uint4 pa[kWaveBlocks / 2];  // bf16 probabilities: A operand of block pair j

    static_for<STEPS>([&](auto step_c) {
      constexpr int step = decltype(step_c)::value;
      uint32_t(&cur)[SLOT] = ring[step % DEPTH];
      constexpr int i = step & (kWaveBlocks - 1);

      if constexpr (step < kWaveBlocks) {
        // ---- QK on block i: S^T (16 keys x 16 heads) ---------------------------
        const int left = rows_left(nt, step);
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
        if constexpr (step == kWaveBlocks) {
          // ---- P: online softmax over this wave's 8 blocks -------------------------
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < kWaveBlocks; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[j][e]);
          mx = fmaxf(mx, swap16(mx));
          mx = fmaxf(mx, swap32(mx));
          const float m_new = fmaxf(m_run, mx);
          // no key of this head in range yet: m stays -inf and every p is 0
          const float ref = m_new == -INFINITY ? 0.f : m_new * scale_log2;
          const float alpha = fast_exp2(m_run * scale_log2 - ref);
          m_run = m_new;
#pragma unroll
          for (int j = 0; j < kWaveBlocks / 2; ++j) {
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
    if (4 * quad + e < G) {
#pragma unroll
      for (int s = 0; s < DPL; ++s) red[wave][4 * quad + e][s * 16 + col] = o[s][e];
      if (col == 0) st_l[wave][4 * quad + e] = lacc[e];
    }
  if (quad == 0 && col < G) st_m[wave][col] = m_run * scale_log2;
  __syncthreads();
  for (int e = threadIdx.x; e < G * D / 4; e += blockDim.x) {
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
    const int64_t row = (int64_t)b * Hq + hq0 + h;
    if (SPLIT) {
      *reinterpret_cast<float4*>(o_part + (row * num_parts + p) * D + d4) =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
      if (d4 == 0) lse[row * num_parts + p] = M + log2f(lsum);
    } else {
      uint2 ov;
      ov.x = pack_bf16x2(sum.x * inv, sum.y * inv);
      ov.y = pack_bf16x2(sum.z * inv, sum.w * inv);
      *reinterpret_cast<uint2*>(out + row * D + d4) = ov;
    }
  }
}

// Log-sum-exp combine of split-K partials (Flash Decode's reduce): one wave
// per (query row, sequence), a row being a query head (or, for multi-query
// decode, a (query, head) pair).  Every load is issued before L is known: lane
// j < num_parts reads lse[j] and each lane reads one 16-byte piece of every
// partial it may need (indices clamped into the workspace); partitions past
// ceil(L / P) were never written and are removed by selects, not arithmetic,
// so stale workspace contents (NaN included) cannot leak.  Then: M = max lse,
// out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M).
template <int D, int MAXP>
__global__ void __launch_bounds__(64)
combine_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
               const float* __restrict__ lse, const int32_t* __restrict__ context_lens, int Hq,
               int num_parts, int part_tokens) {
  constexpr int PIECES = D / 4;     // float4 pieces of one partial row
  constexpr int PPI = 64 / PIECES;  // partials covered by one wave-wide step
  constexpr int NSTEP = MAXP / PPI;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int piece = lane % PIECES, sub = lane / PIECES;
  const int64_t row = (int64_t)b * Hq + h;
  const float* ls = lse + row * num_parts;
  const float* src = o_part + row * num_parts * D + piece * 4;
  const int L = context_lens[b];
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
  const int n = (L + part_tokens - 1) / part_tokens;
  const float M = wave_max(lane < n ? my_lse : -INFINITY);
  if (M == -INFINITY) {  // no partition saw a key of this row (multi-query rows before the cache)
    if (sub == 0) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const float W = wave_sum(lane < n ? exp2f(my_lse - M) : 0.f);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < NSTEP; ++k) {
    const bool in = sub + PPI * k < n;
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

// Fallback for more than 64 partitions: loops over the partitions.
template <int D>
__global__ void __launch_bounds__(64)
combine_many_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
                    const float* __restrict__ lse, const int32_t* __restrict__ context_lens, int Hq,
                    int num_parts, int part_tokens) {
  constexpr int PIECES = D / 4;
  constexpr int PPI = 64 / PIECES;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int piece = lane % PIECES, sub = lane / PIECES;
  const int64_t row = (int64_t)b * Hq + h;
  const int L = context_lens[b];
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

template <int D, int G>
hipError_t launch_dg(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                     int B, int Hkv, int max_blocks, int max_context_len, float scale,
                     int partition_size, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  auto* oo = static_cast<uint16_t*>(out);
  if (partition_size > 0) {
    const int np = (max_context_len + partition_size - 1) / partition_size;
    if (partition_size <= kChunkTokens)
      hipLaunchKernelGGL((decode_kernel<D, G, true, true>), dim3(np, Hkv, B), dim3(256), 0, stream,
                         qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, scale_log2,
                         partition_size, np, oo, o_part, lse);
    else
      hipLaunchKernelGGL((decode_kernel<D, G, true, false>), dim3(np, Hkv, B), dim3(256), 0, stream,
                         qq, kc, vc, block_tables, context_lens, Hkv, max_blocks, scale_log2,
                         partition_size, np, oo, o_part, lse);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, G, false, false>), dim3(1, Hkv, B), dim3(256), 0, stream, qq, kc,
                       vc, block_tables, context_lens, Hkv, max_blocks, scale_log2, 0, 1, oo,
                       o_part, lse);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int G, void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* bt, const int32_t* cl, int B, int Hkv,
                    int mb, int mcl, float scale, int ps, hipStream_t st) {
  switch (G) {
    case 1: return launch_dg<D, 1>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 2: return launch_dg<D, 2>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 3: return launch_dg<D, 3>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 4: return launch_dg<D, 4>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 5: return launch_dg<D, 5>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 6: return launch_dg<D, 6>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 7: return launch_dg<D, 7>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
    case 8: return launch_dg<D, 8>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, Hkv, mb, mcl, scale, ps, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                         int max_blocks, int max_context_len, float scale, int partition_size,
                         hipStream_t stream) {
  const int G = Hq / Hkv;
  if (D == 128)
    return launch_d<128>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens, B,
                         Hkv, max_blocks, max_context_len, scale, partition_size, stream);
  return launch_d<64>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens, B, Hkv,
                      max_blocks, max_context_len, scale, partition_size, stream);
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
    else if (num_partitions <= 64) PA_COMBINE(128, 64);
    else hipLaunchKernelGGL(combine_many_kernel<128>, grid, block, 0, stream, oo, o_part, lse,
                            context_lens, Hq, num_partitions, partition_size);
  } else {
    if (num_partitions <= 16) PA_COMBINE(64, 16);
    else if (num_partitions <= 64) PA_COMBINE(64, 64);
    else hipLaunchKernelGGL(combine_many_kernel<64>, grid, block, 0, stream, oo, o_part, lse,
                            context_lens, Hq, num_partitions, partition_size);
  }
#undef PA_COMBINE
  return hipGetLastError();
}

}  // namespace pa
