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
// taking blocks w, w+4, ..., w+28 of each chunk.  Per chunk each wave:
//   QK   S^T = K Q^T for the 16 keys of a block and the G query heads (padded
//        to 16) with v_mfma_f32_16x16x32_bf16: the key tile is the A operand
//        as it lies in memory (lane = key, 16 contiguous bytes of its row per
//        k-step), the query rows the B operand (16 registers whatever G).
//        Each lane then holds 4 consecutive keys of one head; scaled by
//        scale*log2 e (rows past the range set to -inf by a select), they go
//        to the wave's LDS slice with one 16-byte store.
//   P    the wave's running max/sum per head (online softmax across chunks,
//        wave shuffles); p = 2^(s - m) is rounded to bf16 and stored as
//        (even row, odd row) pairs in the order the PV step reads them.
//   PV   lane (row group, 4 dims) takes 8-byte pieces of 16/TG rows of a V
//        block (rows 2m and 2m+1 for its pairs m); v_perm interleaves the two
//        rows per dim so v_dot2_f32_bf16 applies both probabilities at once,
//        with fp32 accumulation.  Rows past the range are zeroed by a select,
//        so NaN in unused slots never reaches a sum.
// K and V blocks stream through a ring of DEPTH register buffers in the
// order K0..K7, V0..V7, K0' ... so loads run DEPTH blocks ahead of the
// arithmetic across phase and chunk boundaries.  Loads past the last block of
// the range re-read the last valid block (an L2 hit) instead of branching.
// The waves never synchronise until the end, where their (max, sum, output)
// triples are combined through LDS.  The output is the normalised bf16 row
// (single pass) or an fp32 partial plus its base-2 log-sum-exp (split-K),
// reduced by combine_kernel (Flash Decode's reduce).
//
// Block-table entries are read with wave-uniform addresses (scalar loads);
// entries past the sequence's last block are never read.

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
constexpr int kWaveTokens = kWaveBlocks * kBlockSize;    // 128
constexpr int kDepth = 4;     // blocks in flight per wave when chunks repeat (ring slots must cycle per chunk)
constexpr int kDepthOne = PA_DECODE_DEPTH_ONE;  // ... when the range is a single chunk

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// ONE: the range is a single chunk (split-K with partitions of at most 512
// tokens), so the ring need not cycle and can be deeper; no refills past it.
template <int D, int G, bool SPLIT, bool ONE>
__global__ void __launch_bounds__(256, 2)  // 2 waves per SIMD: 8 streaming waves per CU
decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
              const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
              const int32_t* __restrict__ context_lens, int Hkv, int max_blocks,
              float scale_log2, int part_tokens, int num_parts, uint16_t* __restrict__ out,
              float* __restrict__ o_part, float* __restrict__ lse) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head must fit the 16 MFMA columns");
  constexpr int KS = D / 32;          // MFMA k-steps over the head dimension
  constexpr int VL = D / 4;           // lanes per row in the PV layout (4 dims each)
  constexpr int TG = 64 / VL;         // row groups in the PV layout
  constexpr int NPAIR = 8 / TG;       // row pairs per lane per block
  constexpr int SLOT = 4 * KS;        // dwords per lane of a K block (16 bytes per k-step)
  static_assert(SLOT == 4 * NPAIR, "K and V blocks must occupy the same ring slot");
  constexpr int STEPS = 2 * kWaveBlocks;  // K0..K7 then V0..V7
  constexpr int DEPTH = ONE ? kDepthOne : kDepth;
  static_assert(ONE || STEPS % DEPTH == 0, "ring slots must repeat per chunk");
  constexpr int S_WAVE = G * kWaveTokens;  // floats of one wave's score slice
  static_assert(kWaves * S_WAVE >= G * D, "reduction buffer fits in the score slices");

  // Wave slice, head h, block i: 16 floats of scores in key order; after the P
  // step its first 8 dwords hold bf16 probability pairs, pair m at
  // (m % TG) * NPAIR + m / TG (the order a PV lane reads its NPAIR pairs).
  __shared__ __align__(16) float s_buf[kWaves * S_WAVE];
  __shared__ __align__(16) float s_junk[kWaves][64];  // stores of lanes whose head is >= G
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
  const int col = threadIdx.x & 15, quad = (threadIdx.x >> 4) & 3;  // MFMA lane roles
  // B operand: query row of head `col` (zero beyond G), 8 dims per k-step;
  // padding lanes read head 0 and discard it (a select, not a branch)
  uint4 qraw[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
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

  const int tg = lane / VL, dq = lane % VL;  // PV layout: row group, 4-dim piece
  bf16x8_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qb[ks] = __builtin_bit_cast(bf16x8_t, col < G ? qraw[ks] : make_uint4(0u, 0u, 0u, 0u));

  float acc[G][4];
  float m_run[G], l_run[G];  // wave-uniform
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
  }

  float* sw = s_buf + wave * S_WAVE;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;
  const int nchunks = ONE ? 1 : (t_end - t_begin + kChunkTokens - 1) / kChunkTokens;
  const int last_lb = (t_end - 1) / kBlockSize;  // last logical block of the range
  const int lane_k = col * D + quad * 8;         // element offsets inside a block tile
  const int lane_v = 2 * tg * D + dq * 4;

  // Block-table entries of this wave's 8 blocks of chunk c: one vector load,
  // lane j (mod 8) fetching the entry of block j; blocks past the range take
  // the last valid entry.  Fetched a chunk ahead and read with readlane, so a
  // ring refill never waits on the table.
  auto fetch_entries = [&](int c) -> int {
    const int lb = (t_begin + c * kChunkTokens) / kBlockSize + wave + kWaves * (lane & 7);
    return bt_row[min(lb, last_lb)];
  };
  // Ring step `step` (0..7 K blocks, 8..15 V blocks) of the chunk whose entries are `ent`.
  auto load_step = [&](uint32_t (&slot)[SLOT], int ent, int step) {
    const int i = step & (kWaveBlocks - 1);
    const int64_t base = (int64_t)__builtin_amdgcn_readlane(ent, i) * blk_stride + head_off;
    if (step < kWaveBlocks) {
      const uint16_t* src = k_cache + base + lane_k;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 t = *reinterpret_cast<const uint4*>(src + ks * 32);
        slot[4 * ks] = t.x; slot[4 * ks + 1] = t.y; slot[4 * ks + 2] = t.z; slot[4 * ks + 3] = t.w;
      }
    } else {
      // pair k covers rows 2m, 2m+1 with m = tg + TG*k
      const uint16_t* src = v_cache + base + lane_v;
#pragma unroll
      for (int k = 0; k < NPAIR; ++k)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint2 t = *reinterpret_cast<const uint2*>(src + (2 * TG * k + e) * D);
          slot[4 * k + 2 * e] = t.x; slot[4 * k + 2 * e + 1] = t.y;
        }
    }
  };

  int ent_cur = lb_spec <= last_lb ? ent_spec : ent_first;  // == fetch_entries(0)
  int ent_nxt = ONE ? 0 : fetch_entries(nchunks > 1 ? 1 : 0);
  uint32_t ring[DEPTH][SLOT];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) load_step(ring[s], ent_cur, s);

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = t_begin + c * kChunkTokens;
    const int nt = min(kChunkTokens, t_end - c0);  // valid tokens of the chunk
    // LDS bases rebuilt per chunk from an opaque zero, so constant per-step
    // offsets fold into the instructions instead of each taking a register
    const int z = opaque_zero();
    // QK: head col, keys 4*quad..+3; lanes of padding heads write the junk row
    // (a select, not a branch: divergent branches would split the step into
    // blocks across which the compiler sinks the arithmetic, stretching the
    // ring's live ranges)
    float* s_wr = col < G ? sw + z + col * kWaveTokens + quad * 4
                          : &s_junk[wave][0] + z + quad * 4;
    float* sw_c = sw + z;
    const uint32_t* p_rd = reinterpret_cast<const uint32_t*>(sw + z) + tg * NPAIR;

    static_for<STEPS>([&](auto step_c) {
      constexpr int step = decltype(step_c)::value;
      uint32_t(&cur)[SLOT] = ring[step % DEPTH];
      constexpr int i = step & (kWaveBlocks - 1);
      const int left = nt - (wave + kWaves * i) * kBlockSize;  // uniform: rows of block i in range

      if constexpr (step < kWaveBlocks) {
        // ---- QK on block i: S^T (16 keys x 16 heads) ---------------------------
        floatx4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 t = make_uint4(cur[4 * ks], cur[4 * ks + 1], cur[4 * ks + 2], cur[4 * ks + 3]);
          st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t), qb[ks], st,
                                                       0, 0, 0);
        }
        float4 sv;
        sv.x = quad * 4 + 0 < left ? st[0] * scale_log2 : -INFINITY;
        sv.y = quad * 4 + 1 < left ? st[1] * scale_log2 : -INFINITY;
        sv.z = quad * 4 + 2 < left ? st[2] * scale_log2 : -INFINITY;
        sv.w = quad * 4 + 3 < left ? st[3] * scale_log2 : -INFINITY;
        *reinterpret_cast<float4*>(s_wr + (col < G ? i * kBlockSize : 0)) = sv;
      } else {
        if constexpr (step == kWaveBlocks) {
          // ---- P: online softmax over this wave's 128 rows --------------------------
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          // lane holds keys 2*lane, 2*lane+1 of the slice: block lane/8, pair lane%8
          float2 sv[G];
#pragma unroll
          for (int h = 0; h < G; ++h)
            sv[h] = reinterpret_cast<const float2*>(sw_c + h * kWaveTokens)[lane];
          const int pm = lane & 7;
          const int p_idx = (lane >> 3) * kBlockSize + (pm % TG) * NPAIR + pm / TG;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float m_new = uniform(fmaxf(m_run[h], wave_max(fmaxf(sv[h].x, sv[h].y))));
            // a wave whose rows are all past the end keeps m = -inf; p = 0 then
            const float ref = m_new == -INFINITY ? 0.f : m_new;
            const uint32_t pk = pack_bf16x2(exp2f(sv[h].x - ref), exp2f(sv[h].y - ref));
            // the normaliser sums the rounded probabilities the PV step applies
            const float psum = bf16lo(pk) + bf16hi(pk);
            reinterpret_cast<uint32_t*>(sw_c + h * kWaveTokens)[p_idx] = pk;
            const float alpha = exp2f(m_run[h] - ref);
            l_run[h] = uniform(l_run[h] * alpha + wave_sum(psum));
            m_run[h] = m_new;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h][e] *= alpha;
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // ---- PV on block i ------------------------------------------------------
        uint32_t(&vv)[SLOT] = cur;  // consumed in place; refilled after this step
#pragma unroll
        for (int k = 0; k < NPAIR; ++k)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const bool in = 2 * (tg + TG * k) + e < left;  // selects, no branch
            vv[4 * k + 2 * e] = in ? vv[4 * k + 2 * e] : 0u;
            vv[4 * k + 2 * e + 1] = in ? vv[4 * k + 2 * e + 1] : 0u;
          }
        uint32_t pp[G][NPAIR];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t* src = p_rd + h * kWaveTokens + i * kBlockSize;
          if constexpr (NPAIR == 4) {
            const uint4 t = *reinterpret_cast<const uint4*>(src);
            pp[h][0] = t.x; pp[h][1] = t.y; pp[h][2] = t.z; pp[h][3] = t.w;
          } else {
            const uint2 t = *reinterpret_cast<const uint2*>(src);
            pp[h][0] = t.x; pp[h][1] = t.y;
          }
        }
#pragma unroll
        for (int k = 0; k < NPAIR; ++k) {
          const uint32_t a0 = vv[4 * k], a1 = vv[4 * k + 1];      // row 2m: dims 0-1, 2-3
          const uint32_t b0 = vv[4 * k + 2], b1 = vv[4 * k + 3];  // row 2m+1
          const uint32_t d0 = interleave_lo(a0, b0), d1 = interleave_hi(a0, b0);
          const uint32_t d2 = interleave_lo(a1, b1), d3 = interleave_hi(a1, b1);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][0] = dot2_bf16(pp[h][k], d0, acc[h][0]);
            acc[h][1] = dot2_bf16(pp[h][k], d1, acc[h][1]);
            acc[h][2] = dot2_bf16(pp[h][k], d2, acc[h][2]);
            acc[h][3] = dot2_bf16(pp[h][k], d3, acc[h][3]);
          }
        }
        if constexpr (step == STEPS - 1) {
          // this chunk's probabilities consumed before the next chunk's QK overwrites them
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
      // refill the slot just consumed: DEPTH steps ahead (into the next chunk near the end)
      constexpr int ns = step + DEPTH;
      if constexpr (ns < STEPS)
        load_step(cur, ent_cur, ns);
      else if constexpr (!ONE)
        load_step(cur, ent_nxt, ns - STEPS);  // last chunk: ent_nxt re-reads its own blocks
      // keep the refill here: hoisting later steps' loads would hold every
      // block of the chunk in registers at once
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!ONE) {
      ent_cur = ent_nxt;
      ent_nxt = fetch_entries(c + 2 < nchunks ? c + 2 : nchunks - 1);
    }
  }

  // ---- combine row groups (lanes) and waves, write ----------------------------
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = acc[h][e];
#pragma unroll
      for (int off = VL; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[h][e] = x;
    }
  __syncthreads();  // every wave is done with its score slice
  float* red = s_buf;  // [kWaves][G][D]
  if (lane < VL) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      *reinterpret_cast<float4*>(red + (wave * G + h) * D + dq * 4) =
          make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      st_m[wave][h] = m_run[h];
      st_l[wave][h] = l_run[h];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D / 4; e += blockDim.x) {
    const int h = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w][h]);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = st_m[w][h] == -INFINITY ? 0.f : exp2f(st_m[w][h] - M);
      const float4 t = *reinterpret_cast<const float4*>(red + (w * G + h) * D + d4);
      sum.x += wt * t.x; sum.y += wt * t.y; sum.z += wt * t.z; sum.w += wt * t.w;
      lsum += wt * st_l[w][h];
    }
    const float inv = 1.f / lsum;
    const int64_t row = (int64_t)b * Hq + hq0 + h;
    if (SPLIT) {
      *reinterpret_cast<float4*>(o_part + (row * num_parts + p) * D + d4) =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
      if (d4 == 0) lse[row * num_parts + p] = M + log2f(lsum);
    } else {
      uint2 o;
      o.x = pack_bf16x2(sum.x * inv, sum.y * inv);
      o.y = pack_bf16x2(sum.z * inv, sum.w * inv);
      *reinterpret_cast<uint2*>(out + row * D + d4) = o;
    }
  }
}

// Log-sum-exp combine of split-K partials (Flash Decode's reduce): one wave
// per (query head, sequence).  Every load is issued before L is known: lane
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
