// Multi-query paged decode for gfx950: speculative-decoding verification.
//
// Operation (mini-llm-engine post, §3.6: the target model checks the K draft
// tokens in one pass, equivalent to one prefill; §3.1: K/V in 16-token
// physical blocks behind a block table; Pico-vLLM write-up, §1: GQA): each
// sequence b brings NQ consecutive queries (the last accepted token and the
// drafts), already stored in the cache, so query i sits at position
// L_b - NQ + i and attends keys t <= L_b - NQ + i:
//   out[b,i,h] = softmax(scale * q[b,i,h] K_b^T) V_b   (causal over the NQ rows).
//
// It is the decode kernel's layout with NQ * G (query, head) rows instead of G
// heads: one workgroup per (sequence, KV head, partition) reads every K/V byte
// once for all its rows.  Rows r = i * G + h fill up to two 16-row MFMA tiles
// (CT).  A workgroup of NW waves walks its range in chunks of 8 * NW blocks,
// wave w taking blocks w, w+NW, ..., w+7NW, as block pairs in the order
// K(2j), K(2j+1), V(2j), V(2j+1) through a 4-slot register ring (loads run one
// pair ahead).  Partitions of up to 512 tokens are one chunk of 4 waves; those
// of up to 1024 one chunk of 8 waves (two waves per SIMD at two row tiles,
// one workgroup per CU); longer ranges repeat 4-wave chunks.  Single-chunk
// partitions with two row tiles run decode_multi_lds_kernel below instead:
// the same steps with V blocks copied straight into LDS, which leaves the
// register ring to K and keeps two block pairs per wave in flight.  Per pair
// and row tile:
//   QK   S^T = K Q^T (v_mfma_f32_16x16x32_bf16, K straight from memory as the
//        A operand, the tile's query rows as the B operand); keys past the
//        row's causal limit or the range become -inf by a select.
//   P    the pair's max per row (4 lanes per row: two cross-row swaps); the
//        row's reference max is raised only when the pair exceeds it by more
//        than 2^8 (then the accumulators are rescaled), so p = 2^((s - m) *
//        scale * log2 e) stays below 256; rounded to bf16 in place, the 8 p of
//        a lane are its A operand of PV.
//   PV   O = P V: V rows paired per dim with v_perm into B operands shared by
//        the row tiles; a product against a ones operand accumulates l from
//        the same rounded p.  V rows past the range are redirected to row 0 of
//        their block at load time (finite data under p = 0).
// The waves meet once, at the end, through LDS.  Split-K partials are the
// normalised fp32 rows plus base-2 log-sum-exps, reduced by the decode
// combine kernel over NQ * Hq rows per sequence; a row without a visible key in
// a partition writes zeros and lse = -inf.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaveBlocks = 8;                           // blocks per wave per chunk
constexpr int kChunkTokens = 4 * kWaveBlocks * kBlockSize;  // 512: a chunk of 4 waves
constexpr int kDepth = 4;                                // ring slots: one block pair of K and V
constexpr float kLazyLog2 = 8.f;                         // reference max may lag by 2^8
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma_bf16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

typedef short shortx4_t __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// Ring step s of a chunk (0..15): block pair s / 4; s % 4 = K(2j), K(2j+1), V(2j), V(2j+1).
__host__ __device__ constexpr int step_block(int s) { return 2 * (s / 4) + (s % 2); }
__host__ __device__ constexpr bool step_is_v(int s) { return (s % 4) >= 2; }

// ONE: the range is a single chunk (partitions of at most 64 * NW tokens): no
// refills past it.  NW: waves per workgroup (4, or 8 for single-chunk
// partitions of up to 1024 tokens, one workgroup per CU).
// Two row tiles with a ring that cycles over chunks need more than the 256
// registers of two waves per SIMD: that variant runs one wave per SIMD.
template <int D, int G, int CT, bool SPLIT, bool ONE, int NW>
__global__ void __launch_bounds__(64 * NW, (CT == 2 && !ONE) || NW == 8 ? 1 : 2)
decode_multi_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ context_lens, int NQ, int Hkv, int max_blocks,
                    float scale_log2, int part_tokens, int num_parts, uint16_t* __restrict__ out,
                    float* __restrict__ o_part, float* __restrict__ lse) {
  static_assert(CT == 1 || CT == 2, "one or two 16-row tiles");
  constexpr int kWaves = NW;
  constexpr int kChunk = NW * kWaveBlocks * kBlockSize;  // tokens of one chunk
  constexpr int KS = D / 32;    // QK k-steps over the head dimension
  constexpr int DPL = D / 16;   // PV: dims per lane = output tiles of 16 columns
  constexpr int HALF = DPL / 2; // dwords of one V row piece
  constexpr int SLOT = 4 * KS;  // dwords per lane of a K block
  static_assert(SLOT == 4 * HALF, "K and V blocks must occupy the same ring slot");
  constexpr int STEPS = 2 * kWaveBlocks;
  constexpr int ROWS = 16 * CT;

  __shared__ __align__(16) float red[kWaves][ROWS][D];  // per-wave outputs, dim n*DPL+s at s*16+n
  __shared__ float st_m[kWaves][ROWS], st_l[kWaves][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int hq0 = g * G;
  const int R = NQ * G;  // valid rows
  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int L = context_lens[b];
  // first chunk's table entries requested before L is known (clamped; an entry
  // past the sequence is replaced by the range's first block once L arrives)
  const int lb0 = SPLIT ? p * part_tokens / kBlockSize : 0;
  const int lb_spec = lb0 + wave + kWaves * (threadIdx.x & 7);
  const int ent_spec = bt_row[min(lb_spec, max_blocks - 1)];
  const int ent_first = bt_row[lb0];
  const int col = lane & 15, quad = lane >> 4;

  // this lane's rows (one per tile, the S^T column): query row and causal limit
  uint4 qraw[CT][KS];
  int qrow_i[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = min(ct * 16 + col, R - 1);  // padding lanes read a valid row, then zero it
    qrow_i[ct] = r / G;
    const uint16_t* qrow = q + (((int64_t)b * NQ + r / G) * Hq + hq0 + r % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ct][ks] = *reinterpret_cast<const uint4*>(qrow + ks * 32 + quad * 8);
  }
  asm volatile("" ::"v"(ent_spec), "s"(ent_first), "s"(L));

  int t_begin = 0, t_end = L;
  if (SPLIT) {
    t_begin = p * part_tokens;
    if (t_begin >= L) return;  // empty partition: not written, not combined
    t_end = min(t_begin + part_tokens, L);
  } else if (L <= 0) {
    for (int e = threadIdx.x; e < R * D / 2; e += blockDim.x) {
      const int r = e / (D / 2);
      reinterpret_cast<uint32_t*>(out + (((int64_t)b * NQ + r / G) * Hq + hq0 + r % G) * D)[e % (D / 2)] = 0u;
    }
    return;
  }

  uint4 qb[CT][KS];
  int lim[CT];  // exclusive bound on the keys a row sees inside the range
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const bool valid = ct * 16 + col < R;
    lim[ct] = valid ? min(t_end, L - NQ + qrow_i[ct] + 1) : t_begin;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = valid ? qraw[ct][ks] : make_uint4(0u, 0u, 0u, 0u);
  }

  floatx4_t o[CT][DPL];  // O[row 16ct + 4quad + e][dim col*DPL + s] in o[ct][s][e]
  floatx4_t lacc[CT];
  float m_ref[CT];  // reference max of the lane's row (raw scores; -inf: none seen)
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    lacc[ct] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_ref[ct] = -INFINITY;
#pragma unroll
    for (int s = 0; s < DPL; ++s) o[ct][s] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float lazy_raw = kLazyLog2 / scale_log2;

  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;
  const int nchunks = ONE ? 1 : (t_end - t_begin + kChunk - 1) / kChunk;
  const int last_lb = (t_end - 1) / kBlockSize;
  const int lane_k = col * D + quad * 8;
  const int lane_v = col * DPL;
  const uint4 ones = make_uint4(kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2);

  auto fetch_entries = [&](int c) -> int {
    const int lb = (t_begin + c * kChunk) / kBlockSize + wave + kWaves * (lane & 7);
    return bt_row[min(lb, last_lb)];
  };
  // ring step `step` of the chunk whose entries are `ent`; `left` = rows of that block in range
  auto load_step = [&](uint32_t (&slot)[SLOT], int ent, int step, int left) {
    const int i = step_block(step);
    const int64_t base = (int64_t)__builtin_amdgcn_readlane(ent, i) * blk_stride + head_off;
    if (!step_is_v(step)) {
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
        const int row = 4 * quad + r < left ? 4 * quad + r : 0;
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
  auto rows_left = [&](int nt, int step) {
    return nt - (wave + kWaves * step_block(step)) * kBlockSize;
  };

  int ent_cur = lb_spec <= last_lb ? ent_spec : ent_first;  // == fetch_entries(0)
  int ent_nxt = ONE ? 0 : fetch_entries(nchunks > 1 ? 1 : 0);
  const int nt0 = min(kChunk, t_end - t_begin);
  uint32_t ring[kDepth][SLOT];
#pragma unroll
  for (int s = 0; s < kDepth; ++s) load_step(ring[s], ent_cur, s, rows_left(nt0, s));

  for (int c = 0; c < nchunks; ++c) {
    const int c0 = t_begin + c * kChunk;
    const int nt = min(kChunk, t_end - c0);
    const int nt_next = min(kChunk, t_end - c0 - kChunk);
    floatx4_t st[2][CT];  // raw scores of the pair: keys 4*quad+e of its two blocks
    uint4 pa[CT];         // bf16 probabilities of the pair (PV A operand)

    static_for<STEPS>([&](auto step_c) {
      constexpr int step = decltype(step_c)::value;
      uint32_t(&cur)[SLOT] = ring[step % kDepth];
      constexpr int i = step_block(step);

      if constexpr (!step_is_v(step)) {
        // ---- QK on block i ----------------------------------------------------------
        constexpr int h = step % 2;  // first or second block of the pair
        const int kb = c0 + (wave + kWaves * i) * kBlockSize + 4 * quad;  // key of element 0
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = mfma_bf16(make_uint4(cur[4 * ks], cur[4 * ks + 1], cur[4 * ks + 2], cur[4 * ks + 3]),
                            qb[ct][ks], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) st[h][ct][e] = kb + e < lim[ct] ? acc[e] : -INFINITY;
        }
        constexpr int ns = step + kDepth;
        if constexpr (ns < STEPS) load_step(cur, ent_cur, ns, rows_left(nt, ns));
        else if constexpr (!ONE) load_step(cur, ent_nxt, ns - STEPS, rows_left(nt_next, ns - STEPS));

        if constexpr (h == 1) {
          // ---- P: the pair's probabilities against a lazily raised reference ------------
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            // scores are finite or a masked -inf, so the NaN-propagating max is exact
            float mx = maxn(maxn(maxn(st[0][ct][0], st[0][ct][1]), maxn(st[0][ct][2], st[0][ct][3])),
                            maxn(maxn(st[1][ct][0], st[1][ct][1]), maxn(st[1][ct][2], st[1][ct][3])));
            mx = maxn_swap32(maxn_swap16(mx));
            const bool raise = mx > m_ref[ct] + lazy_raw;  // false for -inf pairs
            if (__builtin_amdgcn_ballot_w64(raise)) {
              const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref[ct] - mx) * scale_log2) : 1.f;
              m_ref[ct] = raise ? mx : m_ref[ct];
              // accumulator lane (col, quad) holds rows 4*quad+e: their alphas live in lanes 4*quad+e
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float a = __shfl(alpha, 4 * quad + e);
                lacc[ct][e] *= a;
#pragma unroll
                for (int s = 0; s < DPL; ++s) o[ct][s][e] *= a;
              }
            }
            const float refc = m_ref[ct] == -INFINITY ? 0.f : m_ref[ct] * scale_log2;
            pa[ct].x = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[0][ct][0], scale_log2, -refc)),
                                  __builtin_amdgcn_exp2f(fmaf(st[0][ct][1], scale_log2, -refc)));
            pa[ct].y = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[0][ct][2], scale_log2, -refc)),
                                  __builtin_amdgcn_exp2f(fmaf(st[0][ct][3], scale_log2, -refc)));
            pa[ct].z = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[1][ct][0], scale_log2, -refc)),
                                  __builtin_amdgcn_exp2f(fmaf(st[1][ct][1], scale_log2, -refc)));
            pa[ct].w = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[1][ct][2], scale_log2, -refc)),
                                  __builtin_amdgcn_exp2f(fmaf(st[1][ct][3], scale_log2, -refc)));
          }
        }
      } else if constexpr (step % 2 == 1) {
        // ---- PV on the pair ----------------------------------------------------------------
        uint32_t(&va)[SLOT] = ring[(step - 1) % kDepth];
        uint32_t(&vb)[SLOT] = cur;
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
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) o[ct][s] = mfma_bf16(pa[ct], bv, o[ct][s]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) lacc[ct] = mfma_bf16(pa[ct], ones, lacc[ct]);
        constexpr int na = step - 1 + kDepth, nb = step + kDepth;
        if constexpr (nb < STEPS) {
          load_step(va, ent_cur, na, rows_left(nt, na));
          load_step(vb, ent_cur, nb, rows_left(nt, nb));
        } else if constexpr (!ONE) {
          load_step(va, ent_nxt, na - STEPS, rows_left(nt_next, na - STEPS));
          load_step(vb, ent_nxt, nb - STEPS, rows_left(nt_next, nb - STEPS));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!ONE) {
      ent_cur = ent_nxt;
      ent_nxt = fetch_entries(c + 2 < nchunks ? c + 2 : nchunks - 1);
    }
  }

  // ---- combine the waves through LDS, write ----------------------------------------
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = ct * 16 + 4 * quad + e;
      if (row < R) {
#pragma unroll
        for (int s = 0; s < DPL; ++s) red[wave][row][s * 16 + col] = o[ct][s][e];
        if (col == 0) st_l[wave][row] = lacc[ct][e];
      }
    }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    if (quad == 0 && ct * 16 + col < R)
      st_m[wave][ct * 16 + col] = m_ref[ct] == -INFINITY ? -INFINITY : m_ref[ct] * scale_log2;
  __syncthreads();
  for (int e = threadIdx.x; e < R * D / 4; e += blockDim.x) {
    const int r = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    const int n = d4 / DPL, s0 = d4 % DPL;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w][r]);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = st_m[w][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st_m[w][r] - M);
      const float* rr = &red[w][r][s0 * 16 + n];
      sum.x += wt * rr[0]; sum.y += wt * rr[16]; sum.z += wt * rr[32]; sum.w += wt * rr[48];
      lsum += wt * st_l[w][r];
    }
    // a row without a visible key here contributes nothing: zeros, lse -inf
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int64_t grow = ((int64_t)b * NQ + r / G) * Hq + hq0 + r % G;
    if (SPLIT) {
      *reinterpret_cast<float4*>(o_part + (grow * num_parts + p) * D + d4) =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
      if (d4 == 0) lse[grow * num_parts + p] = lsum > 0.f ? M + log2f(lsum) : -INFINITY;
    } else {
      uint2 ov;
      ov.x = pack_bf16x2(sum.x * inv, sum.y * inv);
      ov.y = pack_bf16x2(sum.z * inv, sum.w * inv);
      *reinterpret_cast<uint2*>(out + grow * D + d4) = ov;
    }
  }
}

// ---------------------------------------------------------------------------
// Single-chunk partitions (up to 64 * NW tokens) with two row tiles: NW waves
// (4, two workgroups per CU, or 8, one), each with 8 blocks (4 pairs), K
// through a 4-slot register ring (two pairs ahead) and V copied from memory
// straight into 4 LDS slots per wave (buffer_load_dwordx4 ... lds, two pairs
// ahead), so a wave keeps two whole block pairs in flight where the register
// ring of decode_multi_kernel holds one.  Both go through buffer loads: with
// an LDS copy in flight the compiler makes every wait on a global load a full
// drain, but counts buffer loads and buffer copies in one ordered stream, so
// each product waits for its own block only.
// A V slot holds the block's 16 rows with the 16-byte pieces of each row
// permuted (piece c of row r at position c ^ vswz(r)).  PV reads its B operand
// with ds_read_b64_tr_b16: within a 16-lane group, lane 4i+c addresses row
// 4*quad+i, dims 16t+4c..16t+4c+3, and lane n receives rows 4*quad..4*quad+3
// at dim 16t+n, so output tile t holds dims 16t+col.  The permutation puts the
// 32 lanes of each half-wave on distinct bank pairs.  At the end each wave
// parks its rows in its own (consumed) slots for the merge.
// ---------------------------------------------------------------------------
constexpr int kNt = 2;  // buffer cache policy: non-temporal (read once)
typedef uint32_t u32x4b_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over one block of one head (4 KiB at most): base, no
// stride, range, the gfx9 format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, 4096, 0x00020000);
}

// 16 bytes per lane at byte offset `off` of the descriptor's range, into registers
// or (DMA) into LDS at lds + 16 * lane.  Plain device functions: a builtin
// called directly in a kernel template keeps the host pass from emitting its
// launch stub.
__device__ __forceinline__ u32x4b_t buf_load16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(u32x4b_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNt));
}
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t rs, void* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr<void>(lds), 16, off, 0, 0, kNt);
}

template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

template <int D, int G, int NW>
__global__ void __launch_bounds__(64 * NW, NW == 8 ? 1 : 2)
decode_multi_lds_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                        const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                        const int32_t* __restrict__ context_lens, int NQ, int Hkv, int max_blocks,
                        float scale_log2, int part_tokens, int num_parts,
                        float* __restrict__ o_part, float* __restrict__ lse) {
  constexpr int CT = 2;
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;          // PV output tiles (16 dims each)
  constexpr int SLOT = 4 * KS;        // dwords per lane of a K block
  constexpr int RB = D * 2;           // bytes of one V row
  constexpr int VB = kBlockSize * RB; // bytes of one V block of one head
  constexpr int NDMA = VB / 1024;     // 1 KiB DMA instructions per block
  constexpr int ROWS = 16 * CT;
  static_assert(ROWS * D * 4 == 4 * VB, "a wave's merge rows fill its four V slots");

  // V slots, one array each (lets the wait counters track each slot's DMA);
  // after the last PV, wave w's four slots hold its rows r of the merge in
  // slot r / 8.
  __shared__ __align__(16) uint8_t vs0[NW][VB], vs1[NW][VB], vs2[NW][VB], vs3[NW][VB];
  __shared__ float st_m[NW][ROWS], st_l[NW][ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int hq0 = g * G;
  const int R = NQ * G;
  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int L = context_lens[b];
  const int lb0 = p * part_tokens / kBlockSize;
  const int lb_spec = lb0 + wave + NW * (threadIdx.x & 7);
  const int ent_spec = bt_row[min(lb_spec, max_blocks - 1)];
  const int ent_first = bt_row[lb0];
  const int col = lane & 15, quad = lane >> 4;

  uint4 qraw[CT][KS];
  int qrow_i[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = min(ct * 16 + col, R - 1);
    qrow_i[ct] = r / G;
    const uint16_t* qrow = q + (((int64_t)b * NQ + r / G) * Hq + hq0 + r % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ct][ks] = *reinterpret_cast<const uint4*>(qrow + ks * 32 + quad * 8);
  }
  asm volatile("" ::"v"(ent_spec), "s"(ent_first), "s"(L));

  const int t_begin = p * part_tokens;
  if (t_begin >= L) return;
  const int t_end = min(t_begin + part_tokens, L);

  uint4 qb[CT][KS];
  int lim[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const bool valid = ct * 16 + col < R;
    lim[ct] = valid ? min(t_end, L - NQ + qrow_i[ct] + 1) : t_begin;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = valid ? qraw[ct][ks] : make_uint4(0u, 0u, 0u, 0u);
  }

  floatx4_t o[CT][NT];  // O[row 16ct + 4quad + e][dim 16t + col] in o[ct][t][e]
  floatx4_t lacc[CT];
  float m_ref[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    lacc[ct] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_ref[ct] = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[ct][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float lazy_raw = kLazyLog2 / scale_log2;

  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;
  const int last_lb = (t_end - 1) / kBlockSize;
  const int nt = t_end - t_begin;
  const int lane_k = col * D + quad * 8;
  const uint4 ones = make_uint4(kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2);
  const int ent = lb_spec <= last_lb ? ent_spec : ent_first;  // entry of block lane & 7 (clamped)

  uint8_t* const vslot[4] = {vs0[wave], vs1[wave], vs2[wave], vs3[wave]};
  auto rows_left = [&](int i) { return nt - (wave + NW * i) * kBlockSize; };
  auto block_base = [&](int i) {
    return (int64_t)__builtin_amdgcn_readlane(ent, i) * blk_stride + head_off;
  };
  // a descriptor per block, so every offset stays inside its 4 KiB
  auto load_k = [&](uint32_t (&slot)[SLOT], int i) {
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(k_cache + block_base(i));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4b_t t = buf_load16(rs, 2 * lane_k + 64 * ks);
      slot[4 * ks] = t.x; slot[4 * ks + 1] = t.y; slot[4 * ks + 2] = t.z; slot[4 * ks + 3] = t.w;
    }
  };
  // V block i into slot s: DMA lane `lane` of instruction m fills LDS bytes
  // m*1024 + 16*lane, i.e. row r, position c; it reads piece c ^ vswz(r) of
  // row r (row 0 for rows past the range: finite data under p = 0)
  auto load_v = [&](uint8_t* slot, int i) {
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(v_cache + block_base(i));
    const int left = rows_left(i);
#pragma unroll
    for (int m = 0; m < NDMA; ++m) {
      const int byte = m * 1024 + 16 * lane;
      const int r = byte / RB, c = (byte % RB) / 16;
      const int sr = r < left ? r : 0;
      buf_lds16(rs, slot + m * 1024, sr * RB + ((c ^ vswz<D>(r)) << 4));
    }
  };

  // PV read address of this lane inside a slot for tile 0 (tile t: ^ 32t)
  const int vr = 4 * quad + (col >> 2), vc = col & 3;
  const int v_lane = vr * RB + ((vswz<D>(vr) >> 1) << 5) + (vc << 3);

  uint32_t kr[4][SLOT];
  load_k(kr[0], 0); load_k(kr[1], 1);
  load_v(vslot[0], 0); load_v(vslot[1], 1);
  load_k(kr[2], 2); load_k(kr[3], 3);
  load_v(vslot[2], 2); load_v(vslot[3], 3);

  static_for<4>([&](auto j_c) {
    constexpr int j = decltype(j_c)::value;
    floatx4_t st[2][CT];
    uint4 pa[CT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t(&cur)[SLOT] = kr[(2 * j + h) % 4];
      const int kb = t_begin + (wave + NW * (2 * j + h)) * kBlockSize + 4 * quad;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = mfma_bf16(make_uint4(cur[4 * ks], cur[4 * ks + 1], cur[4 * ks + 2], cur[4 * ks + 3]),
                          qb[ct][ks], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) st[h][ct][e] = kb + e < lim[ct] ? acc[e] : -INFINITY;
      }
    }
    if constexpr (j + 2 < 4) {
      load_k(kr[(2 * j) % 4], 2 * j + 4);
      load_k(kr[(2 * j + 1) % 4], 2 * j + 5);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float mx = maxn(maxn(maxn(st[0][ct][0], st[0][ct][1]), maxn(st[0][ct][2], st[0][ct][3])),
                      maxn(maxn(st[1][ct][0], st[1][ct][1]), maxn(st[1][ct][2], st[1][ct][3])));
      mx = maxn_swap32(maxn_swap16(mx));
      const bool raise = mx > m_ref[ct] + lazy_raw;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref[ct] - mx) * scale_log2) : 1.f;
        m_ref[ct] = raise ? mx : m_ref[ct];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = __shfl(alpha, 4 * quad + e);
          lacc[ct][e] *= a;
#pragma unroll
          for (int t = 0; t < NT; ++t) o[ct][t][e] *= a;
        }
      }
      const float refc = m_ref[ct] == -INFINITY ? 0.f : m_ref[ct] * scale_log2;
      pa[ct].x = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[0][ct][0], scale_log2, -refc)),
                            __builtin_amdgcn_exp2f(fmaf(st[0][ct][1], scale_log2, -refc)));
      pa[ct].y = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[0][ct][2], scale_log2, -refc)),
                            __builtin_amdgcn_exp2f(fmaf(st[0][ct][3], scale_log2, -refc)));
      pa[ct].z = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[1][ct][0], scale_log2, -refc)),
                            __builtin_amdgcn_exp2f(fmaf(st[1][ct][1], scale_log2, -refc)));
      pa[ct].w = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[1][ct][2], scale_log2, -refc)),
                            __builtin_amdgcn_exp2f(fmaf(st[1][ct][3], scale_log2, -refc)));
    }
    uint8_t* const va = vslot[(2 * j) % 4];
    uint8_t* const vb = vslot[(2 * j + 1) % 4];
    // recomputed per pair (kept from pair j to j + 2, the addresses would spill)
    int vl = v_lane;
    asm volatile("" : "+v"(vl));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const shortx4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<shortx4_t>(va + (vl ^ (t << 5))));
      const shortx4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<shortx4_t>(vb + (vl ^ (t << 5))));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      const uint4 bv = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct][t] = mfma_bf16(pa[ct], bv, o[ct][t]);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) lacc[ct] = mfma_bf16(pa[ct], ones, lacc[ct]);
    if constexpr (j + 2 < 4) {
      load_v(va, 2 * j + 4);
      load_v(vb, 2 * j + 5);
    }
    __builtin_amdgcn_sched_barrier(0);
  });

  // ---- combine the waves through LDS (each wave's rows over its own V slots) ----
  // row r of wave w: slot r / 8 of wave w, at (r % 8) * D floats
  auto red_row = [&](int w, int r) -> float* {
    uint8_t* base = r < 8 ? vs0[w] : r < 16 ? vs1[w] : r < 24 ? vs2[w] : vs3[w];
    return reinterpret_cast<float*>(base) + (r & 7) * D;
  };
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = ct * 16 + 4 * quad + e;
      if (row < R) {
        float* rr = red_row(wave, row);
#pragma unroll
        for (int t = 0; t < NT; ++t) rr[t * 16 + col] = o[ct][t][e];
        if (col == 0) st_l[wave][row] = lacc[ct][e];
      }
    }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    if (quad == 0 && ct * 16 + col < R)
      st_m[wave][ct * 16 + col] = m_ref[ct] == -INFINITY ? -INFINITY : m_ref[ct] * scale_log2;
  __syncthreads();
  for (int e = threadIdx.x; e < R * D / 4; e += blockDim.x) {
    const int r = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, st_m[w][r]);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = st_m[w][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st_m[w][r] - M);
      const float4 v = *reinterpret_cast<const float4*>(red_row(w, r) + d4);
      sum.x += wt * v.x; sum.y += wt * v.y; sum.z += wt * v.z; sum.w += wt * v.w;
      lsum += wt * st_l[w][r];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int64_t grow = ((int64_t)b * NQ + r / G) * Hq + hq0 + r % G;
    *reinterpret_cast<float4*>(o_part + (grow * num_parts + p) * D + d4) =
        make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    if (d4 == 0) lse[grow * num_parts + p] = lsum > 0.f ? M + log2f(lsum) : -INFINITY;
  }
}

template <int D, int G, int CT>
hipError_t launch_g(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* bt, const int32_t* cl, int B, int NQ,
                    int Hkv, int mb, int mcl, float scale, int P, hipStream_t stream) {
  const float sl = scale * 1.4426950408889634f;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  auto* oo = static_cast<uint16_t*>(out);
  if (P > 0) {
    const int np = (mcl + P - 1) / P;
    if (P <= kChunkTokens && CT == 2)
      hipLaunchKernelGGL((decode_multi_lds_kernel<D, G, 4>), dim3(np, Hkv, B), dim3(256), 0,
                         stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, P, np, o_part, lse);
    else if (P <= kChunkTokens)
      hipLaunchKernelGGL((decode_multi_kernel<D, G, CT, true, true, 4>), dim3(np, Hkv, B), dim3(256), 0,
                         stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, P, np, oo, o_part, lse);
    else if (P <= 2 * kChunkTokens && CT == 2)
      hipLaunchKernelGGL((decode_multi_lds_kernel<D, G, 8>), dim3(np, Hkv, B), dim3(512), 0,
                         stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, P, np, o_part, lse);
    else if (P <= 2 * kChunkTokens)
      hipLaunchKernelGGL((decode_multi_kernel<D, G, CT, true, true, 8>), dim3(np, Hkv, B), dim3(512), 0,
                         stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, P, np, oo, o_part, lse);
    else
      hipLaunchKernelGGL((decode_multi_kernel<D, G, CT, true, false, 4>), dim3(np, Hkv, B), dim3(256), 0,
                         stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, P, np, oo, o_part, lse);
  } else {
    hipLaunchKernelGGL((decode_multi_kernel<D, G, CT, false, false, 4>), dim3(1, Hkv, B), dim3(256), 0,
                       stream, qq, kc, vc, bt, cl, NQ, Hkv, mb, sl, 0, 1, oo, o_part, lse);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_ct(void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* bt, const int32_t* cl, int B, int NQ,
                     int Hkv, int mb, int mcl, float scale, int P, hipStream_t stream) {
  if (NQ * G <= 16)
    return launch_g<D, G, 1>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, NQ, Hkv, mb, mcl, scale, P, stream);
  return launch_g<D, G, 2>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, NQ, Hkv, mb, mcl, scale, P, stream);
}

template <int D>
hipError_t launch_d(int G, void* out, float* o_part, float* lse, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* bt, const int32_t* cl, int B, int NQ,
                    int Hkv, int mb, int mcl, float scale, int P, hipStream_t st) {
  switch (G) {
#define PA_MULTI_G(GG) \
    case GG: return launch_ct<D, GG>(out, o_part, lse, q, k_cache, v_cache, bt, cl, B, NQ, Hkv, mb, mcl, scale, P, st);
    PA_MULTI_G(1) PA_MULTI_G(2) PA_MULTI_G(3) PA_MULTI_G(4)
    PA_MULTI_G(5) PA_MULTI_G(6) PA_MULTI_G(7) PA_MULTI_G(8)
#undef PA_MULTI_G
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_multi(void* out, float* o_part, float* lse, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int B,
                               int NQ, int Hq, int Hkv, int D, int max_blocks, int max_context_len,
                               float scale, int partition_size, hipStream_t stream) {
  const int G = Hq / Hkv;
  if (D == 128)
    return launch_d<128>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens, B,
                         NQ, Hkv, max_blocks, max_context_len, scale, partition_size, stream);
  return launch_d<64>(G, out, o_part, lse, q, k_cache, v_cache, block_tables, context_lens, B, NQ,
                      Hkv, max_blocks, max_context_len, scale, partition_size, stream);
}

}  // namespace pa
