// Shared-prefix pass of the decode step for gfx950 on bf16 matrix cores: the
// queries of a group of decode sequences that share their first blocks attend
// that prefix once, together, and leave split-K partials for the reduce.
//
// Operation (mini-llm-engine post, §3.4: full blocks of a common prefix shared
// by several sequences, ref_count > 1; Pico-vLLM write-up, §2: decode kernel in
// the manner of Flash Attention, and the H200 comparison: Flash Decode's split
// and log-sum-exp reduce): for every (sequence s of the group, query head h)
// row and one partition [kbeg, kend) of the shared prefix, the partial
// softmax(scale * q K^T) V over those keys, normalised, with its base-2
// log-sum-exp; GQA query head h reads KV head h / G.
//
// Rows are (sequence, head) pairs of one KV head, r = s * G + h, so the G
// query heads sharing a KV head share every K/V tile.  Workgroup = 8 waves
// over 128 rows: the partition's keys are split in two halves, and wave w takes
// row tiles 2(w%4), 2(w%4)+1 (16 rows each) over half w/4.  Each half streams
// its keys in steps of 64 (four 16-token blocks) through a double-buffered LDS
// stage, filled from registers loaded one step ahead.  Per step and wave:
//   QK   S^T (keys x rows) = K Q^T with v_mfma_f32_16x16x32_bf16: A = K tile
//        from LDS (16-byte chunks XOR-swizzled by key), B = the rows' queries
//        (registers).
//   P    per row the running reference max is raised only when a step's max
//        exceeds it by more than 2^8 (p then stays below 256: exact enough in
//        bf16, safe in fp32 sums), which spares nearly every rescale of the
//        accumulators.  Keys past the partition end are masked by selects.
//        p is rounded to bf16; the S^T accumulator layout is already the B
//        operand of the PV product, so p never moves.
//   PV   O^T (dims x rows) += V^T P^T: A = V^T from LDS, V stored transposed
//        with the key order the P operand implies (8 keys of a lane
//        contiguous) and a 144-byte row stride (64 keys + 8 of padding); a
//        ninth product against a ones operand accumulates the normaliser.
// The two halves meet through LDS at the end (log-sum-exp merge).  Keys at or
// past the partition end are loaded from valid rows and never reach a product
// with a nonzero weight; their table entries are never used as block ids.
// (The chunked prefill itself is k_prefill_chunk.hip.)

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kHalves = 2;                       // key ranges per workgroup
constexpr int kWavesPerHalf = 4;
constexpr int kThreads = 64 * kHalves * kWavesPerHalf;  // 512
constexpr int kHalfThreads = 64 * kWavesPerHalf;        // 256: one half's stream
constexpr int kRowTiles = 2;                     // 16-row tiles per wave
constexpr int kRowsPerWave = 16 * kRowTiles;     // 32
constexpr int kRowsPerWG = kWavesPerHalf * kRowsPerWave;  // 128
constexpr int kStepBlocks = 4;                   // 16-token blocks per step
constexpr int kStepKeys = kStepBlocks * kBlockSize;  // 64
constexpr int kPairs = kStepBlocks / 2;          // 32-key PV products per step
constexpr int kVtStride = kStepKeys + 8;         // bf16 per V^T row: 64 keys + 8 pad (144 bytes)
constexpr float kLazyLog2 = 8.f;                 // reference max may lag the true one by 2^8

// LDS position of key k (0..63) in a V^T row: per 32-key pair, lane group q
// reads its 8 keys 4q..4q+3 and 16+4q..16+4q+3 (the keys its S^T registers
// hold) contiguously.
__device__ __forceinline__ int vt_pos(int k) {
  const int kk = k & 31;
  return (k & 32) + (kk < 16 ? 8 * (kk >> 2) + (kk & 3) : 8 * ((kk - 16) >> 2) + 4 + (kk & 3));
}

__device__ __forceinline__ floatx4_t mfma_bf16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// Shared-prefix mode (PART): a group of decode sequences sharing their first
// blocks.  Group gi is sequences group_start[gi] .. group_start[gi+1]-1, all
// with the same first prefix_lens[group_start[gi]] tokens (whole blocks, read
// through the first sequence's table).  Workgroup (rb, g, gi*parts + kp)
// takes rows (sequence s of the group, head h) r = s*G + h, and keys
// [kp*part_tokens, min((kp+1)*part_tokens, prefix)) with no causal mask, and
// writes the normalised fp32 partial and its base-2 log-sum-exp to slot
// slot0 + kp of each row, in the split-K workspace layout.
struct GroupArgs {
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int part_tokens;  // multiple of kStepKeys
  int parts;        // partitions per group (grid z = groups * parts)
  int slot0;        // first workspace slot of the prefix partitions
  int num_slots;    // slots per row in the workspace
  float* o_part;    // [B][Hq][num_slots][D]
  float* lse;       // [B][Hq][num_slots]
};

template <int D, int G, bool PART>  // PART: the shared-prefix pass (the only mode launched)
__global__ void __launch_bounds__(kThreads)
prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
               const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
               const int32_t* __restrict__ query_start_loc, int Hkv, int max_blocks,
               float scale_log2, const GroupArgs ga) {
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int KS = D / 32;         // MFMA k-steps over the head dimension
  constexpr int DT = D / 16;         // 16-dim output tiles
  constexpr int K_LOADS = kStepKeys * NCH / kHalfThreads;        // K chunks per thread per step
  constexpr int V_LOADS = (kStepKeys / 2) * NCH / kHalfThreads;  // (key pair, 8-dim) V units
  static_assert(K_LOADS >= 1 && V_LOADS >= 1 && (kStepKeys / 2) * NCH % kHalfThreads == 0,
                "tile loads spread evenly over a half's threads");
  constexpr int KS_BYTES = kStepKeys * D * 2;
  constexpr int VT_BYTES = D * kVtStride * 2;
  constexpr int BUF_BYTES = KS_BYTES + VT_BYTES;
  constexpr int MERGE_FLOATS = kWavesPerHalf * kRowTiles * (DT * 4 + 2) * 64;
  static_assert(MERGE_FLOATS * 4 <= kHalves * 2 * BUF_BYTES, "merge area fits the tile buffers");

  __shared__ __align__(16) unsigned char lds[kHalves][2][BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave / kWavesPerHalf, hw = wave % kWavesPerHalf;
  const int htid = tid % kHalfThreads;
  const int col = lane & 15, quad = lane >> 4;
  const int rb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;

  // Chunked prefill: rows of sequence b's chunk, keys [0, kmax) under the
  // causal limits.  Shared prefix: rows of group gi, keys [kbeg, L) where L
  // is the partition's end (keys past it are treated as past the sequence).
  int q0, C, L, kbeg = 0, kp = 0;
  int32_t seq_first;  // sequence whose table is read
  if constexpr (PART) {
    const int gi = b / ga.parts;
    kp = b % ga.parts;
    q0 = ga.group_start[gi];
    C = ga.group_start[gi + 1] - q0;  // sequences of the group
    const int pre = ga.prefix_lens[q0];
    kbeg = kp * ga.part_tokens;
    if (kbeg >= pre) return;
    L = min(kbeg + ga.part_tokens, pre);
    seq_first = q0;
  } else {
    q0 = query_start_loc[b];
    C = query_start_loc[b + 1] - q0;
    L = context_lens[b];
    seq_first = b;
  }
  const int nrows = C * G;
  const int row0_wg = rb * kRowsPerWG;
  if (row0_wg >= nrows) return;
  const int pos_last = min(nrows, row0_wg + kRowsPerWG) - 1;  // last valid row of the WG
  // keys any row of this workgroup can see: up to position L - C + pos_max
  const int kmax = PART ? L : min(L, L - C + pos_last / G + 1);
  const int tbase = kbeg / kStepKeys;
  const int ntiles = (kmax - kbeg + kStepKeys - 1) / kStepKeys;
  const int nsteps = (ntiles + 1) / 2;                 // tiles of half 0 (half 1 has <= as many)
  const int tile0 = tbase + half * nsteps;             // first tile of this wave's half
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;
  const int32_t* bt_row = block_tables + (int64_t)seq_first * max_blocks;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;

  // ---- this lane's rows: one per row tile (lane column) ----------------------
  int lim[kRowTiles];  // last visible key of the row
  bool rvalid[kRowTiles];
  bf16x8_t qb[kRowTiles][KS];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = row0_wg + hw * kRowsPerWave + rt * 16 + col;
    rvalid[rt] = r < nrows;
    const int pos = rvalid[rt] ? r / G : 0;
    const int h = rvalid[rt] ? r % G : 0;
    lim[rt] = PART ? L - 1 : rvalid[rt] ? L - C + pos : L - 1;
    const uint16_t* qrow = q + ((int64_t)(q0 + pos) * Hq + g * G + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 t = *reinterpret_cast<const uint4*>(qrow + ks * 32 + quad * 8);
      if (!rvalid[rt]) t = make_uint4(0u, 0u, 0u, 0u);
      qb[rt][ks] = __builtin_bit_cast(bf16x8_t, t);
    }
  }
  // smallest causal limit over the workgroup's rows (tiles past it need masks)
  const int lim_min_wg = PART ? L - 1 : L - C + row0_wg / G;

  // ---- staging: global -> registers -> LDS ----------------------------------------
  // A step is kStepBlocks blocks.  Every load is unconditional, from an
  // address that is always valid, so no branch splits the load stream:
  //  * table entries are clamped into the sequence's blocks; they are
  //    wave-uniform scalar loads (a per-lane entry load would make the data
  //    loads behind it wait for every load in flight);
  //  * K rows at or past L are loaded but never seen: their scores are
  //    replaced by -inf;
  //  * V rows at or past L are redirected to the first row of the step (a
  //    key below L), so NaN in unused slots cannot meet a zero probability.
  // Steps past the half's range are loaded the same way and never computed.
  struct Stage { u32x4_t k[K_LOADS]; u32x4_t v0[V_LOADS], v1[V_LOADS]; };  // native vectors: no memcpy, no stack
  // A step's four table entries are read one step before its data, so the
  // four scalar loads are in flight together and their latency is hidden.
  struct Entries { int e[kStepBlocks]; };
  static_assert(kStepBlocks == 4, "four table entries per step");
  auto load_entries = [&](int tt) -> Entries {
    const int lb0 = tt * kStepBlocks;
    Entries en;
#pragma unroll
    for (int i = 0; i < kStepBlocks; ++i) en.e[i] = bt_row[min(lb0 + i, nblk_seq - 1)];
    return en;
  };
  auto load_tile = [&](int tt, const Entries& en) -> Stage {
    Stage st;
    const int lb0 = tt * kStepBlocks;
    const int ent0 = en.e[0], ent1 = en.e[1], ent2 = en.e[2], ent3 = en.e[3];
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      // chunk c: block c / (16 NCH), key row, 16-byte chunk (coalesced rows)
      const int c = htid + kHalfThreads * i;
      const int key = (c / NCH) % kBlockSize;
      const int ch = c % NCH;
      const int blk = c / (kBlockSize * NCH);
      const int e = blk == 0 ? ent0 : blk == 1 ? ent1 : blk == 2 ? ent2 : ent3;
      st.k[i] = *reinterpret_cast<const u32x4_t*>(k_cache + (int64_t)e * blk_stride + head_off +
                                                  key * D + ch * 8);
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      // V unit u: keys 2(u % 32), 2(u % 32)+1 of the step, dims 8(u / 32) .. +7
      const int u = htid + kHalfThreads * j;
      const int k0 = 2 * (u % (kStepKeys / 2));
      const int t = lb0 * kBlockSize + k0;
      const int vb = k0 / kBlockSize;
      const int e = vb == 0 ? ent0 : vb == 1 ? ent1 : vb == 2 ? ent2 : ent3;
      const int e_a = t < L ? e : ent0, r_a = t < L ? k0 % kBlockSize : 0;
      const int e_b = t + 1 < L ? e : ent0, r_b = t + 1 < L ? k0 % kBlockSize + 1 : 0;
      const uint16_t* vsrc = v_cache + head_off + (u / (kStepKeys / 2)) * 8;
      st.v0[j] = *reinterpret_cast<const u32x4_t*>(vsrc + (int64_t)e_a * blk_stride + r_a * D);
      st.v1[j] = *reinterpret_cast<const u32x4_t*>(vsrc + (int64_t)e_b * blk_stride + r_b * D);
    }
    return st;
  };
  auto store_tile = [&](const Stage& st, int buf) {
    unsigned char* ks_base = lds[half][buf];
    uint16_t* vt_base = reinterpret_cast<uint16_t*>(lds[half][buf] + KS_BYTES);
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = htid + kHalfThreads * i;
      const int key = (c / NCH) % kBlockSize + kBlockSize * (c / (kBlockSize * NCH));
      const int ch = c % NCH;
      *reinterpret_cast<u32x4_t*>(ks_base + key * D * 2 + ((ch ^ (key & (NCH - 1))) * 16)) = st.k[i];
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int u = htid + kHalfThreads * j;
      const int k0 = 2 * (u % (kStepKeys / 2));
      const int d0 = 8 * (u / (kStepKeys / 2));
      uint32_t* dst = reinterpret_cast<uint32_t*>(vt_base + d0 * kVtStride + vt_pos(k0));
      const uint32_t a[4] = {st.v0[j].x, st.v0[j].y, st.v0[j].z, st.v0[j].w};
      const uint32_t c[4] = {st.v1[j].x, st.v1[j].y, st.v1[j].z, st.v1[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims 2e, 2e+1 of the chunk: (key k0, key k0+1) pairs
        dst[(2 * e) * kVtStride / 2] = interleave_lo(a[e], c[e]);
        dst[(2 * e + 1) * kVtStride / 2] = interleave_hi(a[e], c[e]);
      }
    }
  };

  floatx4_t o[DT][kRowTiles];
  floatx4_t lacc[kRowTiles];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    lacc[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  float m_ref[kRowTiles];  // reference max of the row (raw scores; -inf: none seen)
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) m_ref[rt] = -INFINITY;
  const float lazy_raw = kLazyLog2 / scale_log2;
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                0x3F803F80u, 0x3F803F80u));

  // One step of this half from LDS buffer `buf`, then the next step's tile
  // into the other buffer.  DIAG: some key of the step is past some row's
  // causal limit, so scores need the selects; the two instantiations keep each
  // step one straight-line block, so the row maxima interleave with the QK
  // products and the store of the next tile with the PV products.
  auto step = [&](auto diag_c, int tt, int buf, const Stage& nx) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const unsigned char* ks_base = lds[half][buf];
    const uint16_t* vt_base = reinterpret_cast<const uint16_t*>(lds[half][buf] + KS_BYTES);
    const int key0 = tt * kStepKeys;

    // ---- QK: S^T for kStepBlocks key tiles x 2 row tiles, row maxima as they come
    // (scores are finite or a masked -inf, so the NaN-propagating max is exact)
    floatx4_t st[kStepBlocks][kRowTiles];
    float mt[kRowTiles];
#pragma unroll
    for (int kt = 0; kt < kStepBlocks; ++kt) {
      const int key = kt * 16 + col;
      bf16x8_t ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 4 + quad;
        ka[ks] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(ks_base + key * D * 2 + ((ch ^ (key & (NCH - 1))) * 16)));
      }
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        st[kt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st[kt][rt] = mfma_bf16(ka[ks], qb[rt][ks], st[kt][rt]);
      }
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        if constexpr (DIAG) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st[kt][rt][j] = key0 + kt * 16 + quad * 4 + j <= lim[rt] ? st[kt][rt][j] : -INFINITY;
        }
        const float m4 = maxn(maxn(st[kt][rt][0], st[kt][rt][1]), maxn(st[kt][rt][2], st[kt][rt][3]));
        mt[rt] = kt == 0 ? m4 : maxn(mt[rt], m4);
      }
    }
    // V^T operands of the first key pair: their LDS reads are in flight during
    // the softmax (the second pair's are issued at the start of the products)
    auto read_vt = [&](int pp, int dt) {
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                              vt_base + (dt * 16 + col) * kVtStride + pp * 32 + quad * 8));
    };
    bf16x8_t va0[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) va0[dt] = read_vt(0, dt);
    __builtin_amdgcn_sched_barrier(0);

    // ---- P: softmax numerators against a lazily raised reference max ------------
    bool raise[kRowTiles];
    bool any = false;
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      mt[rt] = maxn_swap32(maxn_swap16(mt[rt]));
      raise[rt] = mt[rt] > m_ref[rt] + lazy_raw;  // false for -inf steps
      any = any || raise[rt];
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        // rows that keep their reference scale by exactly 1 (their m_ref may be -inf)
        const float alpha = raise[rt] ? __builtin_amdgcn_exp2f((m_ref[rt] - mt[rt]) * scale_log2) : 1.f;
        m_ref[rt] = raise[rt] ? mt[rt] : m_ref[rt];
        lacc[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
      }
    }
    float refc[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) refc[rt] = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt] * scale_log2;
    auto probs = [&](int pp, int rt) {
      uint32_t pk[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const floatx4_t& sv = st[2 * pp + h][rt];
        pk[2 * h] = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[0], scale_log2, -refc[rt])),
                               __builtin_amdgcn_exp2f(fmaf(sv[1], scale_log2, -refc[rt])));
        pk[2 * h + 1] = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[2], scale_log2, -refc[rt])),
                                   __builtin_amdgcn_exp2f(fmaf(sv[3], scale_log2, -refc[rt])));
      }
      return __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    };

    // ---- PV: O^T += V^T P^T per 32-key pair; the second pair's probabilities are
    // computed under the first pair's products, the next tile stored under the second's
    static_assert(kPairs == 2, "two key pairs per step");
    bf16x8_t pb0[kRowTiles], pb1[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      pb0[rt] = probs(0, rt);
      lacc[rt] = mfma_bf16(ones, pb0[rt], lacc[rt]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) o[dt][rt] = mfma_bf16(va0[dt], pb0[rt], o[dt][rt]);
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      pb1[rt] = probs(1, rt);
      lacc[rt] = mfma_bf16(ones, pb1[rt], lacc[rt]);
    }
    bf16x8_t va1[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) va1[dt] = read_vt(1, dt);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) o[dt][rt] = mfma_bf16(va1[dt], pb1[rt], o[dt][rt]);
    store_tile(nx, buf ^ 1);
  };

  // ---- main loop: both halves in step ------------------------------------------------
  // Half 1 may have one step fewer than half 0; it computes that step anyway
  // (it would only wait at the barrier): the step's keys are past every row's
  // causal limit, so all its scores are masked and its probabilities are 0.
  // Steps needing the selects are the last ones of the range (tiles from
  // (lim_min_wg + 1) / 64 on), so they run in a second loop: one step body per
  // loop keeps the register allocation of each tight.  Both halves still run
  // nsteps iterations, each ending in the one workgroup barrier.
  store_tile(load_tile(tile0, load_entries(tile0)), 0);
  Entries en_next = load_entries(tile0 + 1);
  __syncthreads();
  auto iteration = [&](auto diag_c, int i) {
    // the next step's loads are in flight while this one computes
    const Stage nx = load_tile(tile0 + i + 1, en_next);
    en_next = load_entries(tile0 + i + 2);
    step(diag_c, tile0 + i, i & 1, nx);
    __syncthreads();
  };
  const int n_plain = min(max((lim_min_wg + 1) / kStepKeys - tile0, 0), nsteps);
  int i = 0;
  for (; i < n_plain; ++i) iteration(std::false_type{}, i);
  for (; i < nsteps; ++i) iteration(std::true_type{}, i);

  // ---- merge the halves through LDS, normalise and write ------------------------------
  // lane holds O^T[dims 4*quad+j of tile dt][row col]; l of row col in lacc[rt][0]
  float* mg = reinterpret_cast<float*>(&lds[0][0][0]);  // [hw][rt][DT*4 + 2][64]
  auto mg_at = [&](int rt, int k) -> float& {
    return mg[((hw * kRowTiles + rt) * (DT * 4 + 2) + k) * 64 + lane];
  };
  if (half == 1) {
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mg_at(rt, dt * 4 + j) = o[dt][rt][j];
      mg_at(rt, DT * 4) = m_ref[rt];
      mg_at(rt, DT * 4 + 1) = lacc[rt][0];
    }
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const float m1 = mg_at(rt, DT * 4), l1 = mg_at(rt, DT * 4 + 1);
    const float m0 = m_ref[rt], l0 = lacc[rt][0];
    const float M = fmaxf(m0, m1);
    const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - M) * scale_log2);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * scale_log2);
    const float lsum = w0 * l0 + w1 * l1;
    const float inv = 1.f / lsum;
    if (!rvalid[rt]) continue;
    const int r = row0_wg + hw * kRowsPerWave + rt * 16 + col;
    const int pos = r / G, h = r % G;
    if constexpr (PART) {
      // partial of row (sequence q0 + pos, head g*G + h) at slot slot0 + kp
      const int64_t slot = ((int64_t)(q0 + pos) * Hq + g * G + h) * ga.num_slots + ga.slot0 + kp;
      float* orow = ga.o_part + slot * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float4 y;
        y.x = (w0 * o[dt][rt][0] + w1 * mg_at(rt, dt * 4 + 0)) * inv;
        y.y = (w0 * o[dt][rt][1] + w1 * mg_at(rt, dt * 4 + 1)) * inv;
        y.z = (w0 * o[dt][rt][2] + w1 * mg_at(rt, dt * 4 + 2)) * inv;
        y.w = (w0 * o[dt][rt][3] + w1 * mg_at(rt, dt * 4 + 3)) * inv;
        *reinterpret_cast<float4*>(orow + dt * 16 + quad * 4) = y;
      }
      if (quad == 0) ga.lse[slot] = M * scale_log2 + log2f(lsum);
      continue;
    }
    uint16_t* orow = out + ((int64_t)(q0 + pos) * Hq + g * G + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (w0 * o[dt][rt][j] + w1 * mg_at(rt, dt * 4 + j)) * inv;
      *reinterpret_cast<uint2*>(orow + dt * 16 + quad * 4) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    }
  }
}

template <int D, bool PART>
hipError_t launch_d(int G, dim3 grid, hipStream_t stream, uint16_t* out, const uint16_t* q,
                    const uint16_t* kc, const uint16_t* vc, const int32_t* bt, const int32_t* cl,
                    const int32_t* qsl, int Hkv, int mb, float sl, const GroupArgs& ga) {
#define PA_PREFILL(GG)                                                                        \
  hipLaunchKernelGGL((prefill_kernel<D, GG, PART>), grid, dim3(kThreads), 0, stream, out, q, kc, vc, \
                     bt, cl, qsl, Hkv, mb, sl, ga)
  switch (G) {
    case 1: PA_PREFILL(1); break;
    case 2: PA_PREFILL(2); break;
    case 3: PA_PREFILL(3); break;
    case 4: PA_PREFILL(4); break;
    case 5: PA_PREFILL(5); break;
    case 6: PA_PREFILL(6); break;
    case 7: PA_PREFILL(7); break;
    case 8: PA_PREFILL(8); break;
    default: return hipErrorInvalidValue;
  }
#undef PA_PREFILL
  return hipGetLastError();
}

}  // namespace

// Shared-prefix partials of decode queries: grid (row blocks, Hkv, groups * parts).
hipError_t launch_group_prefix(float* o_part, float* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* group_start, const int32_t* prefix_lens, int groups,
                               int max_group_size, int max_prefix, int part_tokens, int slot0,
                               int num_slots, int Hq, int Hkv, int D, int max_blocks, float scale,
                               hipStream_t stream) {
  const int G = Hq / Hkv;
  const int parts = (max_prefix + part_tokens - 1) / part_tokens;
  const int rblocks = (max_group_size * G + kRowsPerWG - 1) / kRowsPerWG;
  if (groups <= 0 || parts <= 0 || rblocks <= 0) return hipSuccess;
  const dim3 grid(rblocks, Hkv, groups * parts);
  const GroupArgs ga{group_start, prefix_lens, part_tokens, parts, slot0, num_slots, o_part, lse};
  const float sl = scale * 1.4426950408889634f;
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kc = static_cast<const uint16_t*>(k_cache);
  auto* vc = static_cast<const uint16_t*>(v_cache);
  if (D == 128)
    return launch_d<128, true>(G, grid, stream, nullptr, qq, kc, vc, block_tables, nullptr, nullptr,
                               Hkv, max_blocks, sl, ga);
  return launch_d<64, true>(G, grid, stream, nullptr, qq, kc, vc, block_tables, nullptr, nullptr, Hkv,
                            max_blocks, sl, ga);
}

}  // namespace pa
