// Causal paged chunked prefill for gfx950 on bf16 matrix cores.
//
// Operation (Pico-vLLM write-up, §2: paged prefill kernel in the manner of
// Flash Attention, on the matrix cores; mini-llm-engine post, §3.3: a prompt is
// prefilled in chunks, each chunk attending the cached prefix plus itself;
// §3.1: K/V in 16-token physical blocks behind a block table): chunk row i of
// sequence b sits at position L_b - C_b + i and attends keys t <= L_b - C_b + i
// with softmax(scale * q K^T) V, GQA query head h reading KV head h / G.
//
// Rows are (position, head) pairs of one (sequence, KV head), position-major
// (r = pos * G + h), so the G query heads sharing a KV head share every K/V
// tile.  A workgroup takes 96 rows and all the keys they can see; its 12 waves
// form 4 key ranges ("quarters", consecutive runs of 32-key steps) of 3 waves,
// and each wave owns 32 rows (one 32-column tile of the 32x32 products) over
// its quarter's keys.  96-row workgroups make one workgroup per compute unit
// on the chunked-prefill shape (32 per (sequence, KV head), 8 pairs); 160
// registers per wave let three waves share each SIMD and cover each other's
// latency.
//
// Per 32-key step (two 16-token blocks) and quarter:
//   load  two of the quarter's waves each bring one block's K and V rows straight
//         from global memory into LDS (global_load_lds_dwordx4: lane i of an
//         instruction lands at byte 16*i of its 1 KiB destination), so no
//         register staging; a lane fetches the 16-byte chunk that the XOR
//         swizzle of its destination slot holds.  The next step is loaded
//         while this one computes (two LDS buffers per quarter, kept in two
//         distinct arrays so that reads of one never wait on loads into the
//         other).  V rows at or past L are fetched from row 0 of their block
//         (finite data under a zero probability: NaN in unused slots cannot
//         reach the products).
//   QK    S^T (32 keys x 32 rows) = K Q^T on v_mfma_f32_32x32x16_bf16, one chain
//         of D/16 products: A = 32 keys x 16 dims of K from LDS, B = 16 dims x
//         32 rows of the queries, held in registers.  Lane l ends with 16 keys
//         (8 (r/4) + 4 (l/32) + r%4) of row l%32.
//   P     the row's running reference max is raised only when a step's max
//         exceeds it by more than 2^8 (p then stays below 256: exact enough in
//         bf16, safe in fp32 sums), which spares nearly every rescale; causal
//         limits are selects, on steps that cross a row's limit only; p is
//         rounded to bf16, and the lane's 16 values are already the B operand
//         of PV for the key order the V^T reads below use.  The row sum
//         accumulates the same rounded p with v_dot2_f32_bf16.
//   PV    O^T (32 dims x 32 rows) += V^T P^T per 32-dim tile and 16-key half:
//         A = V^T read from the key-major V tile with the transposing
//         ds_read_b64_tr_b16 (two reads of 4 keys x 16 dims per operand).
// The quarters meet through LDS at the end (log-sum-exp merge, in two rounds
// that fit the freed tile buffers, 16 bytes per lane and access).  Workgroup
// ids are mapped (sequence, KV head)-minor, so consecutive ids -- placed on
// different XCDs -- take different pairs and each XCD's L2 serves the K/V of
// few pairs.

#include "pa_device.h"
#include "pa_internal.h"



namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kQuarters = 4;                       // key ranges per workgroup
constexpr int kWavesPerQ = 3;                      // waves sharing a key range
constexpr int kWaves = kQuarters * kWavesPerQ;     // 12
constexpr int kThreads = 64 * kWaves;              // 768
constexpr int kRowsPerWave = 32;                   // one 32-column tile per wave
constexpr int kRowsPerWG = kWavesPerQ * kRowsPerWave;  // 96
constexpr int kStepKeys = 2 * kBlockSize;          // 32 keys per step
constexpr float kLazyLog2 = 8.f;                   // reference max may lag by 2^8

template <int D>
struct Layout {
  static constexpr int ROW = 2 * D;                // bytes of one key row
  static constexpr int NCH = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = kStepKeys * ROW;     // one K or V tile of a step
  static constexpr int BUF = 2 * TILE;             // K tile, then V tile
  static constexpr int KPI = 1024 / ROW;           // key rows per 1 KiB direct load
  static constexpr int IPB = kBlockSize / KPI;     // direct loads per block and tile
  // XOR swizzles of the 16-byte chunks of a key row: in the K tile, chunk c of
  // key k sits in slot c ^ kx(k); in the V tile, in slot c ^ vx(k).  kx spreads
  // the 16 keys a 16-lane group of a K read touches over 16 slots; vx spreads
  // the 4 keys x 2 chunks of a V^T read's 16-lane group over 8 slots, and keeps
  // the two groups that read the same keys (the two 16-dim halves of a 32-dim
  // tile) on disjoint slots.  A read's byte address is a per-lane base XOR the
  // operand's field (k-step of K, dim tile of V).
  __device__ static __forceinline__ int kx(int k) { return D == 128 ? (k & 15) : ((k >> 1) & 7); }
  __device__ static __forceinline__ int vx(int k) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }
};

__device__ __forceinline__ floatx16_t mfma32(bf16x8_t a, bf16x8_t b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 * i (global_load_lds_dwordx4).  A plain device function: called
// directly in a kernel template, the builtin keeps the host compiler from
// emitting the kernel's launch stub.
__device__ __forceinline__ void load_lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds_ptr<void>(lds), 16, 0, 0);
}

// Shared-prefix mode (PART): the decode queries of a group of sequences that
// share their first blocks attend one partition of that prefix together.
// Group gi is sequences group_start[gi] .. group_start[gi+1]-1, all with the
// same first prefix_lens[group_start[gi]] tokens (whole blocks, read through
// the first sequence's table).  Work item (gi, kp, KV head g) takes rows
// (sequence s of the group, head h) r = s*G + h -- the decode queries are
// q[B][Hq][D], so sequence s of the group is "position" s -- and keys
// [kp*part_tokens, min((kp+1)*part_tokens, prefix)) with no causal mask, and
// writes the normalised fp32 partial and its base-2 log-sum-exp to slot
// slot0 + kp of each row, in the split-K workspace layout.
struct GroupArgs {
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int part_tokens;  // multiple of 32
  int parts;        // partitions per group
  int slot0;        // first workspace slot of the prefix partitions
  int num_slots;    // slots per row in the workspace
  float* o_part;    // [B][Hq][num_slots][D]
  float* lse;       // [B][Hq][num_slots]
};

template <int D, int G, bool PART = false>
__global__ void __launch_bounds__(kThreads, 1)
chunk_prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                     const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                     const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
                     const int32_t* __restrict__ query_start_loc, int Hkv, int max_blocks, int npairs,
                     float scale_log2, const GroupArgs ga) {
  using LY = Layout<D>;
  constexpr int KS = D / 16;   // QK k-steps of 16 dims over the head dimension
  constexpr int DB = D / 32;   // 32-dim output tiles
  constexpr int MERGE4 = DB * 4 + 1;  // float4s per lane of a wave's state (O, then m and l)
  static_assert(kWavesPerQ * MERGE4 * 64 * 16 <= kQuarters * LY::BUF,
                "one quarter's states fit one set of tile buffers");

  // two buffers per quarter, in two arrays (see the header)
  __shared__ __align__(16) unsigned char buf_a[kQuarters][LY::BUF];
  __shared__ __align__(16) unsigned char buf_b[kQuarters][LY::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qq = wave / kWavesPerQ, w = wave % kWavesPerQ;
  const int col = lane & 31, hg = lane >> 5;  // the lane's row in the wave's tile, its key half
  const int pair = blockIdx.x % npairs, rb = blockIdx.x / npairs;
  const int g = pair % Hkv, b = pair / Hkv;
  const int Hq = Hkv * G;

  // Chunked prefill: rows of sequence b's chunk, keys [0, kmax) under the causal
  // limits.  PART: rows of group gi, keys [kbeg, L) with L the partition's end.
  int q0, C, L, kbeg = 0, kp = 0, seq_tab = b;
  if constexpr (PART) {
    const int gi = b / ga.parts;
    kp = b % ga.parts;
    q0 = ga.group_start[gi];
    C = ga.group_start[gi + 1] - q0;  // sequences of the group
    const int pre = ga.prefix_lens[q0];
    kbeg = kp * ga.part_tokens;
    if (kbeg >= pre) return;
    L = min(kbeg + ga.part_tokens, pre);
    seq_tab = q0;
  } else {
    q0 = query_start_loc[b];
    C = query_start_loc[b + 1] - q0;
    L = context_lens[b];
  }
  const int nrows = C * G;
  const int row0 = rb * kRowsPerWG;
  if (row0 >= nrows) return;  // the whole workgroup leaves together
  const int last_row = min(nrows, row0 + kRowsPerWG) - 1;
  const int kmax = PART ? L : L - C + last_row / G + 1;  // keys any row of the workgroup sees
  const int sbase = kbeg / kStepKeys;
  const int ns = (kmax - kbeg + kStepKeys - 1) / kStepKeys;  // steps of the workgroup
  const int s_begin = sbase + qq * ns / kQuarters, s_end = sbase + (qq + 1) * ns / kQuarters;
  const int niter = (ns + kQuarters - 1) / kQuarters;  // steps of the largest quarter
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int32_t* bt_row = block_tables + (int64_t)seq_tab * max_blocks;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;

  // ---- this lane's row (the lane column of the wave's 32-row tile) ---------------
  const int roww0 = row0 + w * kRowsPerWave;
  const int myrow = roww0 + col;
  const int lim = PART ? L - 1 : L - C + (myrow < nrows ? myrow / G : 0);
  // B operand of QK: the row's query, dims 16 ks + 8 hg .. +7 per k-step (rows
  // past the chunk read its first row: finite, never written out)
  bf16x8_t qb[KS];
  {
    const int rr = myrow < nrows ? myrow : row0;
    const uint16_t* qrow = q + ((int64_t)(q0 + rr / G) * Hq + g * G + rr % G) * D + hg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16));
  }
  // Steps of this wave's quarter by what its valid rows need: plain (every key
  // visible to every row), crossing some row's limit (selects), or past every
  // row's limit (not computed).
  int plain_end = s_begin, comp_end = s_begin;
  if (roww0 < nrows) {
    const int lim_lo = PART ? L - 1 : L - C + roww0 / G;
    const int lim_hi = PART ? L - 1 : L - C + min(nrows - 1, roww0 + kRowsPerWave - 1) / G;
    plain_end = min(max((lim_lo + 1) / kStepKeys, s_begin), s_end);
    comp_end = min(max(lim_hi / kStepKeys + 1, s_begin), s_end);
  }

  // ---- direct loads: waves 0 and 1 of the quarter bring blocks 0 and 1 of each step ----
  // Instruction j covers key rows j*KPI .. j*KPI + KPI-1 of the block (1 KiB of
  // LDS); lane i fills slot i % NCH of row j*KPI + i / NCH with the chunk that
  // slot holds, chunk = slot ^ mask(row of the step).  With w*16 + row as the
  // row of the step, both masks reduce to closed forms in i and j (byte offsets
  // in the block):
  //   K  j*1024 + (kl ^ (j << 6)),      kl = (i / NCH)*ROW + (((i % NCH) ^ (i >> 4)) << 4)
  //   V  j*1024 + vl,                   vl = (i / NCH)*ROW + v0,
  //      v0 = ((i % NCH) ^ vx) << 4 with vx = 4 (i >> 4) (D = 128) or 4 ((i >> 4) & 1) (D = 64)
  //   V, rows at or past L: v0 (row 0 of the block).
  // Unsigned 32-bit offsets from the block's scalar base keep each load one
  // instruction with a scalar address.
  const uint32_t kl = (uint32_t)((lane / LY::NCH) * LY::ROW + (((lane % LY::NCH) ^ (lane >> 4)) << 4));
  const uint32_t v0 = (uint32_t)(((lane % LY::NCH) ^ (D == 128 ? 4 * (lane >> 4) : 4 * ((lane >> 4) & 1))) << 4);
  const uint32_t vl = (uint32_t)((lane / LY::NCH) * LY::ROW) + v0;
  auto entry = [&](int s) { return bt_row[min(s * 2 + min(w, 1), nblk - 1)]; };
  auto issue = [&](int s, int e, unsigned char* dst) {
    if (w >= 2) return;  // two blocks per step: waves 0 and 1 load them
    const int tok0 = s * kStepKeys + w * kBlockSize;
    const char* kb = reinterpret_cast<const char*>(k_cache + (int64_t)e * blk_stride + head_off);
    const char* vb = reinterpret_cast<const char*>(v_cache + (int64_t)e * blk_stride + head_off);
#pragma unroll
    for (int j = 0; j < LY::IPB; ++j) {
      const int d = (w * kBlockSize + j * LY::KPI) * LY::ROW;
      load_lds16(kb + ((uint32_t)j * 1024u + (kl ^ ((uint32_t)j << 6))), dst + d);
      const bool in = tok0 + j * LY::KPI + lane / LY::NCH < L;
      load_lds16(vb + (in ? (uint32_t)j * 1024u + vl : v0), dst + LY::TILE + d);
    }
  };

  floatx16_t o[DB];  // O^T[dim 32 db + 8 (r / 4) + 4 hg + r % 4][row col] in o[db][r]
  float lsum = 0.f, m_ref = -INFINITY;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  const float lazy_raw = kLazyLog2 / scale_log2;
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);

  // Per-lane byte offsets of the operand reads inside a tile.  K (A of QK): key
  // col, chunk 2 ks + hg -> key*ROW + ((hg ^ kx) << 4), then ^ (ks << 5) per
  // k-step.  V^T (A of PV, two transposing reads per operand): the lane's
  // 16-lane group q (dims 16 (q % 2) .. +15 of a 32-dim tile, key half hg)
  // reads keys 16 h + 4 hg + l16 / 4 (and + 8), dims 4 (l16 % 4) .. +3 of its
  // 16 -> chunk 2 (q % 2) + (l16 % 4) / 2 of the tile's four, then ^ (db << 6).
  // The key order this gives the PV contraction (lane half hg, element e:
  // key 4 hg + e for e < 4, 8 + 4 hg + e - 4 otherwise, + 16 h) is the order
  // in which the QK result holds the lane's keys, so P needs no exchange.
  const int l16 = lane & 15, grp = lane >> 4;
  const int k_lane = col * LY::ROW + ((hg ^ LY::kx(col)) << 4);
  const int vk = 4 * hg + (l16 >> 2);
  const int v_lane = vk * LY::ROW + (((2 * (grp & 1) + ((l16 & 3) >> 1)) ^ LY::vx(vk)) << 4) + (l16 & 1) * 8;

  // One step from buffer `cur`; `diag`: some key is past some row's limit (the
  // selects are the only code under that branch, so both kinds of step share
  // one body and the accumulators never move between registers).
  auto step = [&](bool diag, int s, const unsigned char* cur) {
    const int z = opaque_zero();  // keeps the read addresses inside the loop
    const int kt = k_lane + z;
    const int vt = v_lane + z;
    const int key0 = s * kStepKeys;

    // ---- QK: S^T (32 keys x 32 rows); lane holds row col, keys 8 (r / 4) + 4 hg + r % 4 ----
    floatx16_t st;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(cur + (kt ^ (ks << 5)));
      if (ks == 0) {
        floatx16_t zero;
#pragma unroll
        for (int r = 0; r < 16; ++r) zero[r] = 0.f;
        st = mfma32(ka, qb[ks], zero);
      } else {
        st = mfma32(ka, qb[ks], st);
      }
    }
    if (diag) {
      const int d = lim - (key0 + 4 * hg);  // key 8 i + j (+ 4 hg) is visible if 8 i + j <= d
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 8 * (r / 4) + (r % 4) <= d ? st[r] : -INFINITY;
    }
    // ---- P ----------------------------------------------------------------------
    // The lane's own maximum decides whether the row's reference must move;
    // only then is the row's maximum over its two lanes taken.
    float mt = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = maxn(mt, st[r]);
    const bool any = mt > m_ref + lazy_raw;  // false for all-masked steps
    if (__builtin_amdgcn_ballot_w64(any)) {
      mt = maxn_swap32(mt);  // the row's maximum, the same in its 2 lanes
      const bool raise = mt > m_ref + lazy_raw;
      const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mt) * scale_log2) : 1.f;
      m_ref = raise ? mt : m_ref;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float refc = m_ref == -INFINITY ? 0.f : m_ref * scale_log2;
    uint32_t pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      pk[k] = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(st[2 * k], scale_log2, -refc)),
                         __builtin_amdgcn_exp2f(fmaf(st[2 * k + 1], scale_log2, -refc)));
    float l = lsum;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[k]), ones2, l, false);
    lsum = l;

    // ---- PV: O^T (32 dims x 32 rows) per dim tile, keys in two halves of 16 ----------
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* va1 = cur + LY::TILE + h * kBlockSize * LY::ROW + (vt ^ (db << 6));
        const shortx4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<shortx4_t>(va1));
        const shortx4_t a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<shortx4_t>(va1 + 8 * LY::ROW));
        const bf16x8_t va = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(a1, a1, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(a1, a1, 2, 3)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(a2, a2, 0, 1)),
                                 __builtin_bit_cast(uint32_t, __builtin_shufflevector(a2, a2, 2, 3))));
        o[db] = mfma32(va, pb, o[db]);
      }
    }
  };

  // The quarter's steps in rotated order: workgroup rb starts at step rb mod n
  // of its range.  The 32-odd workgroups of one (sequence, KV head) read the
  // same K/V; in lockstep every step's lines would miss in L2 for all of them
  // at once, while rotated, a line is fetched once and the others find it in
  // L2.  (The online softmax does not depend on the order of the keys.)
  const int nq = s_end - s_begin;
  const int rot = nq > 0 ? rb % nq : 0;
  auto step_of = [&](int i) {
    const int k = i + rot;
    return s_begin + (k >= nq ? k - nq : k);
  };
  // One step of the loop: load the next step into `nxt`, compute this one from
  // `cur` (the two arrays alternate, each known at compile time).
  int e_next = nq > 1 ? entry(step_of(1)) : 0;
  auto iteration = [&](int i, unsigned char* cur, unsigned char* nxt) {
    if (i + 1 < nq) issue(step_of(i + 1), e_next, nxt);
    if (i + 2 < nq) e_next = entry(step_of(i + 2));
    if (i < nq) {
      const int s = step_of(i);
      if (s < comp_end) step(s >= plain_end, s, cur);
    }
  };

  if (nq > 0) issue(step_of(0), entry(step_of(0)), buf_a[qq]);
  __syncthreads();
  for (int i = 0; i < niter; i += 2) {
    iteration(i, buf_a[qq], buf_b[qq]);
    __syncthreads();
    if (i + 1 < niter) {
      iteration(i + 1, buf_b[qq], buf_a[qq]);
      __syncthreads();
    }
  }

  // ---- row sums over the 2 lanes of each row, then merge the quarters -------------
  lsum += swap32(lsum);
  // a wave's state in merge slot `slot` (0 .. kWavesPerQ-1 in buf_a, the next
  // kWavesPerQ in buf_b): [k][64 lanes] of float4
  auto at = [&](int slot, int k) -> float4& {
    float4* mg = reinterpret_cast<float4*>(slot < kWavesPerQ ? &buf_a[0][0] : &buf_b[0][0]);
    return mg[((slot % kWavesPerQ) * MERGE4 + k) * 64 + lane];
  };
  auto put = [&](int slot) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        at(slot, db * 4 + i) = make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
    at(slot, DB * 4) = make_float4(m_ref, lsum, 0.f, 0.f);
  };
  auto take = [&](int slot) {
    const float4 ml = at(slot, DB * 4);
    const float m1 = ml.x, l1 = ml.y;
    const float m0 = m_ref;
    const float M = fmaxf(m0, m1);
    const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - M) * scale_log2);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * scale_log2);
    m_ref = M;
    lsum = w0 * lsum + w1 * l1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = at(slot, db * 4 + i);
        o[db][4 * i] = w0 * o[db][4 * i] + w1 * v.x;
        o[db][4 * i + 1] = w0 * o[db][4 * i + 1] + w1 * v.y;
        o[db][4 * i + 2] = w0 * o[db][4 * i + 2] + w1 * v.z;
        o[db][4 * i + 3] = w0 * o[db][4 * i + 3] + w1 * v.w;
      }
  };
  // round 1: quarters 2, 3 hand over to quarters 0, 1; round 2: quarter 1 to quarter 0
  if (qq >= 2) put((qq - 2) * kWavesPerQ + w);
  __syncthreads();
  if (qq < 2) take(qq * kWavesPerQ + w);
  __syncthreads();
  if (qq == 1) put(w);
  __syncthreads();
  if (qq != 0) return;
  take(w);

  // ---- normalise and write ------------------------------------------------------------
  if (myrow >= nrows) return;
  if constexpr (PART) {
    // partial of row (sequence q0 + pos, head g*G + h) at slot slot0 + kp
    const int pos = myrow / G, h = myrow % G;
    const float inv = 1.f / lsum;
    const int64_t slot = ((int64_t)(q0 + pos) * Hq + g * G + h) * ga.num_slots + ga.slot0 + kp;
    float* orow = ga.o_part + slot * D + 4 * hg;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(orow + db * 32 + 8 * i) =
            make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
    if (hg == 0) ga.lse[slot] = m_ref * scale_log2 + log2f(lsum);
  } else {
    const int pos = myrow / G, h = myrow % G;
    const float inv = 1.f / lsum;
    uint16_t* orow = out + ((int64_t)(q0 + pos) * Hq + g * G + h) * D + 4 * hg;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y0 = o[db][4 * i] * inv, y1 = o[db][4 * i + 1] * inv;
        const float y2 = o[db][4 * i + 2] * inv, y3 = o[db][4 * i + 3] * inv;
        *reinterpret_cast<uint2*>(orow + db * 32 + 8 * i) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
      }
  }
}

template <int D, bool PART = false>
hipError_t launch_chunk_d(int G, dim3 grid, hipStream_t stream, uint16_t* out, const uint16_t* q,
                          const uint16_t* kc, const uint16_t* vc, const int32_t* bt, const int32_t* cl,
                          const int32_t* qsl, int Hkv, int mb, int npairs, float sl,
                          const GroupArgs& ga = GroupArgs{}) {
#define PA_CHUNK(GG)                                                                                     \
  hipLaunchKernelGGL((chunk_prefill_kernel<D, GG, PART>), grid, dim3(kThreads), 0, stream, out, q, kc, vc, \
                     bt, cl, qsl, Hkv, mb, npairs, sl, ga)
  switch (G) {
    case 1: PA_CHUNK(1); break;
    case 2: PA_CHUNK(2); break;
    case 3: PA_CHUNK(3); break;
    case 4: PA_CHUNK(4); break;
    case 5: PA_CHUNK(5); break;
    case 6: PA_CHUNK(6); break;
    case 7: PA_CHUNK(7); break;
    case 8: PA_CHUNK(8); break;
    default: return hipErrorInvalidValue;
  }
#undef PA_CHUNK
  return hipGetLastError();
}

}  // namespace

int64_t prefill_workgroups(int B, int Hq, int Hkv, int max_query_len) {
  const int64_t rows = (int64_t)max_query_len * (Hq / Hkv);
  return (rows + kRowsPerWG - 1) / kRowsPerWG * Hkv * B;
}

hipError_t launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int B, int Hq, int Hkv, int D,
                          int max_blocks, int max_query_len, float scale, hipStream_t stream) {
  const int G = Hq / Hkv;
  const dim3 grid((unsigned)prefill_workgroups(B, Hq, Hkv, max_query_len));
  const float sl = scale * 1.4426950408889634f;
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kc = static_cast<const uint16_t*>(k_cache);
  auto* vc = static_cast<const uint16_t*>(v_cache);
  if (D == 128)
    return launch_chunk_d<128>(G, grid, stream, o, qq, kc, vc, block_tables, context_lens,
                               query_start_loc, Hkv, max_blocks, Hkv * B, sl);
  return launch_chunk_d<64>(G, grid, stream, o, qq, kc, vc, block_tables, context_lens,
                            query_start_loc, Hkv, max_blocks, Hkv * B, sl);
}

int64_t group_prefix_row_blocks(int max_group_size, int G) {
  return ((int64_t)max_group_size * G + kRowsPerWG - 1) / kRowsPerWG;
}

// Shared-prefix partials of decode queries on the chunked-prefill kernel: work
// items (groups * parts * Hkv) x row blocks.
hipError_t launch_group_prefix(float* o_part, float* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* group_start, const int32_t* prefix_lens, int groups,
                               int max_group_size, int max_prefix, int part_tokens, int slot0,
                               int num_slots, int Hq, int Hkv, int D, int max_blocks, float scale,
                               hipStream_t stream) {
  const int G = Hq / Hkv;
  if (part_tokens <= 0 || part_tokens % kStepKeys != 0) return hipErrorInvalidValue;
  const int parts = (max_prefix + part_tokens - 1) / part_tokens;
  const int64_t rblocks = group_prefix_row_blocks(max_group_size, G);
  const int64_t npairs = (int64_t)groups * parts * Hkv;
  if (groups <= 0 || parts <= 0 || rblocks <= 0) return hipSuccess;
  if (npairs * rblocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(npairs * rblocks));
  const GroupArgs ga{group_start, prefix_lens, part_tokens, parts, slot0, num_slots, o_part, lse};
  const float sl = scale * 1.4426950408889634f;
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kc = static_cast<const uint16_t*>(k_cache);
  auto* vc = static_cast<const uint16_t*>(v_cache);
  if (D == 128)
    return launch_chunk_d<128, true>(G, grid, stream, nullptr, qq, kc, vc, block_tables, nullptr,
                                     nullptr, Hkv, max_blocks, (int)npairs, sl, ga);
  return launch_chunk_d<64, true>(G, grid, stream, nullptr, qq, kc, vc, block_tables, nullptr, nullptr,
                                  Hkv, max_blocks, (int)npairs, sl, ga);
}

}  // namespace pa
