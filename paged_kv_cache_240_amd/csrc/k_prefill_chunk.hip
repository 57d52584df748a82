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
// and each wave owns 32 rows (two 16-row tiles) over its quarter's keys.
// 96-row workgroups make one workgroup per compute unit on the chunked-prefill
// shape (32 per (sequence, KV head), 8 pairs); 32 rows per wave keep a wave
// within 170 registers, so three waves share each SIMD and cover each other's
// latency, and every K/V operand read from LDS feeds two matrix products.
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
//   QK    S^T (keys x rows) = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 keys
//         x 32 dims of K from LDS, B = 32 dims x 16 rows of the queries, held
//         in registers.  A lane ends with 4 consecutive keys of one row.
//   P     the row's running reference max is raised only when a step's max
//         exceeds it by more than 2^8 (p then stays below 256: exact enough in
//         bf16, safe in fp32 sums), which spares nearly every rescale; causal
//         limits are selects, on steps that cross a row's limit only; p is
//         rounded to bf16 and the S^T layout is already the B operand of PV.
//         The row sum accumulates the same rounded p with v_dot2_f32_bf16.
//   PV    O^T (dims x rows) += V^T P^T: A = 16 dims x 32 keys of V^T, read from
//         the key-major V tile with the transposing ds_read_b64_tr_b16 (two
//         reads of 4 keys x 16 dims per operand).
// The quarters meet through LDS at the end (log-sum-exp merge, in two rounds
// that fit the freed tile buffers).  Workgroup ids are mapped (sequence, KV
// head)-minor, so consecutive ids -- placed on different XCDs -- take different
// pairs and each XCD's L2 serves the K/V of few pairs.

#include "pa_device.h"
#include "pa_internal.h"



namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kQuarters = 4;                       // key ranges per workgroup
constexpr int kWavesPerQ = 3;                      // waves sharing a key range
constexpr int kWaves = kQuarters * kWavesPerQ;     // 12
constexpr int kThreads = 64 * kWaves;              // 768
constexpr int kRowTiles = 2;                       // 16-row tiles per wave
constexpr int kRowsPerWave = 16 * kRowTiles;       // 32
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
  // XOR swizzles of the 16-byte chunks of a key row, chosen so that each LDS
  // read below touches distinct banks: in the K tile, chunk c of key k sits in
  // slot c ^ kx(k); in the V tile, in slot c ^ vx(k).  Both masks leave the
  // chunk bits that select the operand (k-step of K, dim tile of V) in a field
  // of their own, so a read's byte address is a per-lane base XOR that field.
  __device__ static __forceinline__ int kx(int k) { return D == 128 ? (k & 15) : ((k >> 1) & 7); }
  __device__ static __forceinline__ int vx(int k) { return D == 128 ? 2 * (k & 7) : 2 * ((k >> 1) & 3); }
};

__device__ __forceinline__ floatx4_t mfma16(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 1)
chunk_prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                     const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                     const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
                     const int32_t* __restrict__ query_start_loc, int Hkv, int max_blocks, int npairs,
                     float scale_log2) {
  using LY = Layout<D>;
  constexpr int KS = D / 32;   // QK k-steps over the head dimension
  constexpr int DT = D / 16;   // 16-dim output tiles
  constexpr int MERGE = DT * kRowTiles * 4 + 2 * kRowTiles;  // floats per lane of a wave's state
  static_assert(kWavesPerQ * MERGE * 64 * 4 <= kQuarters * LY::BUF,
                "one quarter's states fit one set of tile buffers");

  // two buffers per quarter, in two arrays (see the header)
  __shared__ __align__(16) unsigned char buf_a[kQuarters][LY::BUF];
  __shared__ __align__(16) unsigned char buf_b[kQuarters][LY::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qq = wave / kWavesPerQ, w = wave % kWavesPerQ;
  const int col = lane & 15, quad = lane >> 4;
  const int pair = blockIdx.x % npairs, rb = blockIdx.x / npairs;
  const int g = pair % Hkv, b = pair / Hkv;
  const int Hq = Hkv * G;

  const int q0 = query_start_loc[b];
  const int C = query_start_loc[b + 1] - q0;
  const int L = context_lens[b];
  const int nrows = C * G;
  const int row0 = rb * kRowsPerWG;
  if (row0 >= nrows) return;  // the whole workgroup leaves together
  const int last_row = min(nrows, row0 + kRowsPerWG) - 1;
  const int kmax = L - C + last_row / G + 1;          // keys any row of the workgroup sees
  const int ns = (kmax + kStepKeys - 1) / kStepKeys;  // steps of the workgroup
  const int s_begin = qq * ns / kQuarters, s_end = (qq + 1) * ns / kQuarters;
  const int niter = (ns + kQuarters - 1) / kQuarters;  // steps of the largest quarter
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;

  // ---- this lane's rows (one per 16-row tile: the lane column) -----------------
  const int roww0 = row0 + w * kRowsPerWave;
  int lim[kRowTiles];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = roww0 + rt * 16 + col;
    lim[rt] = L - C + (r < nrows ? r / G : 0);
  }
  // B operands of QK: the wave's 32 query rows, 8 dims per k-step (rows past the
  // chunk read its first row: finite, never written out)
  bf16x8_t qb[kRowTiles][KS];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = roww0 + rt * 16 + col;
    const int rr = r < nrows ? r : row0;
    const uint16_t* qrow = q + ((int64_t)(q0 + rr / G) * Hq + g * G + rr % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[rt][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 32 + quad * 8));
  }
  // Steps of this wave's quarter by what its valid rows need: plain (every key
  // visible to every row), crossing some row's limit (selects), or past every
  // row's limit (not computed).
  int plain_end = s_begin, comp_end = s_begin;
  if (roww0 < nrows) {
    const int lim_lo = L - C + roww0 / G;
    const int lim_hi = L - C + min(nrows - 1, roww0 + kRowsPerWave - 1) / G;
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
  //   V  j*1024 + (vl ^ vj),            vl = (i / NCH)*ROW + v0, v0 = ((i % NCH) ^ 2(i >> 4)) << 4
  //   V, rows at or past L: v0 ^ vj (row 0 of the block), vj = D == 128 ? (j & 1) << 7 : 0.
  // Unsigned 32-bit offsets from the block's scalar base keep each load one
  // instruction with a scalar address.
  const uint32_t kl = (uint32_t)((lane / LY::NCH) * LY::ROW + (((lane % LY::NCH) ^ (lane >> 4)) << 4));
  const uint32_t v0 = (uint32_t)(((lane % LY::NCH) ^ (2 * (lane >> 4))) << 4);
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
      const uint32_t vj = D == 128 ? (uint32_t)(j & 1) << 7 : 0u;
      load_lds16(kb + ((uint32_t)j * 1024u + (kl ^ ((uint32_t)j << 6))), dst + d);
      const bool in = tok0 + j * LY::KPI + lane / LY::NCH < L;
      load_lds16(vb + (in ? (uint32_t)j * 1024u + (vl ^ vj) : (v0 ^ vj)), dst + LY::TILE + d);
    }
  };

  floatx4_t o[DT][kRowTiles];
  float lsum[kRowTiles], m_ref[kRowTiles];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    lsum[rt] = 0.f;
    m_ref[rt] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float lazy_raw = kLazyLog2 / scale_log2;
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);

  // Per-lane byte offsets of the operand reads inside a tile.  K (A of QK): key
  // t*16 + col, chunk ks*4 + quad -> (key*ROW + ((quad ^ kx) bits)) ^ (ks << 6),
  // the ks field of the chunk being bits 6.. of the offset.  V^T (A of PV, two
  // transposing reads): lane (l16, quad) reads key 4*quad + l16/4 (+16), dims
  // 16*dt + 4*(l16 % 4) .. +3 -> (key*ROW + ...) ^ (dt << 5).
  const int l16 = lane & 15;
  const int vk = quad * 4 + (l16 >> 2);
  const int k_lane = col * LY::ROW + (((quad ^ LY::kx(col)) & 3) << 4) + ((LY::kx(col) >> 2) << 6);
  const int v_lane = vk * LY::ROW + ((((l16 & 3) >> 1) ^ (LY::vx(vk) & 1)) << 4) +
                     ((LY::vx(vk) >> 1) << 5) + (l16 & 1) * 8;

  // One step from buffer `cur`; `diag`: some key is past some row's limit (the
  // selects are the only code under that branch, so both kinds of step share
  // one body and the accumulators never move between registers).
  auto step = [&](bool diag, int s, const unsigned char* cur) {
    const int z = opaque_zero();  // keeps the read addresses inside the loop
    const unsigned char* kt = cur + (k_lane + z);
    const unsigned char* vt = cur + LY::TILE + (v_lane + z);
    const int key0 = s * kStepKeys;

    // ---- QK ---------------------------------------------------------------------
    floatx4_t st[2][kRowTiles];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t ka[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        ka[t] = *reinterpret_cast<const bf16x8_t*>(cur + ((kt - cur) ^ (ks << 6)) + t * kBlockSize * LY::ROW);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
          st[t][rt] = mfma16(ka[t], qb[rt][ks], ks == 0 ? floatx4_t{0.f, 0.f, 0.f, 0.f} : st[t][rt]);
    }
    if (diag) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
          const int d = lim[rt] - (key0 + t * 16 + quad * 4);  // keys j <= d are visible
#pragma unroll
          for (int j = 0; j < 4; ++j) st[t][rt][j] = j <= d ? st[t][rt][j] : -INFINITY;
        }
    }
    // ---- P ----------------------------------------------------------------------
    // The lane's own maximum per row decides whether any reference must move;
    // only then is the row's maximum over its 4 lanes taken (almost never after
    // the first step: later keys seldom exceed the reference by 2^8).
    float mt[kRowTiles];
    bool any = false;
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      mt[rt] = maxn(maxn(maxn(st[0][rt][0], st[0][rt][1]), maxn(st[0][rt][2], st[0][rt][3])),
                    maxn(maxn(st[1][rt][0], st[1][rt][1]), maxn(st[1][rt][2], st[1][rt][3])));
      any = any || mt[rt] > m_ref[rt] + lazy_raw;  // false for all-masked steps
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        mt[rt] = maxn_swap32(maxn_swap16(mt[rt]));  // the row's maximum, the same in its 4 lanes
        const bool raise = mt[rt] > m_ref[rt] + lazy_raw;
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref[rt] - mt[rt]) * scale_log2) : 1.f;
        m_ref[rt] = raise ? mt[rt] : m_ref[rt];
        lsum[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
      }
    }
    bf16x8_t pb[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      const float refc = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt] * scale_log2;
      uint32_t pk[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const floatx4_t& sv = st[t][rt];
        pk[2 * t] = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[0], scale_log2, -refc)),
                               __builtin_amdgcn_exp2f(fmaf(sv[1], scale_log2, -refc)));
        pk[2 * t + 1] = cvt_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[2], scale_log2, -refc)),
                                   __builtin_amdgcn_exp2f(fmaf(sv[3], scale_log2, -refc)));
      }
      float l = lsum[rt];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[k]), ones2, l, false);
      lsum[rt] = l;
      pb[rt] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }

    // ---- PV ---------------------------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const unsigned char* va1 = cur + LY::TILE + ((vt - cur - LY::TILE) ^ (dt << 5));
      const shortx4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<shortx4_t>(va1));
      const shortx4_t a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          lds_ptr<shortx4_t>(va1 + kBlockSize * LY::ROW));
      const bf16x8_t va = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_shufflevector(a1, a1, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(a1, a1, 2, 3)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(a2, a2, 0, 1)),
                               __builtin_bit_cast(uint32_t, __builtin_shufflevector(a2, a2, 2, 3))));
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) o[dt][rt] = mfma16(va, pb[rt], o[dt][rt]);
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

  // ---- row sums over the 4 lanes of each row, then merge the quarters -------------
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    float l = lsum[rt];
    l += swap16(l);
    lsum[rt] = l + swap32(l);
  }
  // a wave's state in merge slot `slot` (0 .. kWavesPerQ-1 in buf_a, the next kWavesPerQ in buf_b): [k][64 lanes]
  auto at = [&](int slot, int k) -> float& {
    float* mg = reinterpret_cast<float*>(slot < kWavesPerQ ? &buf_a[0][0] : &buf_b[0][0]);
    return mg[((slot % kWavesPerQ) * MERGE + k) * 64 + lane];
  };
  auto put = [&](int slot) {
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) at(slot, (rt * DT + dt) * 4 + j) = o[dt][rt][j];
      at(slot, DT * kRowTiles * 4 + rt) = m_ref[rt];
      at(slot, DT * kRowTiles * 4 + kRowTiles + rt) = lsum[rt];
    }
  };
  auto take = [&](int slot) {
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      const float m1 = at(slot, DT * kRowTiles * 4 + rt);
      const float l1 = at(slot, DT * kRowTiles * 4 + kRowTiles + rt);
      const float m0 = m_ref[rt];
      const float M = fmaxf(m0, m1);
      const float w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m0 - M) * scale_log2);
      const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - M) * scale_log2);
      m_ref[rt] = M;
      lsum[rt] = w0 * lsum[rt] + w1 * l1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[dt][rt][j] = w0 * o[dt][rt][j] + w1 * at(slot, (rt * DT + dt) * 4 + j);
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
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = roww0 + rt * 16 + col;
    if (r >= nrows) continue;
    const int pos = r / G, h = r % G;
    const float inv = 1.f / lsum[rt];
    uint16_t* orow = out + ((int64_t)(q0 + pos) * Hq + g * G + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const floatx4_t y = o[dt][rt] * inv;
      *reinterpret_cast<uint2*>(orow + dt * 16 + quad * 4) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    }
  }
}

template <int D>
hipError_t launch_chunk_d(int G, dim3 grid, hipStream_t stream, uint16_t* out, const uint16_t* q,
                          const uint16_t* kc, const uint16_t* vc, const int32_t* bt, const int32_t* cl,
                          const int32_t* qsl, int Hkv, int mb, int npairs, float sl) {
#define PA_CHUNK(GG)                                                                              \
  hipLaunchKernelGGL((chunk_prefill_kernel<D, GG>), grid, dim3(kThreads), 0, stream, out, q, kc, vc, \
                     bt, cl, qsl, Hkv, mb, npairs, sl)
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

}  // namespace pa
