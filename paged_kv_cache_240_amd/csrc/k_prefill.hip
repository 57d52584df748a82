// Causal paged chunked prefill for gfx950 on bf16 matrix cores.
//
// Operation (Pico-vLLM write-up, §2: paged prefill kernel in the manner of
// Flash Attention, using the matrix cores; mini-llm-engine post, §3.3: a
// prompt is prefilled in chunks, each chunk attending the cached prefix plus
// itself; §3.1: K/V in 16-token physical blocks behind a block table):
// chunk row i of sequence b sits at position L_b - C_b + i and attends keys
// t <= L_b - C_b + i with softmax(scale * q K^T) V, GQA head h -> KV head h/G.
//
// Rows are (position, head) pairs of one (sequence, KV head), position-major
// (r = pos * G + h), so the G query heads sharing a KV head share every K/V
// tile.  Workgroup = 4 waves over 128 rows; a wave owns 2 row tiles of 16.
// Keys are walked in tiles of 32 (two 16-token blocks), double-buffered in
// LDS, the next tile's global loads in flight while the current one computes.
//   QK   S^T (keys x rows) = K Q^T with v_mfma_f32_16x16x32_bf16: A = K tile
//        from LDS (16-byte chunks XOR-swizzled by key so the 16 rows of an
//        operand read hit distinct banks), B = the rows' queries (registers).
//   P    online softmax per row (the row is a lane column: 8 scores per lane,
//        max/sum across the 4 lanes sharing it by row swaps); rows' causal
//        limits are applied by selects on tiles crossing the diagonal.  p is
//        rounded to bf16; the S^T accumulator layout is already the B operand
//        of the PV product, so p never moves.
//   PV   O^T (dims x rows) += V^T P^T: A = V^T from LDS, where V is stored
//        transposed with the key order the P operand implies (8 keys of a
//        lane contiguous) and an 80-byte row stride (conflict-free reads).
// Keys at or past L are written to LDS as zeros (never multiplied by 0: NaN
// in unused slots cannot leak) and their table entries are never read.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRowTiles = 2;                    // 16-row tiles per wave
constexpr int kRowsPerWave = 16 * kRowTiles;    // 32
constexpr int kRowsPerWG = kWaves * kRowsPerWave;  // 128
constexpr int kKeyTile = 32;                    // keys per step (two blocks)
constexpr int kVtStride = 40;                   // bf16 per V^T row: 32 keys + 8 pad (80 bytes)

// LDS position of key k (0..31) in a V^T row: lane group q reads its 8 keys
// 4q..4q+3 and 16+4q..16+4q+3 (the keys its S^T registers hold) contiguously.
__device__ __forceinline__ int vt_pos(int k) {
  return k < 16 ? 8 * (k >> 2) + (k & 3) : 8 * ((k - 16) >> 2) + 4 + (k & 3);
}

template <int D, int G>
__global__ void __launch_bounds__(256)
prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
               const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
               const int32_t* __restrict__ query_start_loc, int Hkv, int max_blocks,
               float scale_log2) {
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int KS = D / 32;         // MFMA k-steps over the head dimension
  constexpr int DT = D / 16;         // 16-dim output tiles
  constexpr int TILE_CHUNKS = 2 * kBlockSize * NCH;  // 16-byte chunks of a K (or V) tile
  constexpr int LOADS = TILE_CHUNKS / 256;           // per thread, per operand
  static_assert(TILE_CHUNKS % 256 == 0, "tile chunks must spread evenly over the workgroup");
  constexpr int KS_BYTES = kKeyTile * D * 2;
  constexpr int VT_BYTES = D * kVtStride * 2;

  __shared__ __align__(16) unsigned char lds[2][KS_BYTES + VT_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int rb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;

  const int q0 = query_start_loc[b];
  const int C = query_start_loc[b + 1] - q0;
  const int L = context_lens[b];
  const int nrows = C * G;
  const int row0_wg = rb * kRowsPerWG;
  if (row0_wg >= nrows) return;
  const int pos_last = min(nrows, row0_wg + kRowsPerWG) - 1;  // last valid row of the WG
  // keys any row of this workgroup can see: up to position L - C + pos_max
  const int kmax = min(L, L - C + pos_last / G + 1);
  const int ntiles = (kmax + kKeyTile - 1) / kKeyTile;
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;
  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;

  // ---- this lane's rows: one per row tile (lane column) ----------------------
  int lim[kRowTiles];  // last visible key of the row
  bool rvalid[kRowTiles];
  bf16x8_t qb[kRowTiles][KS];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = row0_wg + wave * kRowsPerWave + rt * 16 + col;
    rvalid[rt] = r < nrows;
    const int pos = rvalid[rt] ? r / G : 0;
    const int h = rvalid[rt] ? r % G : 0;
    lim[rt] = rvalid[rt] ? L - C + pos : L - 1;
    const uint16_t* qrow = q + ((int64_t)(q0 + pos) * Hq + g * G + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 t = *reinterpret_cast<const uint4*>(qrow + ks * 32 + quad * 8);
      if (!rvalid[rt]) t = make_uint4(0u, 0u, 0u, 0u);
      qb[rt][ks] = __builtin_bit_cast(bf16x8_t, t);
    }
  }
  int lim_min = lim[0];
#pragma unroll
  for (int rt = 1; rt < kRowTiles; ++rt) lim_min = min(lim_min, lim[rt]);
  // smallest causal limit over the workgroup's rows (tiles past it need masks)
  const int lim_min_wg = L - C + row0_wg / G;

  // ---- staging: global -> registers -> LDS ------------------------------------
  uint4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int tt) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      // K: chunk c covers block c / (16 NCH), key row, 16-byte chunk (coalesced rows)
      const int c = tid + 256 * i;
      const int blk = c / (kBlockSize * NCH);
      const int key = (c / NCH) % kBlockSize;
      const int ch = c % NCH;
      const int lb = tt * 2 + blk;
      const int t = lb * kBlockSize + key;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u);
      if (lb < nblk_seq && t < L)
        kv = *reinterpret_cast<const uint4*>(k_cache + (int64_t)bt_row[lb] * blk_stride +
                                             head_off + key * D + ch * 8);
      kreg[i] = kv;
      // V: chunk c covers key c % 32 and dims 8*(c / 32) .. +7
      const int vkey = c % kKeyTile;
      const int vch = c / kKeyTile;
      const int vlb = tt * 2 + vkey / kBlockSize;
      const int vt = vlb * kBlockSize + vkey % kBlockSize;
      uint4 vv = make_uint4(0u, 0u, 0u, 0u);
      if (vlb < nblk_seq && vt < L)
        vv = *reinterpret_cast<const uint4*>(v_cache + (int64_t)bt_row[vlb] * blk_stride +
                                             head_off + (vkey % kBlockSize) * D + vch * 8);
      vreg[i] = vv;
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* ks_base = lds[buf];
    uint16_t* vt_base = reinterpret_cast<uint16_t*>(lds[buf] + KS_BYTES);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int key = (c / NCH) % kBlockSize + kBlockSize * (c / (kBlockSize * NCH));
      const int ch = c % NCH;
      *reinterpret_cast<uint4*>(ks_base + key * D * 2 + ((ch ^ (key & (NCH - 1))) * 16)) = kreg[i];
      const int vkey = c % kKeyTile;
      const int d0 = 8 * (c / kKeyTile);
      uint16_t* dst = vt_base + d0 * kVtStride + vt_pos(vkey);
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[(2 * e) * kVtStride] = (uint16_t)(w[e] & 0xFFFFu);
        dst[(2 * e + 1) * kVtStride] = (uint16_t)(w[e] >> 16);
      }
    }
  };

  floatx4_t o[DT][kRowTiles];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) o[dt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[kRowTiles], l_part[kRowTiles];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    m_run[rt] = -INFINITY;
    l_part[rt] = 0.f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int tt = 0; tt < ntiles; ++tt) {
    const int buf = tt & 1;
    if (tt + 1 < ntiles) load_tile(tt + 1);
    const unsigned char* ks_base = lds[buf];
    const uint16_t* vt_base = reinterpret_cast<const uint16_t*>(lds[buf] + KS_BYTES);
    const int key0 = tt * kKeyTile;

    // ---- QK: S^T for 2 key tiles x 2 row tiles ----------------------------------
    floatx4_t st[2][kRowTiles];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) st[kt][rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      const int key = kt * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 4 + quad;
        const uint4 a = *reinterpret_cast<const uint4*>(ks_base + key * D * 2 +
                                                        ((ch ^ (key & (NCH - 1))) * 16));
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
          st[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[rt][ks], st[kt][rt], 0, 0, 0);
      }
    }

    // ---- P: online softmax per row ----------------------------------------------
    const bool need_mask = key0 + kKeyTile - 1 > lim_min_wg;
    bf16x8_t pb[kRowTiles];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      float s[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = st[kt][rt][j] * scale_log2;
          const int t = key0 + kt * 16 + quad * 4 + j;
          s[kt * 4 + j] = (!need_mask || t <= lim[rt]) ? x : -INFINITY;
        }
      float mt = s[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, s[e]);
      mt = fmaxf(mt, swap16(mt));
      mt = fmaxf(mt, swap32(mt));
      const float m_new = fmaxf(m_run[rt], mt);
      const float ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run[rt] - ref);
      m_run[rt] = m_new;
      uint32_t pk[4];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pk[e] = pack_bf16x2(exp2f(s[2 * e] - ref), exp2f(s[2 * e + 1] - ref));
        ps += bf16lo(pk[e]) + bf16hi(pk[e]);  // the normaliser sums what PV applies
      }
      l_part[rt] = l_part[rt] * alpha + ps;
      pb[rt] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
    }

    // ---- PV: O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint4 a = *reinterpret_cast<const uint4*>(vt_base + (dt * 16 + col) * kVtStride + quad * 8);
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt)
        o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[rt], o[dt][rt], 0, 0, 0);
    }

    if (tt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write: lane holds O^T[dims 4*quad+j of tile dt][row col] ---------
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    float l = l_part[rt];
    l += swap16(l);
    l += swap32(l);
    if (!rvalid[rt]) continue;
    const float inv = 1.f / l;
    const int r = row0_wg + wave * kRowsPerWave + rt * 16 + col;
    const int pos = r / G, h = r % G;
    uint16_t* orow = out + ((int64_t)(q0 + pos) * Hq + g * G + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<uint2*>(orow + dt * 16 + quad * 4) =
          make_uint2(pack_bf16x2(o[dt][rt][0] * inv, o[dt][rt][1] * inv),
                     pack_bf16x2(o[dt][rt][2] * inv, o[dt][rt][3] * inv));
  }
  (void)lim_min;
}

template <int D>
hipError_t launch_d(int G, dim3 grid, hipStream_t stream, uint16_t* out, const uint16_t* q,
                    const uint16_t* kc, const uint16_t* vc, const int32_t* bt, const int32_t* cl,
                    const int32_t* qsl, int Hkv, int mb, float sl) {
#define PA_PREFILL(GG)                                                                        \
  hipLaunchKernelGGL((prefill_kernel<D, GG>), grid, dim3(256), 0, stream, out, q, kc, vc, bt,  \
                     cl, qsl, Hkv, mb, sl)
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

hipError_t launch_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, int B, int Hq, int Hkv, int D,
                          int max_blocks, int max_query_len, float scale, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int rblocks = (max_query_len * G + kRowsPerWG - 1) / kRowsPerWG;
  const dim3 grid(rblocks, Hkv, B);
  const float sl = scale * 1.4426950408889634f;
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kc = static_cast<const uint16_t*>(k_cache);
  auto* vc = static_cast<const uint16_t*>(v_cache);
  if (D == 128)
    return launch_d<128>(G, grid, stream, o, qq, kc, vc, block_tables, context_lens,
                         query_start_loc, Hkv, max_blocks, sl);
  return launch_d<64>(G, grid, stream, o, qq, kc, vc, block_tables, context_lens, query_start_loc,
                      Hkv, max_blocks, sl);
}

}  // namespace pa
