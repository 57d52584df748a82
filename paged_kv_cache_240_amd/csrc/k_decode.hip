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
// Workgroup = 4 waves.  A partition (split-K) or the whole sequence (single
// pass) is walked in chunks of up to 32 blocks (512 tokens); per chunk:
//   QK   each wave takes every 4th block.  Lane (t = lane/4, quarter) holds
//        a quarter of key row t (4 x 16-byte loads, 64 contiguous bytes per
//        row per load) and the matching quarter of the G query rows, takes
//        bf16 dot products with v_dot2_f32_bf16 and sums the 4 quarters with
//        two DPP quad adds.  Scores (times scale*log2 e) go to LDS; rows past
//        the sequence end are set to -inf by a select.
//   P    one wave per head: chunk max, running max, p = 2^(s - m) written back
//        in place, running sum; the rescale factor of earlier chunks to LDS.
//   PV   lane (token group, 8 dims) loads 16-byte pieces of V rows (1 KB
//        contiguous per wave load), reads its p values from LDS with one
//        vector read per head and accumulates in fp32.  Rows past the end are
//        zeroed by a select, so NaN in unused slots never reaches a sum.
// After the last chunk the token groups and the 4 waves are summed and the
// normalised output is written as bf16 (single pass) or as an fp32 partial
// plus its base-2 log-sum-exp (split-K).  A separate kernel combines the
// partials of a sequence (Flash Decode's reduce).
//
// Block-table entries are read with wave-uniform addresses (scalar loads);
// entries past the sequence's last block are never read.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kChunkBlocks = 32;
constexpr int kChunkTokens = kChunkBlocks * kBlockSize;

template <int D, int G, bool SPLIT>
__global__ void __launch_bounds__(256)
decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
              const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
              const int32_t* __restrict__ context_lens, int Hkv, int max_blocks,
              float scale_log2, int part_tokens, int num_parts, uint16_t* __restrict__ out,
              float* __restrict__ o_part, float* __restrict__ lse) {
  constexpr int NCH = D / 8;    // 16-byte chunks in a row
  constexpr int CPL = NCH / 4;  // chunks per lane in the QK layout
  constexpr int TG = 64 / NCH;  // token groups in the PV layout
  constexpr int IPB = 16 / TG;  // tokens per lane per block in the PV layout
  static_assert(G * kChunkTokens >= kWaves * G * D, "reduction buffer aliases the score buffer");

  __shared__ __align__(16) float s_buf[G * kChunkTokens];
  __shared__ float st_m[G], st_l[G], st_a[G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int hq0 = g * G;
  const int L = context_lens[b];

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

  // QK layout
  const int tq = lane >> 2, qd = lane & 3;
  // PV layout
  const int tg = lane / NCH, dc = lane % NCH;

  uint4 qr[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci)
      qr[h][ci] = *reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + hq0 + h) * D +
                                                  (qd + 4 * ci) * 8);

  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  if (threadIdx.x < G) {
    st_m[threadIdx.x] = -INFINITY;
    st_l[threadIdx.x] = 0.f;
  }
  __syncthreads();

  const int32_t* bt_row = block_tables + (int64_t)b * max_blocks;
  const int64_t head_off = (int64_t)g * kBlockSize * D;
  const int64_t blk_stride = (int64_t)Hkv * kBlockSize * D;

  for (int c0 = t_begin; c0 < t_end; c0 += kChunkTokens) {
    const int nt = min(kChunkTokens, t_end - c0);
    const int nblk = (nt + kBlockSize - 1) / kBlockSize;
    const int32_t* bt = bt_row + c0 / kBlockSize;

    // ---- QK: scores of this chunk into LDS -------------------------------
    for (int j = wave; j < nblk; j += kWaves) {
      const uint16_t* tile = k_cache + (int64_t)bt[j] * blk_stride + head_off + tq * D;
      uint4 kv[CPL];
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci)
        kv[ci] = *reinterpret_cast<const uint4*>(tile + (qd + 4 * ci) * 8);
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int ci = 0; ci < CPL; ++ci) {
          a = dot2_bf16(qr[h][ci].x, kv[ci].x, a);
          a = dot2_bf16(qr[h][ci].y, kv[ci].y, a);
          a = dot2_bf16(qr[h][ci].z, kv[ci].z, a);
          a = dot2_bf16(qr[h][ci].w, kv[ci].w, a);
        }
        s[h] = quad_sum(a);
      }
      const bool valid = j * kBlockSize + tq < nt;
      if (qd == 0) {
        const int idx = j * kBlockSize + (tq % TG) * IPB + tq / TG;
#pragma unroll
        for (int h = 0; h < G; ++h) s_buf[h * kChunkTokens + idx] = valid ? s[h] * scale_log2 : -INFINITY;
      }
    }
    __syncthreads();

    // ---- P: running max / sum, probabilities in place ---------------------
    for (int h = wave; h < G; h += kWaves) {
      float* sh = s_buf + h * kChunkTokens;
      const int n = nblk * kBlockSize;
      float m = -INFINITY;
      for (int e = lane; e < n; e += 64) m = fmaxf(m, sh[e]);
      m = wave_max(m);
      const float m_old = st_m[h];
      const float m_new = fmaxf(m_old, m);
      float sum = 0.f;
      for (int e = lane; e < n; e += 64) {
        const float pe = exp2f(sh[e] - m_new);
        sh[e] = pe;
        sum += pe;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        const float alpha = exp2f(m_old - m_new);
        st_a[h] = alpha;
        st_m[h] = m_new;
        st_l[h] = st_l[h] * alpha + sum;
      }
    }
    __syncthreads();

    // ---- PV: accumulate p * V ----------------------------------------------
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = st_a[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
    }
    for (int j = wave; j < nblk; j += kWaves) {
      const uint16_t* tile = v_cache + (int64_t)bt[j] * blk_stride + head_off + dc * 8;
      uint4 vv[IPB];
#pragma unroll
      for (int ii = 0; ii < IPB; ++ii)
        vv[ii] = *reinterpret_cast<const uint4*>(tile + (tg + TG * ii) * D);
      if ((j + 1) * kBlockSize > nt) {
#pragma unroll
        for (int ii = 0; ii < IPB; ++ii)
          if (j * kBlockSize + tg + TG * ii >= nt) vv[ii] = make_uint4(0u, 0u, 0u, 0u);
      }
      float pp[G][IPB];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float* src = s_buf + h * kChunkTokens + j * kBlockSize + tg * IPB;
        if constexpr (IPB == 4) {
          const float4 t4 = *reinterpret_cast<const float4*>(src);
          pp[h][0] = t4.x; pp[h][1] = t4.y; pp[h][2] = t4.z; pp[h][3] = t4.w;
        } else {
          const float2 t2 = *reinterpret_cast<const float2*>(src);
          pp[h][0] = t2.x; pp[h][1] = t2.y;
        }
      }
#pragma unroll
      for (int ii = 0; ii < IPB; ++ii) {
        const float x[8] = {bf16lo(vv[ii].x), bf16hi(vv[ii].x), bf16lo(vv[ii].y), bf16hi(vv[ii].y),
                            bf16lo(vv[ii].z), bf16hi(vv[ii].z), bf16lo(vv[ii].w), bf16hi(vv[ii].w)};
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pp[h][ii], x[e], acc[h][e]);
      }
    }
    __syncthreads();
  }

  // ---- combine token groups (lanes) and waves, write ----------------------
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
#pragma unroll
      for (int off = NCH; off < 64; off <<= 1) x += __shfl_xor(x, off);
      acc[h][e] = x;
    }
  float* red = s_buf;  // [kWaves][G][D]; the score buffer is free after the last barrier
  if (lane < NCH) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(red + (wave * G + h) * D + dc * 8);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D / 4; e += blockDim.x) {
    const int h = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float4 t = *reinterpret_cast<const float4*>(red + (w * G + h) * D + d4);
      sum.x += t.x; sum.y += t.y; sum.z += t.z; sum.w += t.w;
    }
    const float inv = 1.f / st_l[h];
    const int64_t row = (int64_t)b * Hq + hq0 + h;
    if (SPLIT) {
      *reinterpret_cast<float4*>(o_part + (row * num_parts + p) * D + d4) =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
      if (d4 == 0) lse[row * num_parts + p] = st_m[h] + log2f(st_l[h]);
    } else {
      uint2 o;
      o.x = pack_bf16x2(sum.x * inv, sum.y * inv);
      o.y = pack_bf16x2(sum.z * inv, sum.w * inv);
      *reinterpret_cast<uint2*>(out + row * D + d4) = o;
    }
  }
}

// Log-sum-exp combine of split-K partials: one wave per (sequence, query head).
template <int D>
__global__ void __launch_bounds__(64)
combine_kernel(uint16_t* __restrict__ out, const float* __restrict__ o_part,
               const float* __restrict__ lse, const int32_t* __restrict__ context_lens, int Hq,
               int num_parts, int part_tokens) {
  constexpr int PER = D / 64;  // output dims per lane
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)b * Hq + h;
  const int L = context_lens[b];
  uint16_t* o = out + row * D + lane * PER;
  if (L <= 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0;
    return;
  }
  const int n = (L + part_tokens - 1) / part_tokens;
  const float* ls = lse + row * num_parts;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, ls[i]);
  float acc[PER] = {};
  float wsum = 0.f;
  for (int i = 0; i < n; ++i) {
    const float w = exp2f(ls[i] - M);
    wsum += w;
    const float* src = o_part + (row * num_parts + i) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
  const float inv = 1.f / wsum;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    o[0] = (uint16_t)f32_to_bf16_rne(acc[0] * inv);
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
    hipLaunchKernelGGL((decode_kernel<D, G, true>), dim3(np, Hkv, B), dim3(256), 0, stream, qq, kc,
                       vc, block_tables, context_lens, Hkv, max_blocks, scale_log2, partition_size,
                       np, oo, o_part, lse);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, G, false>), dim3(1, Hkv, B), dim3(256), 0, stream, qq, kc,
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
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(Hq, B), dim3(64), 0, stream, oo, o_part, lse,
                       context_lens, Hq, num_partitions, partition_size);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3(Hq, B), dim3(64), 0, stream, oo, o_part, lse,
                       context_lens, Hq, num_partitions, partition_size);
  return hipGetLastError();
}

}  // namespace pa
