// Device ceilings for the rooflines: how fast this device streams reads from
// HBM and how fast its matrix cores multiply bf16, measured rather than taken
// from the data sheet (decode and the store are bound by the first, prefill by
// the second: Pico-vLLM write-up, H200 comparison; the 15x-on-a-T4 article).
//
// stream_read: a grid-stride walk over a buffer with 16-byte non-temporal
// loads, eight in flight per thread, folded into a 32-bit sum per lane so the
// loads cannot be removed; one sum per workgroup is written.
// gather_read: the buffer as 4 KiB tiles visited in a scrambled order (tile t
// at (t * 0x9E3779B1) mod ntiles, a bijection for a power-of-two count), each
// wave loading its 4 tiles with all 16 of its 16-byte loads in flight, then
// leaving: one pass, the access granularity and the scattered placement of a
// paged K/V read.  Sums as stream_read.
// mfma_bf16: every wave runs `iters` rounds of four independent
// v_mfma_f32_16x16x32_bf16 chains on operands of bf16 ones, so each
// accumulator element ends at exactly 32 * iters; lane 0 of each wave writes
// the sum of its first elements (4 * 32 * iters).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const uint4* __restrict__ buf, int64_t n16, uint32_t* __restrict__ sums) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 t[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) t[u] = load_stream16(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc += t[u].x + t[u].y + t[u].z + t[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 t = load_stream16(buf + i);
    acc += t.x + t.y + t.z + t.w;
  }
  __shared__ uint32_t part[kProbeThreads / 64];
  // wave sum through LDS (integer, order-free)
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) s += part[w];
    sums[blockIdx.x] = s;
  }
}

constexpr int kTileWords16 = 4096 / 16;  // 16-byte pieces of a 4 KiB tile
constexpr int kGatherTiles = 4;           // tiles per wave (the fastest one-launch read of a sweep over 2, 4, 8, 16)

__global__ void __launch_bounds__(kProbeThreads)
gather_read_kernel(const uint4* __restrict__ buf, int64_t ntiles, uint32_t* __restrict__ sums) {
  const int lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)) * kGatherTiles;
  uint32_t acc = 0;
  uint4 t[kGatherTiles][4];
#pragma unroll
  for (int j = 0; j < kGatherTiles; ++j) {
    // tiles past the end re-read the last one and are not counted
    const int64_t lt = min(t0 + j, ntiles - 1);
    const int64_t tile = (int64_t)((uint64_t)lt * 0x9E3779B1ull & (uint64_t)(ntiles - 1));
    const uint4* src = buf + tile * kTileWords16 + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) t[j][k] = load_stream16(src + k * 64);
  }
#pragma unroll
  for (int j = 0; j < kGatherTiles; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc += t0 + j < ntiles ? t[j][k].x + t[j][k].y + t[j][k].z + t[j][k].w : 0u;
  __shared__ uint32_t part[kProbeThreads / 64];
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) s += part[w];
    sums[blockIdx.x] = s;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads)
mfma_bf16_kernel(int iters, float* __restrict__ out) {
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                0x3F803F80u, 0x3F803F80u));
  floatx4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ones, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ones, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ones, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ones, c3, 0, 0, 0);
  }
  if ((threadIdx.x & 63) == 0)
    out[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = c0[0] + c1[0] + c2[0] + c3[0];
}

// Issue mix: per iteration, a wave runs (mode & 1) sixteen 16x16x32 bf16
// products on bf16 ones into 8 independent accumulators, and/or (mode & 2)
// thirty-two exp2 + FMA steps on 16 independent chains.  Each lane writes
// out[thread] = (sum of its accumulators' first elements) + (sum of its
// chains), both deterministic; timing the launch per mode and per waves per
// SIMD shows whether the SIMD overlaps the two kinds of work.
template <int MODE>
__global__ void __launch_bounds__(kProbeThreads)
issue_mix_kernel(int iters, float* __restrict__ out) {
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                0x3F803F80u, 0x3F803F80u));
  floatx4_t c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = 1e-3f * (float)((threadIdx.x & 63) + k);
  for (int it = 0; it < iters; ++it) {
    if constexpr ((MODE & 1) != 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ones, c[k], 0, 0, 0);
    }
    if constexpr ((MODE & 2) != 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = __builtin_amdgcn_exp2f(fmaf(v[k], -0.5f, 0.125f));  // contracts to a fixed point
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += c[k][0];
#pragma unroll
  for (int k = 0; k < 16; ++k) sum += v[k];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = sum;
}

}  // namespace

hipError_t launch_probe_issue_mix(int mode, int iters, float* out, int grid, hipStream_t stream) {
  switch (mode) {
    case 1: hipLaunchKernelGGL(issue_mix_kernel<1>, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out); break;
    case 2: hipLaunchKernelGGL(issue_mix_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out); break;
    default: hipLaunchKernelGGL(issue_mix_kernel<3>, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sums, int grid,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sums);
  return hipGetLastError();
}

int64_t probe_gather_read_groups(int64_t bytes) {
  const int64_t per_group = (int64_t)(kProbeThreads / 64) * kGatherTiles;
  return (bytes / 4096 + per_group - 1) / per_group;
}

hipError_t launch_probe_gather_read(const void* buf, int64_t bytes, uint32_t* sums,
                                    hipStream_t stream) {
  const int64_t groups = probe_gather_read_groups(bytes);
  hipLaunchKernelGGL(gather_read_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 4096, sums);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_bf16(int iters, float* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace pa
