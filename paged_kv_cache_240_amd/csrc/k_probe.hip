// Device ceilings for the rooflines: how fast this device streams reads from
// HBM and how fast its matrix cores multiply bf16, measured rather than taken
// from the data sheet (decode and the store are bound by the first, prefill by
// the second: Pico-vLLM write-up, H200 comparison; the 15x-on-a-T4 article).
//
// stream_read: a grid-stride walk over a buffer with 16-byte non-temporal
// loads, eight in flight per thread, folded into a 32-bit sum per lane so the
// loads cannot be removed; one sum per workgroup is written.
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

}  // namespace

hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sums, int grid,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sums);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_bf16(int iters, float* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace pa
