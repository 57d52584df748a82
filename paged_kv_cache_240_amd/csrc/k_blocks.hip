// Block copies between KV pools for gfx950: copy-on-write and swap.
//
// Operation (mini-llm-engine post, §3.4: a block shared by several sequences
// (ref_count > 1) is copied to a fresh block before one of them writes it;
// §3.5: under memory pressure a preempted sequence's blocks are moved to host
// memory and brought back into new device blocks later): for every pair i,
//   dst_k[dst[i]] = src_k[src[i]],  dst_v[dst[i]] = src_v[src[i]]
// where a block is the whole [Hkv][16][D] tile of one physical block id.  The
// pools may be device memory or device-accessible pinned host memory, so the
// same kernel serves copy-on-write (device to device) and swap-out / swap-in
// (device to host / host to device, over PCIe).
//
// Mapping: workgroup (i, pool) copies block pair i of the K (pool 0) or V
// (pool 1) pools with 16-byte loads and stores, four per thread in flight;
// every byte is read once and written once.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte pieces in flight per thread

__global__ void __launch_bounds__(kCopyThreads)
block_copy_kernel(uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
                  const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
                  const int32_t* __restrict__ src_ids, const int32_t* __restrict__ dst_ids,
                  int64_t pieces_per_block) {
  const int i = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int64_t s = (int64_t)src_ids[i] * pieces_per_block;
  const int64_t d = (int64_t)dst_ids[i] * pieces_per_block;
  const uint4* src = (is_v ? src_v : src_k) + s;
  uint4* dst = (is_v ? dst_v : dst_k) + d;
  for (int64_t e = threadIdx.x; e < pieces_per_block; e += kCopyThreads * kCopyUnroll) {
    uint4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t j = e + (int64_t)u * kCopyThreads;
      if (j < pieces_per_block) t[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t j = e + (int64_t)u * kCopyThreads;
      if (j < pieces_per_block) dst[j] = t[u];
    }
  }
}

}  // namespace

hipError_t launch_block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                             const int32_t* src_ids, const int32_t* dst_ids, int n,
                             int64_t bytes_per_block, hipStream_t stream) {
  const dim3 grid(n, 2), block(kCopyThreads);
  hipLaunchKernelGGL(block_copy_kernel, grid, block, 0, stream, static_cast<uint4*>(dst_k),
                     static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
                     static_cast<const uint4*>(src_v), src_ids, dst_ids, bytes_per_block / 16);
  return hipGetLastError();
}

}  // namespace pa
