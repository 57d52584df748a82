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
// Mapping: a workgroup copies four block pairs of the K (pool 0) or V (pool 1)
// pools with 16-byte loads and stores, eight per thread in flight; every byte
// is read once and written once.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyBlocks = 4;  // block pairs per workgroup
constexpr int kCopyPer = 2;     // 16-byte pieces per thread and pair per round

// Workgroup (x, pool) copies pairs kCopyBlocks*x .. +kCopyBlocks-1 of the K
// (pool 0) or V (pool 1) pools.  Per round a thread loads kCopyPer pieces of
// each of the pairs (eight 16-byte loads in flight) before storing any.
__global__ void __launch_bounds__(kCopyThreads)
block_copy_kernel(uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
                  const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
                  const int32_t* __restrict__ src_ids, const int32_t* __restrict__ dst_ids, int n,
                  int64_t pieces_per_block) {
  const int first = blockIdx.x * kCopyBlocks;
  const int nb = min(kCopyBlocks, n - first);
  const bool is_v = blockIdx.y != 0;
  const uint4* src = is_v ? src_v : src_k;
  uint4* dst = is_v ? dst_v : dst_k;
  int64_t s_base[kCopyBlocks], d_base[kCopyBlocks];
#pragma unroll
  for (int b = 0; b < kCopyBlocks; ++b) {
    const int i = first + min(b, nb - 1);
    s_base[b] = (int64_t)src_ids[i] * pieces_per_block;
    d_base[b] = (int64_t)dst_ids[i] * pieces_per_block;
  }
  for (int64_t base = threadIdx.x; base < pieces_per_block; base += kCopyThreads * kCopyPer) {
    uint4 t[kCopyBlocks][kCopyPer];
#pragma unroll
    for (int b = 0; b < kCopyBlocks; ++b)
#pragma unroll
      for (int u = 0; u < kCopyPer; ++u) {
        // unconditional, from a valid address (pairs past n repeat the last
        // pair, pieces past the tile its last piece): a branch here would
        // keep t in memory
        const int64_t j = min(base + u * kCopyThreads, pieces_per_block - 1);
        t[b][u] = src[s_base[b] + j];
      }
    // every load is issued here, before the guarded stores (the compiler would
    // otherwise sink each load into its store's branch: one load in flight)
#pragma unroll
    for (int b = 0; b < kCopyBlocks; ++b)
#pragma unroll
      for (int u = 0; u < kCopyPer; ++u)
        asm volatile("" ::"v"(t[b][u].x), "v"(t[b][u].y), "v"(t[b][u].z), "v"(t[b][u].w));
#pragma unroll
    for (int b = 0; b < kCopyBlocks; ++b)
#pragma unroll
      for (int u = 0; u < kCopyPer; ++u) {
        const int64_t j = base + u * kCopyThreads;
        if (b < nb && j < pieces_per_block) dst[d_base[b] + j] = t[b][u];
      }
  }
}

}  // namespace

hipError_t launch_block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                             const int32_t* src_ids, const int32_t* dst_ids, int n,
                             int64_t bytes_per_block, hipStream_t stream) {
  const dim3 grid((n + kCopyBlocks - 1) / kCopyBlocks, 2), block(kCopyThreads);
  hipLaunchKernelGGL(block_copy_kernel, grid, block, 0, stream, static_cast<uint4*>(dst_k),
                     static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
                     static_cast<const uint4*>(src_v), src_ids, dst_ids, n, bytes_per_block / 16);
  return hipGetLastError();
}

}  // namespace pa
