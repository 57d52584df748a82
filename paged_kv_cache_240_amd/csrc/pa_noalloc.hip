// pa_decode_noalloc: pa_decode for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The split-K partials live in a file-scope device array, `scratch`, instead
// of a caller-provided workspace; everything else is pa_decode's path.
//
// The array's name in host code is a host-side stand-in, not a device
// address, so it is never passed to a kernel: its device address on each GPU
// is looked up once (hipGetSymbolAddress, with that GPU current) and that
// pointer is what the kernels receive.  Every call on one GPU shares that
// GPU's array: calls that overlap on one GPU (other streams, other threads)
// race.  Nothing in the array needs clearing between calls: each call writes
// every partial slot it later reads.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"

namespace {

constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch`, looked up on its first use there;
// NULL if the lookup fails (the error is cleared, so it cannot surface later).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t B, int32_t Hq,
                                       int32_t Hkv, int32_t D, int32_t block_size,
                                       int32_t max_blocks, int32_t max_context_len, float scale,
                                       int32_t partition_size, pa_stream_t stream) {
  // the workspace this call needs (0 for a single pass), checked before anything
  // else touches the device: larger than the array is refused
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0)) return PA_ERR_SHAPE;
  const int32_t P = partition_size == -1 && B > 0 && Hkv > 0 && max_context_len > 0
                        ? pa_decode_partition_size(B, Hkv, max_context_len)
                        : partition_size;
  const size_t need = P > 0 && B > 0 && max_context_len > 0
                          ? pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, P)
                          : 0;
  if (need > kScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (ws == nullptr) return PA_ERR_HIP;
  return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D, block_size,
                   max_blocks, max_context_len, scale, P, ws, kScratchBytes, stream);
}
