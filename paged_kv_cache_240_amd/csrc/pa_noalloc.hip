// The device array behind pa_decode_noalloc (pa_api.cpp): pa_decode for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its split-K partials live in a file-scope
// device array, `scratch`, instead of a caller-provided workspace.
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
#include "pa_internal.h"

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

namespace pa {
void* decode_scratch() { return device_scratch(); }
}  // namespace pa
