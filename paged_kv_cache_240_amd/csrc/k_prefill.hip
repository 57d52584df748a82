// Causal paged chunked prefill for gfx950 (bf16 MFMA).  Placeholder launcher
// until the kernel lands: reports "not supported".
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_prefill(void*, const void*, const void*, const void*, const int32_t*,
                          const int32_t*, const int32_t*, int, int, int, int, int, int, float,
                          hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
