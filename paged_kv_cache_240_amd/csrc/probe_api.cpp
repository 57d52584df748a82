// C ABI of libpa_probe: the device-ceiling measurement kernels (include/pa_probe.h),
// kept out of the paged-attention library.  Validation on the host, then the
// launch; nothing here allocates, synchronises or throws.

#include <hip/hip_runtime.h>

#include "../../include/pa_probe.h"
#include "pa_internal.h"

namespace {
pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }
}  // namespace

extern "C" {

pa_status pa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sums, int32_t grid,
                               pa_stream_t stream) {
  if (!buf || !sums) return PA_ERR_NULL;
  if (bytes <= 0 || bytes % 16 != 0 || grid <= 0) return PA_ERR_SHAPE;
  return from_hip(pa::launch_probe_stream_read(buf, bytes, sums, grid, static_cast<hipStream_t>(stream)));
}

int64_t pa_probe_gather_read_groups(int64_t bytes) {
  return bytes > 0 ? pa::probe_gather_read_groups(bytes) : 0;
}

pa_status pa_probe_gather_read(const void* buf, int64_t bytes, uint32_t* sums, pa_stream_t stream) {
  if (!buf || !sums) return PA_ERR_NULL;
  const int64_t tiles = bytes / 4096;
  if (bytes <= 0 || bytes % 4096 != 0 || (tiles & (tiles - 1)) != 0) return PA_ERR_SHAPE;
  if (pa::probe_gather_read_groups(bytes) > 0x7fffffff) return PA_ERR_SHAPE;
  return from_hip(pa::launch_probe_gather_read(buf, bytes, sums, static_cast<hipStream_t>(stream)));
}

pa_status pa_probe_mfma_bf16(int32_t iters, float* out, int32_t grid, pa_stream_t stream) {
  if (!out) return PA_ERR_NULL;
  if (iters <= 0 || grid <= 0) return PA_ERR_SHAPE;
  return from_hip(pa::launch_probe_mfma_bf16(iters, out, grid, static_cast<hipStream_t>(stream)));
}

pa_status pa_probe_issue_mix(int32_t mode, int32_t iters, float* out, int32_t grid, pa_stream_t stream) {
  if (!out) return PA_ERR_NULL;
  if (mode < 1 || mode > 3 || iters <= 0 || grid <= 0) return PA_ERR_SHAPE;
  return from_hip(pa::launch_probe_issue_mix(mode, iters, out, grid, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
