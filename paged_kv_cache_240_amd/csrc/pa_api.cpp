// C ABI of libpa: argument validation, partition choice, workspace sizing and
// dispatch to the gfx950 kernels.  Every check runs on the host before any
// work is enqueued; nothing here allocates, synchronises or throws.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {
constexpr int kBlockSizeHost = 16;  // the only block size the kernels implement
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool head_shape_ok(int32_t Hq, int32_t Hkv, int32_t D, pa_status* st) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) {
    *st = PA_ERR_SHAPE;
    return false;
  }
  const int32_t G = Hq / Hkv;
  if ((D != 64 && D != 128) || G > 8) {
    *st = PA_ERR_UNSUPPORTED;
    return false;
  }
  return true;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validation shared by the decode entry points.
pa_status check_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                       int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                       int32_t max_context_len) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  pa_status st = PA_OK;
  if (!head_shape_ok(Hq, Hkv, D, &st)) return st;
  if (block_size != pa::kBlockSizeHost) return block_size > 0 ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  if (B < 0 || max_blocks <= 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks * block_size) return PA_ERR_SHAPE;
  return PA_OK;
}

// True when the device can read and write p directly: device memory, or
// pinned host memory mapped for the device.  Pageable host memory (which a
// kernel cannot touch) and unknown pointers are refused; a failed query's
// error state is cleared so it cannot surface in a later launch check.
bool device_accessible(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeDevice) return true;
  return a.type == hipMemoryTypeHost && a.devicePointer != nullptr;
}

int32_t resolve_partition(int32_t partition_size, int32_t B, int32_t Hkv, int32_t max_context_len) {
  return partition_size == -1 ? pa_decode_partition_size(B, Hkv, max_context_len) : partition_size;
}

// partition_size -1 for the multi-query decode: the decode choice, except that
// rows filling two 16-row tiles (NQ * G > 16) move from 512 to 1024 tokens while
// the 1024-token grid still gives every CU a workgroup.  A 1024-token partition
// runs as one chunk of 8 waves, two per SIMD, and halves the partials to
// reduce: measured 29.4 against 30.9 us per call on 16 x 8192 tokens, NQ = 5.
int32_t resolve_multi_partition(int32_t partition_size, int32_t B, int32_t NQ, int32_t Hq,
                                int32_t Hkv, int32_t max_context_len) {
  if (partition_size != -1) return partition_size;
  const int32_t P = pa_decode_partition_size(B, Hkv, max_context_len);
  if (P == 512 && Hkv > 0 && (int64_t)NQ * (Hq / Hkv) > 16 &&
      (int64_t)B * Hkv * ceil_div(max_context_len, 1024) >= device_cu_count())
    return 1024;
  return P;
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: sizes are inconsistent or out of range";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape not implemented (block_size 16, head_dim 64/128, Hq/Hkv <= 8)";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported an error";
    case PA_ERR_MEMORY: return "PA_ERR_MEMORY: a pointer is neither device memory nor device-accessible pinned host memory";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY: not enough free blocks or output space";
  }
  return "unknown pa_status";
}

pa_status pa_cache_store(void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                         const int32_t* slot_mapping, const int32_t* positions,
                         const float* cos_sin, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int64_t num_blocks, int32_t max_pos,
                         pa_stream_t stream) {
  if (T < 0 || num_blocks < 0 || max_pos < 0) return PA_ERR_SHAPE;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !positions || !cos_sin)
    return PA_ERR_NULL;
  pa_status st = PA_OK;
  if (!head_shape_ok(q ? Hq : Hkv, Hkv, D, &st)) return st;
  if (block_size != pa::kBlockSizeHost) return block_size > 0 ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  if (T == 0) return PA_OK;
  if (num_blocks == 0 || max_pos == 0) return PA_ERR_SHAPE;
  return from_hip(pa::launch_cache_store(q, k, v, k_cache, v_cache, slot_mapping, positions,
                                         cos_sin, T, Hq, Hkv, D,
                                         static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_partition_size(int32_t B, int32_t Hkv, int32_t max_context_len) {
  // Measured on MI355X (Qwen head shape, 1 to 128 sequences of 512 to 32768
  // tokens): partitions of up to 256 tokens put every K/V load of a wave in
  // flight at once, a launch runs best with up to two workgroups per CU, and
  // the reduce is a launch of its own, cheap up to 64 partitions per sequence.
  // So:
  //  * (sequence, KV head) pairs that already give every CU a workgroup, or
  //    contexts that fit one 128-token partition: one pass, no reduce;
  //  * otherwise the smallest of 128, 256 and 512 tokens that keeps the grid
  //    within two workgroups per CU and a sequence within 64 partitions;
  //  * failing that, 512, doubled while a sequence needs more than 64.
  if (B <= 0 || Hkv <= 0 || max_context_len <= 0) return 0;
  const int64_t cus = device_cu_count();
  const int64_t pairs = (int64_t)B * Hkv;
  if (pairs >= cus || max_context_len <= 128) return 0;
  for (int64_t P = 128; P <= 512; P *= 2)
    if (pairs * ceil_div(max_context_len, P) <= 2 * cus && ceil_div(max_context_len, P) <= 64)
      return (int32_t)P;
  int64_t P = 512;
  while (ceil_div(max_context_len, P) > 64) P *= 2;
  return (int32_t)P;
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_context_len, int32_t partition_size) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_context_len < 0) return 0;
  const int32_t P = resolve_partition(partition_size, B, Hkv, max_context_len);
  if (P <= 0 || P % 16 != 0) return 0;
  const int64_t np = ceil_div(max_context_len, P);
  return (size_t)((int64_t)B * Hq * np * (D + 1) * (int64_t)sizeof(float));
}

pa_status pa_decode_partitions(float* o_part, float* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t block_size, int32_t max_blocks,
                               int32_t max_context_len, float scale, int32_t partition_size,
                               pa_stream_t stream) {
  if (!o_part || !lse) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0) return PA_ERR_SHAPE;
  if (B == 0 || max_context_len == 0) return PA_OK;
  return from_hip(pa::launch_decode(nullptr, o_part, lse, q, k_cache, v_cache, block_tables,
                                    context_lens, B, Hq, Hkv, D, max_blocks, max_context_len, scale,
                                    partition_size, static_cast<hipStream_t>(stream)));
}

pa_status pa_decode_combine(void* out, const float* o_part, const float* lse,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t D,
                            int32_t max_context_len, int32_t partition_size, pa_stream_t stream) {
  if (!out || !o_part || !lse || !context_lens) return PA_ERR_NULL;
  if (B < 0 || Hq <= 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (D != 64 && D != 128) return D > 0 ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  if (partition_size <= 0 || partition_size % 16 != 0) return PA_ERR_SHAPE;
  if (B == 0) return PA_OK;
  const int np = (int)ceil_div(max_context_len, partition_size);
  return from_hip(pa::launch_decode_combine(out, o_part, lse, context_lens, B, Hq, D,
                                            np > 0 ? np : 1, partition_size,
                                            static_cast<hipStream_t>(stream)));
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (!out) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0)) return PA_ERR_SHAPE;
  const int32_t P = resolve_partition(partition_size, B, Hkv, max_context_len);
  if (B == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (P == 0 || max_context_len == 0)
    return from_hip(pa::launch_decode(out, nullptr, nullptr, q, k_cache, v_cache, block_tables,
                                      context_lens, B, Hq, Hkv, D, max_blocks, max_context_len,
                                      scale, 0, s));
  const size_t need = pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, P);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const int64_t np = ceil_div(max_context_len, P);
  float* o_part = static_cast<float*>(workspace);
  float* lse = o_part + (int64_t)B * Hq * np * D;
  hipError_t e = pa::launch_decode(nullptr, o_part, lse, q, k_cache, v_cache, block_tables,
                                   context_lens, B, Hq, Hkv, D, max_blocks, max_context_len, scale,
                                   P, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  return from_hip(pa::launch_decode_combine(out, o_part, lse, context_lens, B, Hq, D, (int)np, P, s));
}

pa_status pa_decode_step(void* out, const void* q, const void* k, const void* v, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                         const float* cos_sin, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t max_blocks, int32_t max_context_len,
                         int32_t max_pos, float scale, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, pa_stream_t stream) {
  if (!out || !k || !v || !cos_sin) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0)) return PA_ERR_SHAPE;
  if (max_pos < max_context_len) return PA_ERR_SHAPE;
  const int32_t P = resolve_partition(partition_size, B, Hkv, max_context_len);
  if (B == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (P == 0 || max_context_len == 0)
    return from_hip(pa::launch_decode_step(out, nullptr, nullptr, q, k, v, k_cache, v_cache,
                                           block_tables, context_lens, cos_sin, B, Hq, Hkv, D,
                                           max_blocks, max_context_len, scale, 0, true, s));
  const size_t need = pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, P);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const int64_t np = ceil_div(max_context_len, P);
  float* o_part = static_cast<float*>(workspace);
  float* lse = o_part + (int64_t)B * Hq * np * D;
  return from_hip(pa::launch_decode_step(out, o_part, lse, q, k, v, k_cache, v_cache,
                                         block_tables, context_lens, cos_sin, B, Hq, Hkv, D,
                                         max_blocks, max_context_len, scale, P, true, s));
}

pa_status pa_decode_step_partitions(float* o_part, float* lse, const void* q, const void* k,
                                    const void* v, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    const float* cos_sin, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t block_size, int32_t max_blocks,
                                    int32_t max_context_len, int32_t max_pos, float scale,
                                    int32_t partition_size, pa_stream_t stream) {
  if (!o_part || !lse || !k || !v || !cos_sin) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0) return PA_ERR_SHAPE;
  if (max_pos < max_context_len) return PA_ERR_SHAPE;
  if (B == 0 || max_context_len == 0) return PA_OK;
  return from_hip(pa::launch_decode_step(nullptr, o_part, lse, q, k, v, k_cache, v_cache,
                                         block_tables, context_lens, cos_sin, B, Hq, Hkv, D,
                                         max_blocks, max_context_len, scale, partition_size, false,
                                         static_cast<hipStream_t>(stream)));
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                            int32_t max_blocks, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_stream_t stream) {
  // the workspace this call needs (0 for a single pass), checked before anything
  // touches the device: more than the library's array is refused
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0)) return PA_ERR_SHAPE;
  const int32_t P = resolve_partition(partition_size, B, Hkv, max_context_len);
  const size_t need = P > 0 && B > 0 && max_context_len > 0
                          ? pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, P)
                          : 0;
  if (need > PA_DECODE_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = pa::decode_scratch();
  if (ws == nullptr) return PA_ERR_HIP;
  return pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D, block_size,
                   max_blocks, max_context_len, scale, P, ws, PA_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}

namespace {
constexpr int kPrefixPartTokens = 128;  // smallest shared-prefix partition: one 32-key step per key range
constexpr int kMaxCascadeSlots = 64;
constexpr int kOneLaunchPrefix = 512;   // prefix partition of the one-launch path
constexpr int kOneLaunchMaxItems = 1;   // its prefix items per CU, at most

int32_t cascade_slots(int32_t max_suffix, int32_t P, int32_t max_prefix, int32_t Pg = kPrefixPartTokens) {
  return (int32_t)(ceil_div(max_suffix, P) + ceil_div(max_prefix, Pg));
}

// Prefix partition size of the group pass: 512 tokens (measured best or
// within a few percent of the best on groups of 64-256 sequences over
// 2000-8192-token prefixes: smaller partitions multiply the partials to write
// and reduce, larger ones leave CUs idle); halved while the grid would hold
// fewer workgroups than a quarter of the CUs, doubled while the slots would
// not fit; 0 if no size fits.
int32_t prefix_partition(int32_t row_blocks, int32_t max_prefix, int32_t suffix_slots) {
  const int cus = device_cu_count();
  int32_t Pg = 4 * kPrefixPartTokens;
  while (Pg > kPrefixPartTokens && (int64_t)row_blocks * ceil_div(max_prefix, Pg) < cus / 4) Pg /= 2;
  while (suffix_slots + ceil_div(max_prefix, Pg) > kMaxCascadeSlots) {
    if (Pg >= 8 * kPrefixPartTokens) return 0;
    Pg *= 2;
  }
  return Pg;
}
}  // namespace

size_t pa_decode_shared_prefix_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                               int32_t max_suffix_len, int32_t max_prefix,
                                               int32_t partition_size) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_suffix_len < 0 || max_prefix < 0) return 0;
  // -1: the smallest partition the library may choose, so the most slots
  const int32_t P = partition_size == -1 ? 64 : partition_size;
  if (P <= 0 || P % 16 != 0) return 0;
  const int64_t slots = cascade_slots(std::max(max_suffix_len, 1), P, max_prefix);
  return (size_t)((int64_t)B * Hq * slots * (D + 1) * (int64_t)sizeof(float));
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens, int32_t B,
                                  int32_t num_groups, int32_t max_group_size, int32_t max_prefix,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                  int32_t max_blocks, int32_t max_context_len, int32_t max_suffix_len,
                                  float scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, pa_stream_t stream) {
  if (!out || !prefix_lens || (num_groups > 0 && !group_start)) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (num_groups < 0 || max_prefix < 0 || max_prefix % 16 != 0 || max_prefix > max_context_len ||
      max_suffix_len < 0 || max_suffix_len > max_context_len)
    return PA_ERR_SHAPE;
  if (num_groups > 0 && (max_group_size <= 0 || max_group_size > B)) return PA_ERR_SHAPE;
  if (partition_size < -1 || partition_size == 0 || (partition_size > 0 && partition_size % 16 != 0))
    return PA_ERR_SHAPE;
  if (B == 0 || max_context_len == 0) return B == 0 ? PA_OK : from_hip(pa::launch_decode(
      out, nullptr, nullptr, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
      max_blocks, max_context_len, scale, 0, static_cast<hipStream_t>(stream)));
  const int32_t suf = std::max(max_suffix_len, 1);
  // the library's choice for the suffixes: pa_decode's rule on the suffix length
  // (about two workgroups per CU), at least 64 tokens, one partition when the
  // batch alone fills the device
  int32_t P = partition_size;
  if (P == -1) {
    P = pa_decode_partition_size(B, Hkv, suf);
    P = P == 0 ? (int32_t)(ceil_div(suf, 16) * 16) : P;
    P = std::max<int32_t>(P, 64);
  }
  const int32_t suffix_slots = (int32_t)ceil_div(suf, P);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // One partition launch for prefixes and suffixes together: prefix items of one
  // 16-row tile (16 / G sequences of a group), prefix partitions of kOneLaunchPrefix
  // tokens; taken when there is a prefix, the suffix partitions are single
  // chunks and the prefix items stay within kOneLaunchMaxItems per CU.  (With no
  // prefix the suffix pass below is pa_decode's own partition kernel.)
  {
    const int32_t Pc = kOneLaunchPrefix;
    const int64_t sub = 16 / (Hq / Hkv);
    const int64_t pre_items = (num_groups > 0 && max_prefix > 0)
                                  ? (int64_t)num_groups * ceil_div(std::max(max_group_size, 1), sub) *
                                        ceil_div(max_prefix, Pc) * Hkv
                                  : 0;
    const int32_t slots = cascade_slots(suf, P, max_prefix, Pc);
    if (pre_items > 0 && P <= 512 && slots <= kMaxCascadeSlots &&
        pre_items <= kOneLaunchMaxItems * device_cu_count()) {
      const size_t need = (size_t)((int64_t)B * Hq * slots * (D + 1) * (int64_t)sizeof(float));
      if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
      float* o_part = static_cast<float*>(workspace);
      float* lse = o_part + (int64_t)B * Hq * slots * D;
      hipError_t e = pa::launch_cascade_decode(o_part, lse, q, k_cache, v_cache, block_tables,
                                               context_lens, group_start, prefix_lens, B, num_groups,
                                               max_group_size, max_prefix, Pc, suf, P, suffix_slots,
                                               slots, Hq, Hkv, D, max_blocks, scale, s);
      if (e != hipSuccess) return PA_ERR_HIP;
      return from_hip(pa::launch_decode_combine_cascade(out, o_part, lse, context_lens, prefix_lens,
                                                        B, Hq, D, slots, P, suffix_slots, Pc, s));
    }
  }
  // Otherwise the group pass on the matrix cores (the chunked-prefill kernel's
  // 96-row workgroups), then the suffix partitions, then the reduce.
  // row blocks of (sequence, head) rows per group, times KV heads and groups
  const int32_t row_blocks = (int32_t)(pa::group_prefix_row_blocks(std::max(max_group_size, 1), Hq / Hkv) *
                                       Hkv * std::max(num_groups, 1));
  const int32_t Pg = max_prefix > 0 ? prefix_partition(row_blocks, max_prefix, suffix_slots)
                                    : kPrefixPartTokens;
  if (Pg == 0) return PA_ERR_UNSUPPORTED;
  const int32_t slots = cascade_slots(suf, P, max_prefix, Pg);
  if (slots > kMaxCascadeSlots) return PA_ERR_UNSUPPORTED;
  // the workspace query sizes for the smallest prefix partition: always enough
  const size_t need = (size_t)((int64_t)B * Hq * slots * (D + 1) * (int64_t)sizeof(float));
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  float* o_part = static_cast<float*>(workspace);
  float* lse = o_part + (int64_t)B * Hq * slots * D;
  const int32_t slot0 = suffix_slots;
  if (num_groups > 0 && max_prefix > 0) {
    hipError_t e = pa::launch_group_prefix(o_part, lse, q, k_cache, v_cache, block_tables, group_start,
                                           prefix_lens, num_groups, max_group_size, max_prefix,
                                           Pg, slot0, slots, Hq, Hkv, D, max_blocks, scale, s);
    if (e != hipSuccess) return PA_ERR_HIP;
  }
  hipError_t e = pa::launch_decode_suffix(o_part, lse, q, k_cache, v_cache, block_tables,
                                          context_lens, prefix_lens, B, Hq, Hkv, D, max_blocks,
                                          suf, scale, P, slots, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  return from_hip(pa::launch_decode_combine_cascade(out, o_part, lse, context_lens, prefix_lens, B,
                                                    Hq, D, slots, P, slot0, Pg, s));
}

size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t NQ, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t max_context_len, int32_t partition_size) {
  if (NQ <= 0 || B < 0 || Hq <= 0 || Hkv <= 0 || max_context_len < 0) return 0;
  const int32_t P = resolve_multi_partition(partition_size, B, NQ, Hq, Hkv, max_context_len);
  const size_t per_query = pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, P);
  return per_query * (size_t)NQ;
}

pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t NQ, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                          int32_t max_blocks, int32_t max_context_len, float scale,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          pa_stream_t stream) {
  if (!out) return PA_ERR_NULL;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D,
                              block_size, max_blocks, max_context_len);
  if (st != PA_OK) return st;
  if (NQ <= 0) return PA_ERR_SHAPE;
  if ((int64_t)NQ * (Hq / Hkv) > 32) return PA_ERR_UNSUPPORTED;
  if (partition_size < -1 || (partition_size > 0 && partition_size % 16 != 0)) return PA_ERR_SHAPE;
  const int32_t P = resolve_multi_partition(partition_size, B, NQ, Hq, Hkv, max_context_len);
  if (B == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (P == 0 || max_context_len == 0)
    return from_hip(pa::launch_decode_multi(out, nullptr, nullptr, q, k_cache, v_cache,
                                            block_tables, context_lens, B, NQ, Hq, Hkv, D,
                                            max_blocks, max_context_len, scale, 0, s));
  const size_t need = pa_decode_multi_workspace_bytes(B, NQ, Hq, Hkv, D, max_context_len, P);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const int64_t np = ceil_div(max_context_len, P);
  float* o_part = static_cast<float*>(workspace);
  float* lse = o_part + (int64_t)B * NQ * Hq * np * D;
  hipError_t e = pa::launch_decode_multi(nullptr, o_part, lse, q, k_cache, v_cache, block_tables,
                                         context_lens, B, NQ, Hq, Hkv, D, max_blocks,
                                         max_context_len, scale, P, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  // rows of sequence b are its NQ * Hq (query, head) pairs
  return from_hip(pa::launch_decode_combine(out, o_part, lse, context_lens, B, NQ * Hq, D, (int)np,
                                            P, s));
}

pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t n,
                         int32_t Hkv, int32_t D, int32_t block_size, pa_stream_t stream) {
  if (!dst_k || !dst_v || !src_k || !src_v) return PA_ERR_NULL;
  if (n < 0 || Hkv <= 0 || D <= 0) return PA_ERR_SHAPE;
  if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != pa::kBlockSizeHost) return block_size > 0 ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  if (n == 0) return PA_OK;  // the id lists may then be NULL
  if (!src_blocks || !dst_blocks) return PA_ERR_NULL;
  const void* ptrs[6] = {dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks};
  for (const void* p : ptrs)
    if (!device_accessible(p)) return PA_ERR_MEMORY;
  const int64_t bytes = (int64_t)Hkv * block_size * D * 2;
  return from_hip(pa::launch_block_copy(dst_k, dst_v, src_k, src_v, src_blocks, dst_blocks, n,
                                        bytes, static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t n, int32_t Hkv, int32_t D,
                         int32_t block_size, int64_t num_blocks, pa_stream_t stream) {
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (num_blocks < 0 || (n > 0 && num_blocks == 0)) return PA_ERR_SHAPE;
  return pa_swap_blocks(k_cache, v_cache, k_cache, v_cache, src_blocks, dst_blocks, n, Hkv, D,
                        block_size, stream);
}

pa_status pa_rmsnorm_residual(void* out, void* residual, const void* x, const void* weight,
                              int32_t T, int32_t H, float eps, pa_stream_t stream) {
  if (!out || !x || !weight) return PA_ERR_NULL;
  if (T < 0 || H <= 0 || !(eps >= 0.f)) return PA_ERR_SHAPE;
  if (H % 8 != 0 || H > 16384) return PA_ERR_UNSUPPORTED;
  if (T == 0) return PA_OK;
  return from_hip(pa::launch_rmsnorm(out, residual, x, weight, T, H, eps,
                                     static_cast<hipStream_t>(stream)));
}

pa_status pa_swiglu(void* out, const void* gate_up, int64_t T, int32_t I, pa_stream_t stream) {
  if (!out || !gate_up) return PA_ERR_NULL;
  if (T < 0 || I <= 0) return PA_ERR_SHAPE;
  if (I % 8 != 0 || I > (1 << 26) || T > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (T == 0) return PA_OK;
  return from_hip(pa::launch_swiglu(out, gate_up, T, I, static_cast<hipStream_t>(stream)));
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start_loc, int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                     int32_t D, int32_t block_size, int32_t max_blocks, int32_t max_query_len,
                     float scale, pa_stream_t stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PA_ERR_NULL;
  pa_status st = PA_OK;
  if (!head_shape_ok(Hq, Hkv, D, &st)) return st;
  if (block_size != pa::kBlockSizeHost) return block_size > 0 ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  if (B < 0 || T < 0 || max_blocks <= 0 || max_query_len < 0) return PA_ERR_SHAPE;
  if (B == 0 || T == 0 || max_query_len == 0) return PA_OK;
  if (max_query_len > T) return PA_ERR_SHAPE;
  if (pa::prefill_workgroups(B, Hq, Hkv, max_query_len) > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_prefill(out, q, k_cache, v_cache, block_tables, context_lens,
                                     query_start_loc, B, Hq, Hkv, D, max_blocks, max_query_len,
                                     scale, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
