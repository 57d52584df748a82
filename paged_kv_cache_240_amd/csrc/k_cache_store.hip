// Fused rotate-half RoPE + slot-mapped KV-cache store for gfx950.
//
// Operation (Pico-vLLM write-up, §2 kernel layer: the position encoding is
// fused with the cache write; §1: rotate_half computed in place;
// mini-llm-engine post, §3.1: a slot is a row of a 16-token physical block):
// for each token with a non-negative slot, rotate its query heads in place,
// rotate its key heads into the slot's row of the K pool and copy its value
// heads into the same row of the V pool.
//
// Bit-exactness: every output element is two fp32 products and one fp32
// add/sub, each rounded separately (FMA contraction is switched off for this
// file), then rounded to bf16 to nearest even.
//
// Mapping: one workgroup per token (the store moves ~10 KB per token at the
// Qwen2.5-1.5B head shape, so it is bandwidth-bound and tiny).  Work items
// are 4 rotate pairs (j .. j+3 with j+D/2 .. j+D/2+3) of one q or k head,
// read with 8-byte loads, followed by 16-byte pieces of the v rows.  A
// thread's first item is loaded together with the slot and position, before
// the padding test, so the critical path is two round trips: the token's
// rows and position, then its cos/sin row.

#include "pa_device.h"
#include "pa_internal.h"

#pragma clang fp contract(off)

namespace pa {
namespace {

template <int D>
__global__ void __launch_bounds__(256)
cache_store_kernel(uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, uint16_t* __restrict__ k_cache,
                   uint16_t* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping,
                   const int32_t* __restrict__ positions, const float* __restrict__ cos_sin,
                   int Hq, int Hkv) {
  constexpr int HALF = D / 2;
  constexpr int ITEMS_PER_HEAD = HALF / 4;
  constexpr int CHUNKS = D / 8;  // 16-byte pieces of a v row
  const int i = blockIdx.x;
  const int heads = Hkv + (q != nullptr ? Hq : 0);
  const int n_rot = heads * ITEMS_PER_HEAD;
  const int n_items = n_rot + Hkv * CHUNKS;

  // item `it`: rotate pairs of a head (it < n_rot) or a piece of a v row.
  // Both sources are loaded for every item, with clamped (always valid)
  // indices, so the loads carry no branch in front of them.
  struct Item { uint2 xa, xb; uint4 vv; };
  auto load_item = [&](int it) {
    const int r = min(it, n_rot - 1);
    const int head = r / ITEMS_PER_HEAD;
    const int64_t roff = head < Hkv ? ((int64_t)i * Hkv + head) * D : ((int64_t)i * Hq + (head - Hkv)) * D;
    const uint16_t* src = (head < Hkv ? k : q) + roff + (r % ITEMS_PER_HEAD) * 4;
    const int c = min(max(it - n_rot, 0), Hkv * CHUNKS - 1);
    Item x;
    x.xa = *reinterpret_cast<const uint2*>(src);
    x.xb = *reinterpret_cast<const uint2*>(src + HALF);
    x.vv = *reinterpret_cast<const uint4*>(v + ((int64_t)i * Hkv + c / CHUNKS) * D + (c % CHUNKS) * 8);
    return x;
  };

  const int slot = slot_mapping[i];
  const int pos = positions[i];
  const Item first = load_item(threadIdx.x);
  // keep the row loads above the padding test (the compiler would otherwise
  // sink them behind it and add a round trip)
  asm volatile("" ::"v"(first.xa.x), "v"(first.xa.y), "v"(first.xb.x), "v"(first.xb.y),
               "v"(first.vv.x), "v"(first.vv.y), "v"(first.vv.z), "v"(first.vv.w), "s"(pos));
  if (slot < 0) return;  // padding token: nothing written (its rows were only read)
  const int64_t blk = slot / kBlockSize;
  const int row = slot % kBlockSize;
  const float* cs = cos_sin + (int64_t)pos * D;

  auto store_item = [&](int it, const Item& x) {
    const int r = min(it, n_rot - 1);
    const int head = r / ITEMS_PER_HEAD;
    const int j0 = (r % ITEMS_PER_HEAD) * 4;
    const float4 c = *reinterpret_cast<const float4*>(cs + j0);
    const float4 s = *reinterpret_cast<const float4*>(cs + HALF + j0);
    if (it < n_rot) {
      uint16_t* dst = head < Hkv ? k_cache + ((blk * Hkv + head) * kBlockSize + row) * D
                                 : q + ((int64_t)i * Hq + (head - Hkv)) * D;
      const float a[4] = {bf16lo(x.xa.x), bf16hi(x.xa.x), bf16lo(x.xa.y), bf16hi(x.xa.y)};
      const float b[4] = {bf16lo(x.xb.x), bf16hi(x.xb.x), bf16lo(x.xb.y), bf16hi(x.xb.y)};
      const float cc[4] = {c.x, c.y, c.z, c.w};
      const float ss[4] = {s.x, s.y, s.z, s.w};
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ac = a[e] * cc[e];
        const float bs = b[e] * ss[e];
        const float bc = b[e] * cc[e];
        const float as = a[e] * ss[e];
        lo[e] = ac - bs;
        hi[e] = bc + as;
      }
      uint2 ya, yb;
      ya.x = pack_bf16x2(lo[0], lo[1]);
      ya.y = pack_bf16x2(lo[2], lo[3]);
      yb.x = pack_bf16x2(hi[0], hi[1]);
      yb.y = pack_bf16x2(hi[2], hi[3]);
      *reinterpret_cast<uint2*>(dst + j0) = ya;
      *reinterpret_cast<uint2*>(dst + HALF + j0) = yb;
    } else if (it < n_items) {
      const int cv = it - n_rot;
      *reinterpret_cast<uint4*>(v_cache + ((blk * Hkv + cv / CHUNKS) * kBlockSize + row) * D +
                                (cv % CHUNKS) * 8) = x.vv;
    }
  };

  store_item(threadIdx.x, first);
  for (int it = threadIdx.x + blockDim.x; it < n_items; it += blockDim.x) store_item(it, load_item(it));
}

}  // namespace

hipError_t launch_cache_store(void* q, const void* k, const void* v, void* k_cache, void* v_cache,
                              const int32_t* slot_mapping, const int32_t* positions,
                              const float* cos_sin, int T, int Hq, int Hkv, int D,
                              hipStream_t stream) {
  const dim3 grid(T), block(256);
  auto* qq = static_cast<uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* kc = static_cast<uint16_t*>(k_cache);
  auto* vc = static_cast<uint16_t*>(v_cache);
  if (D == 128)
    hipLaunchKernelGGL(cache_store_kernel<128>, grid, block, 0, stream, qq, kk, vv, kc, vc,
                       slot_mapping, positions, cos_sin, Hq, Hkv);
  else
    hipLaunchKernelGGL(cache_store_kernel<64>, grid, block, 0, stream, qq, kk, vv, kc, vc,
                       slot_mapping, positions, cos_sin, Hq, Hkv);
  return hipGetLastError();
}

}  // namespace pa
