// Device helpers shared by the gfx950 kernels of libpa: bf16 bit handling,
// round-to-nearest-even narrowing and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace pa {

constexpr int kBlockSize = 16;  // tokens per physical KV block

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 packed in one 32-bit word -> the low / high element as fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN -> canonical 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Eight bf16 in a 16-byte piece <-> fp32 (exact widening; narrowing rounds
// to nearest even with the integer rounding above).
__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float (&f)[8]) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z); f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}
__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Interleave two packed bf16 pairs: (a.lo, b.lo) and (a.hi, b.hi).
__device__ __forceinline__ uint32_t interleave_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t interleave_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// A zero the compiler cannot see through.  Adding it to a base pointer inside
// a loop keeps constant offsets from that base inside the loop, where they fold
// into the memory instruction's immediate offset (hoisted, each offset would
// hold a register of its own for the whole loop).
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("; opaque zero" : "+s"(z));
  return z;
}

// Loads of data read once per launch (K/V tiles), with the non-temporal hint:
// the lines are not kept for reuse, which streams a gather of scattered 4 KiB
// tiles faster than ordinary loads do.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// Wave-uniform float into a scalar register.
__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// a.x*b.x + a.y*b.y + c on two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 4 lanes of a quad, result in every lane (two DPP quad_perm adds).
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return x;
}

// Sum over the 8 lanes of an aligned octet, result in every lane: two quad
// adds, then row_half_mirror (lane i of the octet reads lane 7-i), which pairs
// each lane of one quad with a lane of the other.
__device__ __forceinline__ float octet_sum(float x) {
  x = quad_sum(x);
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                             0x141, 0xF, 0xF, false));
  return x;
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1: a loop whose
// index is a compile-time constant in the body (register arrays stay in
// registers however large the body is).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Cross-lane partners without LDS: DPP inside 16-lane rows, then the gfx950
// row swaps (v_permlane16_swap: rows 0<->1 and 2<->3; v_permlane32_swap:
// lanes 0-31 <-> 32-63).  Each returns, in every lane, the value its partner
// row holds in the same position.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float swap16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  // r[0]: own value in even rows, partner's in odd rows; r[1]: the reverse
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float swap32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// IEEE maximum (a NaN operand gives NaN).  Unlike fmaxf it needs no
// canonicalising of its operands, and chains of it fold into three-input
// v_maximum3_f32.
__device__ __forceinline__ float maxn(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// maxn of x and the value the partner row holds (16-lane rows 0<->1 and
// 2<->3, or the two 32-lane halves), in every lane.  The partner's value is
// taken with the lane select of swap16 / swap32: a maximum of the two
// results of a permlane swap of x with itself is folded by the compiler to
// the first result alone, which drops the partner in half of the lanes.
__device__ __forceinline__ float maxn_swap16(float x) { return maxn(x, swap16(x)); }
__device__ __forceinline__ float maxn_swap32(float x) { return maxn(x, swap32(x)); }

// Reductions over the 64 lanes of a wave, result in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp<0x140>(x));  // row_mirror
  x = fmaxf(x, swap16(x));
  return fmaxf(x, swap32(x));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  x += swap16(x);
  return x + swap32(x);
}

}  // namespace pa
