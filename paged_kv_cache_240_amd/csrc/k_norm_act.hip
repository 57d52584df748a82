// Fused RMSNorm + residual add and fused SwiGLU for gfx950: the elementwise
// neighbours of attention in a decoder layer (Pico-vLLM write-up, §2 kernel
// layer: RMSNorm fused with the residual add; SwiGLU fused).
//
// rmsnorm_residual, one row of H values per workgroup:
//   r'  = bf16(x + r)                          (written back over r; exact in fp32)
//   out = bf16(w * r' / sqrt(mean(r'^2) + eps)) (fp32, one rounding)
// With no residual, r' = x and nothing is written back.
// swiglu, per element of a row of 2I values [gate | up]:
//   out = bf16(silu(gate) * up),  silu(g) = g / (1 + e^-g)   (fp32, see swiglu_piece)
//
// Both read every input once and write every output once with 16-byte
// accesses: HBM-bound.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kNormThreads = 256;

// A row's pieces stay in registers between the sum of squares and the scaling:
// PER = pieces of 8 values per thread (H <= 8 * PER * kNormThreads).
template <int PER, bool RESID>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(uint16_t* __restrict__ out, uint16_t* __restrict__ residual,
               const uint16_t* __restrict__ x, const uint16_t* __restrict__ weight, int H,
               float eps) {
  __shared__ float part[kNormThreads / 64];
  const int row = blockIdx.x;
  const int n8 = H / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)row * H);
  uint4* rr = reinterpret_cast<uint4*>(residual + (int64_t)row * H);
  float v[PER][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * kNormThreads;
    if (i < n8) {
      unpack_bf16x8(xr[i], v[k]);
      if (RESID) {
        float r[8];
        unpack_bf16x8(rr[i], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[k][e] = bf16lo(f32_to_bf16_rne(v[k][e] + r[e]));
        rr[i] = pack_bf16x8(v[k]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[k][e], v[k][e], ss);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += part[w];
  const float inv = 1.f / sqrtf(tot / (float)H + eps);
  const uint4* wr = reinterpret_cast<const uint4*>(weight);
  uint4* orow = reinterpret_cast<uint4*>(out + (int64_t)row * H);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * kNormThreads;
    if (i < n8) {
      float w[8];
      unpack_bf16x8(wr[i], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = w[e] * (v[k][e] * inv);
      orow[i] = pack_bf16x8(w);
    }
  }
}

constexpr int kActThreads = 256;
constexpr int kActPieces = 2;  // 8-value pieces per thread: 4 loads of 16 B in flight

// silu(g) * u = g * u * sigma(g), sigma(g) = 1 / (1 + 2^a), a = -g log2(e), from
// v_exp_f32 and v_rcp_f32 (a few fp32 ulps, far below the final bf16 rounding).
// Past a = 64 (g < -44.4) sigma(g) = 2^-a to within 2^-64 relative; there it is
// applied as 2^-(a - n) times an exact scaling by 2^-n, so results that are
// tiny but still representable (down to the subnormals) are not lost to an
// overflow of 2^a.  That path is taken only when some value of the piece
// needs it, so the common case runs without per-value branches.
constexpr float kNegLog2e = -1.44269504088896341f;

__device__ __forceinline__ uint4 swiglu_piece(const uint4 gw, const uint4 uw) {
  float g[8], u[8], y[8], a[8];
  unpack_bf16x8(gw, g);
  unpack_bf16x8(uw, u);
  float amax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = g[e] * kNegLog2e;
    y[e] = g[e] * u[e] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a[e]));
    amax = fmaxf(amax, a[e]);
  }
  if (amax > 64.f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (a[e] > 64.f) {
        const float n = fminf(__builtin_floorf(a[e]), 320.f);
        y[e] = __builtin_amdgcn_ldexpf(g[e] * u[e] * __builtin_amdgcn_exp2f(n - a[e]), -(int)n);
      }
    }
  }
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y[0], (__bf16)y[1]});
  r.y = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y[2], (__bf16)y[3]});
  r.z = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y[4], (__bf16)y[5]});
  r.w = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)y[6], (__bf16)y[7]});
  return r;
}

// Row t = blockIdx.x; the row's I/8 pieces are cut into gridDim.y chunks of
// `chunk` pieces, and thread i of a workgroup takes pieces i and i + 256 of
// its chunk (no index division; all loads issued before any arithmetic).
__global__ void __launch_bounds__(kActThreads)
swiglu_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ gate_up, int I, int chunk) {
  const int n8 = I / 8;
  const int64_t t = blockIdx.x;
  const uint4* grow = reinterpret_cast<const uint4*>(gate_up + t * 2 * I);
  const uint4* urow = grow + n8;
  uint4* orow = reinterpret_cast<uint4*>(out + t * I);
  const int c0 = blockIdx.y * chunk;
  const int c_end = min(c0 + chunk, n8);
  uint4 g[kActPieces], u[kActPieces];
#pragma unroll
  for (int j = 0; j < kActPieces; ++j) {
    const int c = c0 + j * kActThreads + (int)threadIdx.x;
    if (c < c_end) {
      g[j] = load_stream16(grow + c);
      u[j] = load_stream16(urow + c);
    }
  }
#pragma unroll
  for (int j = 0; j < kActPieces; ++j) {
    const int c = c0 + j * kActThreads + (int)threadIdx.x;
    if (c < c_end) orow[c] = swiglu_piece(g[j], u[j]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(void* out, void* residual, const void* x, const void* weight, int T,
                          int H, float eps, hipStream_t stream) {
  const int n8 = H / 8;
  auto* o = static_cast<uint16_t*>(out);
  auto* r = static_cast<uint16_t*>(residual);
  const auto* xx = static_cast<const uint16_t*>(x);
  const auto* w = static_cast<const uint16_t*>(weight);
#define PA_NORM(PER)                                                                          \
  do {                                                                                        \
    if (r) hipLaunchKernelGGL((rmsnorm_kernel<PER, true>), dim3(T), dim3(kNormThreads), 0,   \
                              stream, o, r, xx, w, H, eps);                                   \
    else hipLaunchKernelGGL((rmsnorm_kernel<PER, false>), dim3(T), dim3(kNormThreads), 0,    \
                            stream, o, r, xx, w, H, eps);                                     \
  } while (0)
  if (n8 <= kNormThreads) PA_NORM(1);
  else if (n8 <= 2 * kNormThreads) PA_NORM(2);
  else if (n8 <= 4 * kNormThreads) PA_NORM(4);
  else PA_NORM(8);
#undef PA_NORM
  return hipGetLastError();
}

hipError_t launch_swiglu(void* out, const void* gate_up, int64_t T, int I, hipStream_t stream) {
  // balanced chunks of at most kActPieces * kActThreads pieces per row
  const int n8 = I / 8;
  const int per_wg = kActPieces * kActThreads;
  const int chunks = (n8 + per_wg - 1) / per_wg;
  const int chunk = (n8 + chunks - 1) / chunks;
  hipLaunchKernelGGL(swiglu_kernel, dim3((uint32_t)T, chunks), dim3(kActThreads), 0, stream,
                     static_cast<uint16_t*>(out), static_cast<const uint16_t*>(gate_up), I, chunk);
  return hipGetLastError();
}

}  // namespace pa
