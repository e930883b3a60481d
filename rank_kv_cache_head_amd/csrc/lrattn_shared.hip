// gfx950 kernel of the shared-latent decode's first step: q~ per query head.
//
// AttentionPack page, section 2.A: the keys of all heads are factored
// together, so the cache holds one compressed row per token shared by the
// heads, and head h rebuilds its keys with its own block B_K[h] (r x d) of
// the decompression matrix.  The absorbed query of head h is therefore
// q~_h = qscale * q_h . B_K[h]^T, one product per head (the grouped path's
// single product per kv-head does not apply), formed here once per decode
// step; the partition kernels then read it instead of absorbing.
//
// Grid (Hq, sequence blocks of 8); thread (coordinate j, block row s) forms
// q~ for sequences s, s + 256 / r, ... of the block: the factor row B_K[h][j]
// is streamed once per thread in 8-element pieces and reused across those
// sequences; the query rows sit in LDS.  Every product is exact in fp32 and
// the sums run over i in increasing order.
#include "lrattn.h"
#include "lrattn_internal.hpp"

namespace lrattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float elem(const void* p, size_t i, int dt) {
  if (dt == LRATTN_F32) return static_cast<const float*>(p)[i];
  const uint32_t h = static_cast<const uint16_t*>(p)[i];
  if (dt == LRATTN_BF16) return __uint_as_float(h << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int R>
__global__ __launch_bounds__(kThreads) void absorb_heads_kernel(AbsorbHeadsArgs a) {
  constexpr int SB = 8;          // sequences per workgroup
  constexpr int TPJ = kThreads / R;  // threads per latent coordinate
  constexpr int KPT = (SB + TPJ - 1) / TPJ;  // sequences per thread
  const int h = blockIdx.x, b0 = blockIdx.y * SB;
  const int tid = threadIdx.x, j = tid % R, s0 = tid / R;
  const int d = a.d;
  __shared__ float qs[SB][kMaxHeadDim];
  for (int e = tid; e < SB * d; e += kThreads) {
    const int s = e / d, i = e - s * d, b = b0 + s;
    qs[s][i] = b < a.B ? elem(a.q, ((size_t)b * a.Hq + h) * d + i, a.q_dtype) : 0.f;
  }
  __syncthreads();
  if (s0 >= TPJ) return;  // r = 48: 16 threads without a coordinate
  float acc[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) acc[k] = 0.f;
  const size_t row = ((size_t)h * R + j) * d;
  for (int i0 = 0; i0 < d; i0 += 8) {
    float f[8];
    if (a.f_dtype == LRATTN_F32) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.BK) + row + i0);
      const float4 y =
          *reinterpret_cast<const float4*>(static_cast<const float*>(a.BK) + row + i0 + 4);
      f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
      f[4] = y.x; f[5] = y.y; f[6] = y.z; f[7] = y.w;
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.BK) + row + i0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (a.f_dtype == LRATTN_BF16) {
          f[2 * k] = __uint_as_float(w[k] << 16);
          f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        } else {
          f[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xffffu));
          f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int s = s0 + k * TPJ;
      if (s < SB) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k] = fmaf(qs[s][i0 + e], f[e], acc[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int s = s0 + k * TPJ, b = b0 + s;
    if (s < SB && b < a.B) a.qt[((size_t)b * a.Hq + h) * R + j] = acc[k] * a.qscale;
  }
}

template <int R>
hipError_t launch_r(const AbsorbHeadsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((absorb_heads_kernel<R>), dim3(a.Hq, (a.B + 7) / 8), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_heads(const AbsorbHeadsArgs& a, hipStream_t s) {
  switch (a.r) {
    case 16: return launch_r<16>(a, s);
    case 32: return launch_r<32>(a, s);
    case 48: return launch_r<48>(a, s);
    case 64: return launch_r<64>(a, s);
    case 128: return launch_r<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrattn
