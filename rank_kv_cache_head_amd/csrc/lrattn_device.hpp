// Device helpers shared by the kernel sources: vector types, element
// conversions, bounded buffer loads, DPP lane reductions, exp2, and the exact
// three-term bf16 split.  Header-only, inline, gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ formats

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------ buffer loads
// Raw buffer resources bound a kernel's own rows: any load whose byte offset
// is at or past num_records returns zero and touches no memory, which makes
// ragged tails and idle lanes branch-free and keeps padding unread.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: 32-bit data format, no swizzle, raw addressing.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
constexpr uint32_t kOffNone = 0x80000000u;  // beyond any buffer: loads zero

// Hand-off of LDS data between the lanes of one wave: after the call, every
// lane sees the LDS stores the wave's lanes issued before it.  A wave's LDS
// instructions are performed in issue order, so no wait is needed; the
// wavefront-scope release/acquire fences and the wave barrier keep the
// compiler from moving LDS accesses across the point.  (HIP's __syncwarp
// has the same body.)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// -------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N a power of two <= 16); every lane of
// a group ends with the same bits (each step adds two commuted operands).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror: other quad of 8
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror: other half of 16
  return x;
}

// Maximum over aligned groups of 16 lanes (a DPP row); every lane of the row
// ends with it.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// Sum (maximum) over the lanes l, l ^ 16, l ^ 32 and l ^ 48, i.e. over the
// four 16-lane rows at one position, in the order (x_a + x_b) + (x_c + x_d)
// with a, b and c, d the pairs l ^ 16 joins; every lane of the four gets the
// same bits.
__device__ __forceinline__ float sum_quarters(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float max_quarters(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest base-2 logit excess over the running reference max before the
// reference is moved (weights stay <= 2^8).
constexpr float kLazyLog2 = 8.0f;

// ------------------------------------------------------ exact bf16 split
// Three bf16x8 operands holding the exact split of 8 fp32 values:
// x == hi + mid + lo, each term rounded to nearest even by the packed
// hardware conversion (v_cvt_pk_bf16_f32); each remainder is exact in fp32 and
// the last one has at most 8 significant bits, so lo takes it exactly.
__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}
__device__ __forceinline__ void split3x8(const float (&x)[8], bf16x8 (&t)[3]) {
  u32x4 w[3];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const bf16x2 h = cvt2(x[j], x[j + 1]);
    const float r0 = x[j] - (float)h[0], r1 = x[j + 1] - (float)h[1];
    const bf16x2 m = cvt2(r0, r1);
    const bf16x2 l = cvt2(r0 - (float)m[0], r1 - (float)m[1]);
    w[0][j / 2] = __builtin_bit_cast(uint32_t, h);
    w[1][j / 2] = __builtin_bit_cast(uint32_t, m);
    w[2][j / 2] = __builtin_bit_cast(uint32_t, l);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) t[k] = __builtin_bit_cast(bf16x8, w[k]);
}

}  // namespace lrattn
