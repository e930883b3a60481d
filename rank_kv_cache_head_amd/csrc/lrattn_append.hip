// gfx950 kernel of the append step: a new token's latent rows.
//
// WSVD page, section 2.A: each head's key (value) projection is factored per
// head, W_Kh = A_Kh . B_Kh, so a new token with hidden state x enters the
// cache as its latent x . A_Kh (r values); section 2.C stores such latents in
// low precision (int8 here, with one scale per token, kv-head and K / V).
//
// Two launches.  The partial kernel, one workgroup per (kv-head g, K or V,
// chunk z of D), forms the chunk's contribution to the rows of all B
// sequences: Lat_z (B x r) = X[:, chunk] . A_g[:, chunk]^T, A_g stored [r, D]
// (row j = the weights of latent coordinate j), on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}: exact products, fp32 sums).  Both operands
// load as 16 contiguous bytes per lane: lane l takes row l % 16 (a sequence
// of X, a latent coordinate of A) and elements 8 (l / 16) .. + 7 of each
// 32-wide step of D.  The four waves take a quarter of the chunk each; their
// tiles are added in LDS in wave order, and the chunk's rows go to the
// workspace.  The finish kernel, one workgroup per (g, K or V), adds the
// chunks in order z = 0, 1, ... (every order is fixed: bitwise reproducible)
// and converts each row to the latent type (round to nearest even), or
// quantizes it: s = max |row| / 127, code = rint(row / s) in fp32 (ties to
// even); rows are written at the sequence's position, and positions outside
// [0, T) are skipped.  Chunks are sized so the partial launch covers the chip
// (the step reads A once: a few MB that few workgroups cannot stream).
//
// Float latents need no row-wide quantity, so when there are enough
// (kv-head, K or V, 16-coordinate tile) triples to fill the chip they take
// one launch (append_direct_kernel): a workgroup of 16 waves per triple sums
// the whole of D for its tile.  Wave w takes the 32-wide steps w, w + 16, ...
// of D with four steps' loads in flight, the waves' tiles are added in LDS in
// wave order, and each thread rounds one (sequence, coordinate) and writes
// it.  Otherwise they take the two launches, as int8 latents always do.
#include <float.h>

#include "lrattn.h"
#include "lrattn_append.hpp"
#include "lrattn_device.hpp"

namespace lrattn {
namespace {

constexpr int kThreads = 256, kWaves = 4;

template <int R, int RB, bool kF16>
__global__ __launch_bounds__(kThreads) void append_partial_kernel(AppendArgs a) {
  constexpr int NT = R / 16;  // 16-column tiles of the latent row
  constexpr int U = 4;        // 32-wide steps of D whose loads are in flight together
  const int g = blockIdx.x, kv = blockIdx.y, z = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int D = a.D, B = a.B;

  __shared__ float red[RB * 16][R];

  const auto ra = make_rsrc(static_cast<const uint16_t*>(kv ? a.AV : a.AK) + (size_t)g * R * D,
                            (uint32_t)(R * D) * 2u);
  const auto rx = make_rsrc(a.x, (uint32_t)(B * D) * 2u);
  const int chunk = D / a.KS;           // a multiple of 128
  const int steps = chunk / (32 * kWaves);  // per wave
  const int kbeg = z * chunk + wave * steps * 32;

  f32x4 acc[RB][NT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int s0 = 0; s0 < steps; s0 += U) {
    u32x4 xf[U][RB], af[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < steps;
      const int k0 = kbeg + 32 * (s0 + u) + 8 * kg;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int b = 16 * rb + row;
        const uint32_t off = ok && b < B ? (uint32_t)(b * D + k0) * 2u : kOffNone;
        xf[u][rb] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t off = ok ? (uint32_t)((16 * t + row) * D + k0) * 2u : kOffNone;
        af[u][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (kF16)
            acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, xf[u][rb]), __builtin_bit_cast(f16x8, af[u][t]),
                acc[rb][t], 0, 0, 0);
          else
            acc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xf[u][rb]), __builtin_bit_cast(bf16x8, af[u][t]),
                acc[rb][t], 0, 0, 0);
        }
      }
    }
  }

  // waves' tiles added in wave order: lane l, register i holds
  // (sequence 16 rb + 4 (l / 16) + i, coordinate 16 t + l % 16)
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float& dst = red[16 * rb + 4 * kg + i][16 * t + row];
            dst = w == 0 ? acc[rb][t][i] : dst + acc[rb][t][i];
          }
        }
      }
    }
    __syncthreads();
  }
  float* part = a.ws + (((size_t)g * 2 + kv) * a.KS + z) * B * R;
  for (int e = tid; e < B * R; e += kThreads) part[e] = red[e / R][e % R];
}

// Rows [z RPB, (z + 1) RPB) of one (g, K or V): thread (row lb, coordinate j)
// adds its KS chunk partials in order z = 0, 1, ..., 16 loads in flight at a
// time (chunks past KS load zeros: adding +0 leaves every sum unchanged).
template <int R>
__global__ __launch_bounds__(kThreads) void append_finish_kernel(AppendArgs a) {
  constexpr int RPB = kThreads / R;  // rows per workgroup
  constexpr int Z = 16;
  const int g = blockIdx.x, kv = blockIdx.y;
  const int tid = threadIdx.x;
  const int lb = tid / R, j = tid - lb * R;
  const int b = blockIdx.z * RPB + lb;
  const int B = a.B, KS = a.KS;
  const bool active = lb < RPB && b < B;
  __shared__ float rows[RPB * R];
  __shared__ float rscale[RPB];

  const auto rp = make_rsrc(a.ws + ((size_t)g * 2 + kv) * KS * B * R, (uint32_t)(KS * B * R) * 4u);
  const uint32_t e = (uint32_t)(b * R + j);
  float v = 0.f;
  for (int z0 = 0; z0 < KS; z0 += Z) {
    float t[Z];
#pragma unroll
    for (int u = 0; u < Z; ++u) {
      const uint32_t off = active && z0 + u < KS ? ((uint32_t)(z0 + u) * B * R + e) * 4u : kOffNone;
      t[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, (int)off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < Z; ++u) v = z0 + u == 0 ? t[u] : v + t[u];
  }
  if (lb < RPB) rows[tid] = v;
  __syncthreads();
  const bool int8 = a.latent_dtype == LRATTN_I8;
  const int p = active ? a.positions[b] : -1;
  if (int8 && active && j == 0) {
    float m = 0.f;
    for (int k = 0; k < R; ++k) m = fmaxf(m, fabsf(rows[lb * R + k]));
    const float sc = m / 127.0f;
    rscale[lb] = sc;
    if (p >= 0 && p < a.T) a.scales[(((size_t)kv * B + b) * a.Hkv + g) * a.T + p] = sc;
  }
  __syncthreads();
  if (!active || p < 0 || p >= a.T) return;
  void* L = kv ? a.LV : a.LK;
  const size_t off = (((size_t)b * a.Hkv + g) * a.T + p) * R + j;
  switch (a.latent_dtype) {
    case LRATTN_F32: static_cast<float*>(L)[off] = v; break;
    case LRATTN_BF16: static_cast<__bf16*>(L)[off] = (__bf16)v; break;
    case LRATTN_F16: static_cast<_Float16*>(L)[off] = (_Float16)v; break;
    default: {
      const float sc = rscale[lb];
      const float c = sc > 0.f ? fminf(fmaxf(rintf(v / sc), -127.f), 127.f) : 0.f;
      static_cast<int8_t*>(L)[off] = (int8_t)c;
    }
  }
}

constexpr int kDirectWaves = 16;


template <int R, int RB, bool kF16>
__global__ __launch_bounds__(64 * kDirectWaves) void append_direct_kernel(AppendArgs a) {
  constexpr int U = 4;  // steps of D whose loads are in flight together
  const int g = blockIdx.x, kv = blockIdx.y, c = blockIdx.z;  // c: 16-coordinate tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int D = a.D, B = a.B, steps = D / 32;

  __shared__ float part[kDirectWaves][RB * 16][16];

  const auto ra = make_rsrc(static_cast<const uint16_t*>(kv ? a.AV : a.AK) + (size_t)g * R * D,
                            (uint32_t)(R * D) * 2u);
  const auto rx = make_rsrc(a.x, (uint32_t)(B * D) * 2u);
  f32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; wave + kDirectWaves * i0 < steps; i0 += U) {
    u32x4 xf[U][RB], af[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = wave + kDirectWaves * (i0 + u);
      const bool ok = st < steps;
      const int k0 = 32 * st + 8 * kg;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int b = 16 * rb + row;
        const uint32_t off = ok && b < B ? (uint32_t)(b * D + k0) * 2u : kOffNone;
        xf[u][rb] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
      }
      const uint32_t off = ok ? (uint32_t)((16 * c + row) * D + k0) * 2u : kOffNone;
      af[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (kF16)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, xf[u][rb]),
                                                           __builtin_bit_cast(f16x8, af[u]),
                                                           acc[rb], 0, 0, 0);
        else
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf[u][rb]),
                                                            __builtin_bit_cast(bf16x8, af[u]),
                                                            acc[rb], 0, 0, 0);
      }
    }
  }
  // lane l, register i: (sequence 16 rb + 4 (l / 16) + i, coordinate 16 c + l % 16)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][16 * rb + 4 * kg + i][row] = acc[rb][i];
  }
  __syncthreads();
  // thread (sequence tid / 16, coordinate tid % 16): the waves' sums in order
  const int b = tid >> 4, j = tid & 15;
  if (b >= B) return;
  float v = part[0][b][j];
#pragma unroll
  for (int w = 1; w < kDirectWaves; ++w) v += part[w][b][j];
  const int p = a.positions[b];
  if (p < 0 || p >= a.T) return;
  void* L = kv ? a.LV : a.LK;
  const size_t off = (((size_t)b * a.Hkv + g) * a.T + p) * R + 16 * c + j;
  switch (a.latent_dtype) {
    case LRATTN_F32: static_cast<float*>(L)[off] = v; break;
    case LRATTN_BF16: static_cast<__bf16*>(L)[off] = (__bf16)v; break;
    default: static_cast<_Float16*>(L)[off] = (_Float16)v; break;
  }
}

template <int R, bool kF16>
hipError_t launch_r(const AppendArgs& a, hipStream_t s) {
  if (append_direct(a.latent_dtype, a.Hkv, R)) {
    const dim3 grid(a.Hkv, 2, R / 16), block(64 * kDirectWaves);
    switch ((a.B + 15) / 16) {
      case 1: hipLaunchKernelGGL((append_direct_kernel<R, 1, kF16>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((append_direct_kernel<R, 2, kF16>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((append_direct_kernel<R, 3, kF16>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((append_direct_kernel<R, 4, kF16>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid(a.Hkv, 2, a.KS), block(kThreads);
  switch ((a.B + 15) / 16) {
    case 1: hipLaunchKernelGGL((append_partial_kernel<R, 1, kF16>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((append_partial_kernel<R, 2, kF16>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((append_partial_kernel<R, 3, kF16>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((append_partial_kernel<R, 4, kF16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = kThreads / R;
  hipLaunchKernelGGL((append_finish_kernel<R>), dim3(a.Hkv, 2, (a.B + RPB - 1) / RPB), block, 0,
                     s, a);
  return hipGetLastError();
}

template <bool kF16>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  switch (a.r) {
    case 16: return launch_r<16, kF16>(a, s);
    case 32: return launch_r<32, kF16>(a, s);
    case 48: return launch_r<48, kF16>(a, s);
    case 64: return launch_r<64, kF16>(a, s);
    case 128: return launch_r<128, kF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The one-launch path streams A through only Hkv * 2 * r / 16 workgroups, each
// reading all of x: it pays off once those cover most of the chip.  Measured
// per call: ragged (240 workgroups) 9.4 us against 11.7 on two launches;
// gqa_vlm (64) 8.8 against 7.5, llm7b (128) 7.6 against 6.6.
constexpr int kDirectMinBlocks = 192;

bool append_direct(int latent_dtype, int hkv, int r) {
  return latent_dtype != LRATTN_I8 && (int64_t)hkv * 2 * (r / 16) >= kDirectMinBlocks;
}

bool append_supported(int rank, int batch, int model_dim) {
  const bool r_ok = rank == 16 || rank == 32 || rank == 48 || rank == 64 || rank == 128;
  return r_ok && batch >= 1 && batch <= kAppendMaxBatch && model_dim >= 128 &&
         model_dim % 128 == 0 && (int64_t)rank * model_dim * 2 < (int64_t(1) << 31) &&
         (int64_t)batch * model_dim * 2 < (int64_t(1) << 31);
}

int append_chunks(int num_kv_heads, int model_dim) {
  const int pieces = model_dim / 128;  // the finest chunking
  int ks = (512 + 2 * num_kv_heads - 1) / (2 * num_kv_heads);
  if (ks > pieces) ks = pieces;
  if (ks < 1) ks = 1;
  while (pieces % ks) --ks;  // chunks divide D into multiples of 128
  return ks;
}

size_t append_workspace_bytes(int num_kv_heads, int batch, int rank, int chunks) {
  const size_t b = (size_t)num_kv_heads * 2 * chunks * batch * rank * 4;
  return (b + 255) / 256 * 256;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  return a.x_dtype == LRATTN_F16 ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace lrattn
