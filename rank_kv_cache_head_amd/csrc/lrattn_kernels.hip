// gfx950 kernels for single-token decode attention over a per-head low-rank
// KV cache.
//
// Method: WSVD page, section 2.A (per-head latent times per-head factor) and
// section 2.C (one fused flow of low-rank rebuild, attention and Flash
// Decoding, intermediates on chip); AttentionPack page, section 2.C
// (decompression folded into the score computation).  The rebuild is folded
// by associativity: the partition kernel scores q~ . Lk[t] with
// q~ = scale * log2(e) * q . B_K^T and accumulates sum_t 2^(s_t - m) Lv[t] in
// the r-dimensional latent space; the combine kernel merges the partitions
// and applies B_V once per query head.  No K or V row ever exists.
//
// Work decomposition (Flash Decoding split of the token axis):
//   partition grid (P, Hkv, B), 256 threads = 4 wave64.  One workgroup owns
//   the tokens [p*S, min((p+1)*S, seq_len)) of one (b, kv-head) and all G
//   query heads of that kv-head, so each latent byte is read once for the
//   whole group.
//   combine grid (Hkv, B), 256 threads.
//
// Lane mapping inside a wave (the hot loop):
//   a latent row of r elements is kRowBytes bytes = kAct 16-byte pieces.
//   kLPR (= kAct rounded up to a power of two) consecutive lanes form a "slot"
//   that holds one row: lane cc of the slot loads bytes [16cc, 16cc+16).  A
//   wave holds kRPW = 64 / kLPR slots, so one 16-byte load instruction covers
//   kRPW consecutive rows = one contiguous span of memory.  Each slot runs its
//   own online softmax (running max m, exp-sum l, accumulator) over the rows
//   it sees; slots and waves are merged once, at the end of the partition.
//   The per-row dot product is summed across the slot's lanes with DPP
//   (quad_perm, row_half_mirror, row_mirror), which leaves the identical sum
//   in every lane of the slot.
#include <float.h>
#include <type_traits>

#include "lrattn_internal.hpp"

namespace lrattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ formats

struct LatF32 { static constexpr int kBytes = 4; };
struct LatBF16 { static constexpr int kBytes = 2; };
struct LatF16 { static constexpr int kBytes = 2; };
struct LatI8 { static constexpr int kBytes = 1; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// 16 bytes of latent row -> 16 / kBytes fp32 values (every conversion exact).
template <class LT> struct Unpack;
template <> struct Unpack<LatF32> {
  static __device__ __forceinline__ void run(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[k]);
  }
};
template <> struct Unpack<LatBF16> {
  static __device__ __forceinline__ void run(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = bf16_lo(v[k]); x[2 * k + 1] = bf16_hi(v[k]); }
  }
};
template <> struct Unpack<LatF16> {
  static __device__ __forceinline__ void run(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = f16_lo(v[k]); x[2 * k + 1] = f16_hi(v[k]); }
  }
};
template <> struct Unpack<LatI8> {
  static __device__ __forceinline__ void run(const u32x4& v, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * k + i] = (float)(int8_t)(v[k] >> (8 * i));
    }
  }
};

// One element of q or of a factor, runtime dtype (prologue / epilogue only).
__device__ __forceinline__ float load_elem(const void* p, size_t i, int dt) {
  if (dt == LRATTN_F32) return static_cast<const float*>(p)[i];
  const uint32_t h = static_cast<const uint16_t*>(p)[i];
  if (dt == LRATTN_BF16) return __uint_as_float(h << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Eight consecutive factor elements starting at element i (i % 8 == 0).
__device__ __forceinline__ void load8(const void* p, size_t i, int dt, float* x) {
  if (dt == LRATTN_F32) {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 a = f[0], b = f[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    return;
  }
  const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  if (dt == LRATTN_BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = bf16_lo(ww[k]); x[2 * k + 1] = bf16_hi(ww[k]); }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[2 * k] = f16_lo(ww[k]); x[2 * k + 1] = f16_hi(ww[k]); }
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------ buffer loads
// Raw buffer resources bound the partition's own rows: any load whose byte
// offset is at or past num_records returns zero and touches no memory, which
// makes the ragged tail and idle lanes branch-free and keeps padding unread.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: 32-bit data format, no swizzle, raw addressing.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
constexpr uint32_t kOffNone = 0x80000000u;  // beyond any partition: loads zero

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ partition

template <class LT, int R, int G>
struct Geo {
  static constexpr int kRowBytes = R * LT::kBytes;
  static constexpr int kEPL = 16 / LT::kBytes;            // elements per lane load
  static constexpr int kAct = kRowBytes / 16;             // lanes carrying a row
  static constexpr int kLPR = kAct <= 1 ? 1 : kAct <= 2 ? 2 : kAct <= 4 ? 4 : kAct <= 8 ? 8 : 16;
  static constexpr int kRPW = 64 / kLPR;                  // rows per wave load
  static constexpr int kU = G >= 4 ? 2 : 4;               // rows per slot per step
  static constexpr int kChunk = kU * kRPW;                // rows per wave per step
  static_assert(kRowBytes % 16 == 0, "latent row must be whole 16-byte pieces");
  static_assert(kAct <= 16, "latent row wider than 256 bytes");
};

template <class LT, int R, int G, bool kMask>
__device__ __forceinline__ void partition_step(
    int cb, int ntok, int slot, uint32_t lane_off,
    __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
    __amdgpu_buffer_rsrc_t rsk, __amdgpu_buffer_rsrc_t rsv,
    const float (&qt)[G][Geo<LT, R, G>::kEPL], float (&m)[G], float (&l)[G],
    float (&acc)[G][Geo<LT, R, G>::kEPL]) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, U = Gm::kU, RPW = Gm::kRPW;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  u32x4 kv[U], vv[U];
  float sk[U], sv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) kv[u] = bload16(rk, (uint32_t)(cb + u * RPW) * Gm::kRowBytes + lane_off);
#pragma unroll
  for (int u = 0; u < U; ++u) vv[u] = bload16(rv, (uint32_t)(cb + u * RPW) * Gm::kRowBytes + lane_off);
  if constexpr (kInt8) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t so = (uint32_t)(cb + u * RPW + slot) * 4u;
      sk[u] = bload4f(rsk, so);
      sv[u] = bload4f(rsv, so);
    }
  }

  // scores: s[u][h] = q~_h . Lk[row]   (base-2 logits)
  float s[U][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[EPL];
    Unpack<LT>::run(kv[u], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) t = fmaf(qt[h][e], x[e], t);
      t = group_sum<Gm::kLPR>(t);
      if constexpr (kInt8) t *= sk[u];
      if constexpr (kMask) {
        if (cb + u * RPW + slot >= ntok) t = -INFINITY;
      }
      s[u][h] = t;
    }
  }

  // online softmax per slot and head; w[u][h] = weight of row u
  float w[U][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = m[h];
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][h]);
    const float corr = fast_exp2(m[h] - mx);
    float es = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = fast_exp2(s[u][h] - mx);
      es += e;
      w[u][h] = kInt8 ? e * sv[u] : e;
    }
    l[h] = fmaf(l[h], corr, es);
    m[h] = mx;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] *= corr;
  }

  // latent-space value accumulation
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[EPL];
    Unpack<LT>::run(vv[u], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w[u][h], x[e], acc[h][e]);
    }
  }
}

template <class LT, int R, int G>
__global__ __launch_bounds__(kThreads) void partition_kernel(PartitionArgs a) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, LPR = Gm::kLPR, CH = Gm::kChunk;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int len = min(max(a.seq_lens[b], 0), a.T);
  const int t0 = p * a.S;
  const int t1 = min(t0 + a.S, len);
  if (t0 >= t1) return;  // partition past the sequence: nothing to write
  const int ntok = t1 - t0;

  __shared__ float q_lds[G * kMaxHeadDim];
  __shared__ float qt_lds[G * R];
  __shared__ float red_acc[kWaves * G * R];
  __shared__ float red_m[kWaves * G];
  __shared__ float red_l[kWaves * G];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, cc = lane % LPR;
  const bool colact = cc < Gm::kAct;

  const size_t bg = (size_t)b * a.Hkv + g;
  const size_t row0 = bg * (size_t)a.T + (size_t)t0;
  const uint32_t nbytes = (uint32_t)ntok * Gm::kRowBytes;
  const auto rk = make_rsrc(static_cast<const char*>(a.LK) + row0 * Gm::kRowBytes, nbytes);
  const auto rv = make_rsrc(static_cast<const char*>(a.LV) + row0 * Gm::kRowBytes, nbytes);
  __amdgpu_buffer_rsrc_t rsk = rk, rsv = rv;
  if constexpr (kInt8) {
    const size_t plane = (size_t)a.B * a.Hkv * a.T;
    rsk = make_rsrc(a.scales + row0, (uint32_t)ntok * 4u);
    rsv = make_rsrc(a.scales + plane + row0, (uint32_t)ntok * 4u);
  }
  const uint32_t lane_off = colact ? (uint32_t)(slot * Gm::kRowBytes + cc * 16) : kOffNone;

  // ---- absorption: q~[h][j] = qscale * sum_i q[h][i] * B_K[g][j][i]
  const int d = a.d;
  for (int i = tid; i < G * d; i += kThreads) {
    const int h = i / d, k = i - h * d;
    q_lds[h * kMaxHeadDim + k] =
        load_elem(a.q, ((size_t)b * a.Hq + (size_t)g * G + h) * d + k, a.q_dtype);
  }
  __syncthreads();
  const int nch = d >> 3;  // 8-element pieces per factor row; R * nch % 64 == 0
  for (int it = tid; it < R * nch; it += kThreads) {
    const int j = it / nch, c = it - j * nch;
    float f[8];
    load8(a.BK, ((size_t)g * R + j) * d + (size_t)c * 8, a.f_dtype, f);
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) t = fmaf(q_lds[h * kMaxHeadDim + c * 8 + k], f[k], t);
      part[h] = t;
    }
    for (int off = 1; off < nch; off <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] += __shfl_xor(part[h], off);
    }
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) qt_lds[h * R + j] = part[h] * a.qscale;
    }
  }
  __syncthreads();

  float qt[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qt[h][e] = colact ? qt_lds[h * R + cc * EPL + e] : 0.f;
  }

  // ---- stream the partition
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -FLT_MAX;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  for (int cb = wave * CH; cb < ntok; cb += kWaves * CH) {
    if (cb + CH <= ntok)
      partition_step<LT, R, G, false>(cb, ntok, slot, lane_off, rk, rv, rsk, rsv, qt, m, l, acc);
    else
      partition_step<LT, R, G, true>(cb, ntok, slot, lane_off, rk, rv, rsk, rsv, qt, m, l, acc);
  }

  // ---- merge the slots of this wave (lanes with equal cc)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = fast_exp2(m[h] - M);
    float L = l[h] * f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
    for (int off = LPR; off < 64; off <<= 1) {
      L += __shfl_xor(L, off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
    m[h] = M;
    l[h] = L;
  }
  if (slot == 0 && colact) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_acc[(wave * G + h) * R + cc * EPL + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[wave * G + h] = m[h];
      red_l[wave * G + h] = l[h];
    }
  }
  __syncthreads();

  // ---- merge the waves (fixed order) and write the partial record
  for (int it = tid; it < G * R; it += kThreads) {
    const int h = it / R, j = it - h * R;
    float M = red_m[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w * G + h]);
    float sacc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(red_m[w * G + h] - M);
      sacc = fmaf(f, red_acc[(w * G + h) * R + j], sacc);
      L = fmaf(f, red_l[w * G + h], L);
    }
    float* rec = a.ws + (((size_t)b * a.Hq + (size_t)g * G + h) * a.P + p) * (R + kRecPad);
    rec[j] = sacc;
    if (j == 0) {
      rec[R] = M;
      rec[R + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ combine

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

template <int G>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.r, RS = a.r + kRecPad;
  const int len = min(max(a.seq_lens[b], 0), a.T);
  const int np = (len + a.S - 1) / a.S;

  __shared__ float vt[G * kMaxRank];
  __shared__ float wmax[kWaves];
  __shared__ float wl[kWaves];
  __shared__ float wacc[kWaves * kMaxRank];

  const size_t out_row0 = ((size_t)b * a.Hq + (size_t)g * G) * a.d;
  if (np == 0) {  // no valid token: defined as a zero row
    for (int i = tid; i < G * a.d; i += kThreads) {
      if (a.out_dtype == LRATTN_F32) static_cast<float*>(a.out)[out_row0 + i] = 0.f;
      else static_cast<uint16_t*>(a.out)[out_row0 + i] = 0;
    }
    return;
  }

  for (int h = 0; h < G; ++h) {
    const float* base = a.ws + ((size_t)b * a.Hq + (size_t)g * G + h) * a.P * RS;
    float M = -FLT_MAX;
    for (int pp = tid; pp < np; pp += kThreads) M = fmaxf(M, base[(size_t)pp * RS + R]);
    M = wave_max(M);
    if (lane == 0) wmax[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

    float L = 0.f, v0 = 0.f, v1 = 0.f;
    for (int pp = wave; pp < np; pp += kWaves) {
      const float* rec = base + (size_t)pp * RS;
      const float f = fast_exp2(rec[R] - M);
      L = fmaf(f, rec[R + 1], L);
      if (lane < R) v0 = fmaf(f, rec[lane], v0);
      if (lane + 64 < R) v1 = fmaf(f, rec[lane + 64], v1);
    }
    if (lane == 0) wl[wave] = L;
    wacc[wave * kMaxRank + lane] = v0;
    wacc[wave * kMaxRank + 64 + lane] = v1;
    __syncthreads();
    if (tid < R) {
      const float Ls = ((wl[0] + wl[1]) + wl[2]) + wl[3];
      const float vs = ((wacc[tid] + wacc[kMaxRank + tid]) + wacc[2 * kMaxRank + tid]) +
                       wacc[3 * kMaxRank + tid];
      vt[h * kMaxRank + tid] = vs / Ls;
    }
    __syncthreads();
  }

  // out[b, g*G + h, i] = sum_j v~[h][j] * B_V[g][j][i]
  for (int i = tid; i < a.d; i += kThreads) {
    float o[G];
#pragma unroll
    for (int h = 0; h < G; ++h) o[h] = 0.f;
    for (int j = 0; j < R; ++j) {
      const float bv = load_elem(a.BV, ((size_t)g * R + j) * a.d + i, a.f_dtype);
#pragma unroll
      for (int h = 0; h < G; ++h) o[h] = fmaf(vt[h * kMaxRank + j], bv, o[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t oi = out_row0 + (size_t)h * a.d + i;
      if (a.out_dtype == LRATTN_F32) static_cast<float*>(a.out)[oi] = o[h];
      else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o[h]);
    }
  }
}

// ------------------------------------------------------------------ probes

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                              size_t n16, float* __restrict__ sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    x ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int off = 1; off < 64; off <<= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t s[kWaves];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = __uint_as_float(s[0] ^ s[1] ^ s[2] ^ s[3]);
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(u32x4* __restrict__ dst,
                                                              const u32x4* __restrict__ src,
                                                              size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// ------------------------------------------------------------ dispatch

template <class LT, int R>
hipError_t launch_pg(int group, const PartitionArgs& a, hipStream_t s) {
  const dim3 grid(a.P, a.Hkv, a.B), block(kThreads);
  switch (group) {
    case 1: hipLaunchKernelGGL((partition_kernel<LT, R, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((partition_kernel<LT, R, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((partition_kernel<LT, R, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((partition_kernel<LT, R, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class LT>
hipError_t launch_pr(int rank, int group, const PartitionArgs& a, hipStream_t s) {
  switch (rank) {
    case 16: return launch_pg<LT, 16>(group, a, s);
    case 32: return launch_pg<LT, 32>(group, a, s);
    case 48: return launch_pg<LT, 48>(group, a, s);
    case 64: return launch_pg<LT, 64>(group, a, s);
    case 128:
      if constexpr (LT::kBytes <= 2) return launch_pg<LT, 128>(group, a, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool partition_supported(int latent_dtype, int rank, int group) {
  int esz;
  switch (latent_dtype) {
    case LRATTN_F32: esz = 4; break;
    case LRATTN_BF16: case LRATTN_F16: esz = 2; break;
    case LRATTN_I8: esz = 1; break;
    default: return false;
  }
  const bool rank_ok = rank == 16 || rank == 32 || rank == 48 || rank == 64 || rank == 128;
  const bool group_ok = group == 1 || group == 2 || group == 4 || group == 8;
  return rank_ok && group_ok && rank * esz <= 256;
}

hipError_t launch_partition(int latent_dtype, int rank, int group, const PartitionArgs& a,
                            hipStream_t s) {
  switch (latent_dtype) {
    case LRATTN_F32: return launch_pr<LatF32>(rank, group, a, s);
    case LRATTN_BF16: return launch_pr<LatBF16>(rank, group, a, s);
    case LRATTN_F16: return launch_pr<LatF16>(rank, group, a, s);
    case LRATTN_I8: return launch_pr<LatI8>(rank, group, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(int group, const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.Hkv, a.B), block(kThreads);
  switch (group) {
    case 1: hipLaunchKernelGGL((combine_kernel<1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((combine_kernel<2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((combine_kernel<4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((combine_kernel<8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kThreads), 0, s,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace lrattn
