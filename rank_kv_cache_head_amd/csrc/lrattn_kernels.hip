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
//   combine grid (Hq, B), 256 threads.
//
// Lane mapping inside a wave (the hot loop):
//   a latent row of r elements is kRowBytes bytes = kAct pieces of kVec bytes
//   (16, or 8 for int8 latents with 4+ heads).  kLPR (= kAct rounded up to a
//   power of two) consecutive lanes form a "slot" that holds one row: lane cc
//   of the slot loads bytes [kVec*cc, kVec*(cc+1)).  A wave holds
//   kRPW = 64 / kLPR slots, so one load instruction covers kRPW consecutive
//   rows = one contiguous span of memory.  Each slot runs its own online
//   softmax (reference max m, exp-sum l, accumulator) over the rows it sees;
//   slots and waves are merged once, at the end of the partition.
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

// kWords 32-bit words of a latent row -> fp32 values (every conversion exact).
template <class LT> struct Unpack;
template <> struct Unpack<LatF32> {
  template <int kWords>
  static __device__ __forceinline__ void run(const uint32_t (&w)[kWords], float* x) {
#pragma unroll
    for (int k = 0; k < kWords; ++k) x[k] = __uint_as_float(w[k]);
  }
};
template <> struct Unpack<LatBF16> {
  template <int kWords>
  static __device__ __forceinline__ void run(const uint32_t (&w)[kWords], float* x) {
#pragma unroll
    for (int k = 0; k < kWords; ++k) { x[2 * k] = bf16_lo(w[k]); x[2 * k + 1] = bf16_hi(w[k]); }
  }
};
template <> struct Unpack<LatF16> {
  template <int kWords>
  static __device__ __forceinline__ void run(const uint32_t (&w)[kWords], float* x) {
#pragma unroll
    for (int k = 0; k < kWords; ++k) { x[2 * k] = f16_lo(w[k]); x[2 * k + 1] = f16_hi(w[k]); }
  }
};
template <> struct Unpack<LatI8> {
  template <int kWords>
  static __device__ __forceinline__ void run(const uint32_t (&w)[kWords], float* x) {
#pragma unroll
    for (int k = 0; k < kWords; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * k + i] = (float)(int8_t)(w[k] >> (8 * i));
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

// Largest base-2 logit excess over the running reference max before the
// reference is moved (weights stay <= 2^8).
constexpr float kLazyLog2 = 8.0f;

// ------------------------------------------------------------ partition
// Compile-time tuning knobs (ordinary parameters; every setting computes the
// same result):
//   LRATTN_UNROLL_SMALL_G  rows per slot per step, 1-2 heads, 2- and 4-byte latents
//   LRATTN_UNROLL_LARGE_G  rows per slot per step, 4-8 heads
//   LRATTN_UNROLL_I8       rows per slot per step, 1-2 heads, int8 latents
//   LRATTN_PREFETCH        1: load step i+1 while step i computes
//   LRATTN_LOAD_AUX        cache-policy bits of the streaming latent loads;
//                          2 = non-temporal: each latent byte is used once, so
//                          it should not displace reusable lines in L2
#ifndef LRATTN_UNROLL_SMALL_G
#define LRATTN_UNROLL_SMALL_G 4
#endif
#ifndef LRATTN_UNROLL_LARGE_G
#define LRATTN_UNROLL_LARGE_G 2
#endif
#ifndef LRATTN_UNROLL_I8
#define LRATTN_UNROLL_I8 2
#endif
#ifndef LRATTN_PREFETCH
#define LRATTN_PREFETCH 0
#endif
#ifndef LRATTN_LOAD_AUX
#define LRATTN_LOAD_AUX 2
#endif


template <class LT, int R, int G>
struct Geo {
  static constexpr int kRowBytes = R * LT::kBytes;
  // bytes per lane load: 16, or 8 for int8 latents with 4+ heads, whose 16
  // values per lane would need 32+ registers per head for q~ and accumulators
  static constexpr int kVec = (LT::kBytes == 1 && G >= 4 && kRowBytes >= 16) ? 8 : 16;
  static constexpr int kWords = kVec / 4;
  static constexpr int kEPL = kVec / LT::kBytes;          // elements per lane load
  static constexpr int kAct = kRowBytes / kVec;           // lanes carrying a row
  static constexpr int kLPR = kAct <= 1 ? 1 : kAct <= 2 ? 2 : kAct <= 4 ? 4 : kAct <= 8 ? 8 : 16;
  static constexpr int kRPW = 64 / kLPR;                  // rows per wave load
  // q~ and the accumulators take kEPL * G registers each; when that reaches
  // 128 (int8 latents with 8 heads) q~ is read from LDS in the score loop
  // instead of being held in registers, and one row per slot is processed
  // per step.
  static constexpr bool kQtInLds = kEPL * G >= 128;
  static constexpr int kU = kQtInLds ? 1
                           : G >= 4 ? LRATTN_UNROLL_LARGE_G
                           : (LT::kBytes == 1 ? LRATTN_UNROLL_I8 : LRATTN_UNROLL_SMALL_G);
  static constexpr int kChunk = kU * kRPW;                // rows per wave per step
  // Occupancy target (waves per SIMD) the register allocation must meet:
  // 4 (<= 128 VGPRs) unless q~ plus accumulators alone need more than 64.
  static constexpr int kWavesPerEU =
      (kEPL * G <= 16 && kEPL * G * kU <= 32) || (kEPL * G <= 32 && R >= 64) ? 4 : 2;
  static_assert(kRowBytes % 16 == 0, "latent row must be whole 16-byte pieces");
  static_assert(kAct <= 16, "latent row wider than 16 lane loads");
};

// One lane load of kWords 32-bit words (16 or 8 bytes), streaming cache policy.
template <int kWords>
__device__ __forceinline__ void load_words(uint32_t (&w)[kWords], __amdgpu_buffer_rsrc_t r,
                                           uint32_t off) {
  if constexpr (kWords == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, LRATTN_LOAD_AUX);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, LRATTN_LOAD_AUX);
    w[0] = v[0]; w[1] = v[1];
  }
}

// The latent data of one step of one wave: kU rows per slot of K and of V
// (and their int8 scales).
template <class LT, int R, int G>
struct Step {
  uint32_t k[Geo<LT, R, G>::kU][Geo<LT, R, G>::kWords];
  uint32_t v[Geo<LT, R, G>::kU][Geo<LT, R, G>::kWords];
  float sk[Geo<LT, R, G>::kU];
  float sv[Geo<LT, R, G>::kU];
};

template <class LT, int R, int G>
__device__ __forceinline__ void load_step(Step<LT, R, G>& st, int cb, int slot, uint32_t lane_off,
                                          __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          __amdgpu_buffer_rsrc_t rsk, __amdgpu_buffer_rsrc_t rsv) {
  using Gm = Geo<LT, R, G>;
  constexpr int U = Gm::kU, RPW = Gm::kRPW;
#pragma unroll
  for (int u = 0; u < U; ++u)
    load_words<Gm::kWords>(st.k[u], rk, (uint32_t)(cb + u * RPW) * Gm::kRowBytes + lane_off);
#pragma unroll
  for (int u = 0; u < U; ++u)
    load_words<Gm::kWords>(st.v[u], rv, (uint32_t)(cb + u * RPW) * Gm::kRowBytes + lane_off);
  if constexpr (std::is_same<LT, LatI8>::value) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t so = (uint32_t)(cb + u * RPW + slot) * 4u;
      st.sk[u] = bload4f(rsk, so);
      st.sv[u] = bload4f(rsv, so);
    }
  }
}

// q~ of this lane's columns: registers, or (kQtInLds) LDS rows of stride R.
template <class LT, int R, int G>
struct QtView {
  static constexpr bool kLds = Geo<LT, R, G>::kQtInLds;
  float reg[kLds ? 1 : G][Geo<LT, R, G>::kEPL];
  const float* lds;  // &qt_lds[cc * kEPL]
  __device__ __forceinline__ float at(int h, int e) const {
    if constexpr (kLds) return lds[h * R + e];
    else return reg[h][e];
  }
};

template <class LT, int R, int G, bool kMask>
__device__ __forceinline__ void compute_step(
    const Step<LT, R, G>& st, int cb, int ntok, int slot, const QtView<LT, R, G>& qt,
    float (&m)[G], float (&l)[G], float (&acc)[G][Geo<LT, R, G>::kEPL]) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, U = Gm::kU, RPW = Gm::kRPW;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  // scores: s[u][h] = q~_h . Lk[row]   (base-2 logits)
  float s[U][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[EPL];
    Unpack<LT>::run(st.k[u], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) t = fmaf(qt.at(h, e), x[e], t);
      t = group_sum<Gm::kLPR>(t);
      if constexpr (kInt8) t *= st.sk[u];
      if constexpr (kMask) {
        if (cb + u * RPW + slot >= ntok) t = -INFINITY;
      }
      s[u][h] = t;
    }
  }

  // online softmax per slot and head, with a lazily moved reference max: the
  // running reference m only moves when a score exceeds it by more than
  // kLazyLog2 (base-2 logits), so weights 2^(s - m) stay <= 2^kLazyLog2 and
  // the accumulator rescale (and its exp) is skipped unless some lane of the
  // wave needs it.  Any reference gives the same result: the record stores m
  // with the sums taken relative to it.
  float mx[G];
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = s[0][h];
#pragma unroll
    for (int u = 1; u < U; ++u) mx[h] = fmaxf(mx[h], s[u][h]);
    need |= mx[h] > m[h] + kLazyLog2;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {  // wave-uniform
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float nm = mx[h] > m[h] + kLazyLog2 ? mx[h] : m[h];
      const float corr = fast_exp2(m[h] - nm);
      l[h] *= corr;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= corr;
      m[h] = nm;
    }
  }
  float w[U][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float es = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = fast_exp2(s[u][h] - m[h]);
      es += e;
      w[u][h] = kInt8 ? e * st.sv[u] : e;
    }
    l[h] += es;
  }

  // latent-space value accumulation
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[EPL];
    Unpack<LT>::run(st.v[u], x);
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w[u][h], x[e], acc[h][e]);
    }
  }
}

// Sum of `x` over aligned groups of n lanes, n in {8, 16, 32} (runtime, uniform).
__device__ __forceinline__ float piece_sum(float x, int n) {
  if (n <= 8) return group_sum<8>(x);
  x = group_sum<16>(x);
  if (n > 16) x += __shfl_xor(x, 16);
  return x;
}

// ------------------------------------------------------------------ merge

// Zero rows for a sequence with no valid token (attention over no tokens is
// defined as a zero output).
__device__ __forceinline__ void write_zero_rows(const MergeArgs& mg, size_t out_row0, int n) {
  for (int i = threadIdx.x; i < n; i += kThreads) {
    if (mg.out_dtype == LRATTN_F32) static_cast<float*>(mg.out)[out_row0 + i] = 0.f;
    else static_cast<uint16_t*>(mg.out)[out_row0 + i] = 0;
  }
}

// ------------------------------------------------------------ partition kernel

template <int R, int G>
struct PartLds {
  float q[G * kMaxHeadDim];
  float qt[G * R];
  float acc[kWaves * G * R];
  float m[kWaves * G];
  float l[kWaves * G];
};

template <class LT, int R, int G>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Geo<LT, R, G>::kWavesPerEU)))
void partition_kernel(PartitionArgs a) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, LPR = Gm::kLPR, CH = Gm::kChunk;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // seq_lens[b] is one value for the whole workgroup; keeping it in a scalar
  // register keeps the buffer descriptors below scalar (a descriptor the
  // compiler must treat as per-lane costs a readfirstlane loop per load)
  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  const int t0 = p * a.S;
  const int t1 = min(t0 + a.S, len);
  if (t0 >= t1) return;  // partition past the sequence: nothing to write
  const int ntok = t1 - t0;

  __shared__ PartLds<R, G> lds;
  float* q_lds = lds.q;
  float* qt_lds = lds.qt;

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
  const uint32_t lane_off = colact ? (uint32_t)(slot * Gm::kRowBytes + cc * Gm::kVec) : kOffNone;

  // The first step's latents are requested before the prologue, so their
  // latency overlaps the absorption instead of following it.
  Step<LT, R, G> cur;
  load_step(cur, wave * CH, slot, lane_off, rk, rv, rsk, rsv);

  // ---- absorption: q~[h][j] = qscale * sum_i q[h][i] * B_K[g][j][i]
  // All q and B_K loads of a thread are issued before any is used (one
  // memory round trip); the G*d query values are contiguous.
  const int d = a.d;
  {
    constexpr int kQPer = (G * kMaxHeadDim + kThreads - 1) / kThreads;
    const size_t q0 = ((size_t)b * a.Hq + (size_t)g * G) * d;
    float qv[kQPer];
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = tid + k * kThreads;
      qv[k] = i < G * d ? load_elem(a.q, q0 + i, a.q_dtype) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = tid + k * kThreads;
      if (i < G * d) {
        const int h = i / d;
        q_lds[h * kMaxHeadDim + (i - h * d)] = qv[k];
      }
    }
  }
  __syncthreads();
  const int nch = d >> 3;  // 8-element pieces per factor row; R * nch % 64 == 0
  // pieces per thread whose loads are in flight together: all of them for
  // d = 128 and r <= 64
  constexpr int kPieceBatch = R / 16 < 4 ? R / 16 : 4;
  for (int base = 0; base < R * nch; base += kPieceBatch * kThreads) {
    float f[kPieceBatch][8];
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) {
      const int it = base + tid + k * kThreads;
      if (it < R * nch) {
        const int j = it / nch, c = it - j * nch;
        load8(a.BK, ((size_t)g * R + j) * d + (size_t)c * 8, a.f_dtype, f[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) {
      const int it = base + k * kThreads + (tid & ~63);  // wave-uniform guard
      if (it < R * nch) {
        const int itl = it + lane;
        const int j = itl / nch, c = itl - j * nch;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) t = fmaf(q_lds[h * kMaxHeadDim + c * 8 + e], f[k][e], t);
          t = piece_sum(t, nch);
          if (c == 0) qt_lds[h * R + j] = t * a.qscale;
        }
      }
    }
  }
  __syncthreads();

  QtView<LT, R, G> qt;
  // idle lanes (cc >= kAct) load zeros, so their q~ is never read
  qt.lds = qt_lds + (colact ? cc * EPL : 0);
  if constexpr (!QtView<LT, R, G>::kLds) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qt.reg[h][e] = colact ? qt_lds[h * R + cc * EPL + e] : 0.f;
    }
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
    Step<LT, R, G> nxt;
    if constexpr (LRATTN_PREFETCH) {
      // double buffering: step i+1 is in flight while step i computes; past
      // the partition the loads return zero without touching memory
      load_step(nxt, cb + kWaves * CH, slot, lane_off, rk, rv, rsk, rsv);
    }
    if (cb + CH <= ntok)
      compute_step<LT, R, G, false>(cur, cb, ntok, slot, qt, m, l, acc);
    else
      compute_step<LT, R, G, true>(cur, cb, ntok, slot, qt, m, l, acc);
    if constexpr (LRATTN_PREFETCH) {
      cur = nxt;
    } else {
      load_step(cur, cb + kWaves * CH, slot, lane_off, rk, rv, rsk, rsv);
    }
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
  float* red_acc = lds.acc;
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
      lds.m[wave * G + h] = m[h];
      lds.l[wave * G + h] = l[h];
    }
  }
  __syncthreads();

  // ---- merge the waves (fixed order) and write the partial record
  float* const rec0 = a.ws + ((size_t)b * a.Hq + (size_t)g * G) * (size_t)a.P * (R + kRecPad);
  for (int it = tid; it < G * R; it += kThreads) {
    const int h = it / R, j = it - h * R;
    float M = lds.m[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds.m[w * G + h]);
    float sacc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(lds.m[w * G + h] - M);
      sacc = fmaf(f, red_acc[(w * G + h) * R + j], sacc);
      L = fmaf(f, lds.l[w * G + h], L);
    }
    float* rec = rec0 + ((size_t)h * a.P + p) * (R + kRecPad);
    rec[j] = sacc;
    if (j == 0) {
      rec[R] = M;
      rec[R + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ combine
// Second kernel of the decode step: one workgroup per (b, query head) merges
// that head's partial records and projects through B_V.  The kernel boundary
// is what makes every partition's records visible to it: on this multi-XCD
// part an in-kernel hand-off (last-arriving workgroup merges) needs an
// agent-scope fence per workgroup, i.e. an L2 writeback each, which measured
// several times slower than the second launch.
//
// The kernel is latency-bound, so every load is issued as early as possible
// and dependency chains are kept short:
//   1. each thread loads its slice of B_V[g] (column i = tid % d, row block
//      jb = tid / d of NB = kThreads / d blocks) before anything else;
//   2. the head's records are staged into LDS with 16-byte loads, all issued
//      together (one round trip per chunk of partitions);
//   3. thread (pg, j) folds coordinate j over partitions pg, pg + NPG, ...
//      in ascending order (online log-sum-exp rule; NPG = kThreads / r
//      groups shorten the chain), then the NPG groups are folded in
//      ascending order: v~ = acc / l;
//   4. thread (jb, i) forms the row-block partial of v~ . B_V[g][:, i] and
//      the NB partials are added in ascending order.
// Every order is fixed, so results are bitwise reproducible.

template <int R>
struct CombineLds {
  static constexpr int kNPG = kThreads / R;                 // partition groups
  static constexpr int kStage = 4096;                       // staged floats
  static constexpr int kChunk = kStage / (R + kRecPad);     // partitions per chunk
  float4 stage[kStage / 4];
  float m[kNPG * R];
  float l[kNPG * R];
  float v[kNPG * R];
  float vt[R];
  float part[kThreads];  // [jb][i], NB * d == kThreads
};

template <int R>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void combine_kernel(CombineArgs a) {
  using CL = CombineLds<R>;
  constexpr int RS = R + kRecPad;
  constexpr int kNPG = CL::kNPG, kChunk = CL::kChunk;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int g = hq / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const int d = a.d;
  const MergeArgs& mg = a.merge;

  // 1. B_V slice: rows [jb * RB, (jb + 1) * RB) of column i
  const int NB = kThreads / d;  // d in {64, 128, 256}
  const int RB = R / NB;
  const int i_col = tid % d, jb = tid / d;
  float bv[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    bv[k] = 0.f;
    if (k < RB)
      bv[k] = load_elem(mg.BV, ((size_t)g * R + jb * RB + k) * d + i_col, mg.f_dtype);
  }

  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  const int np = (len + a.S - 1) / a.S;
  const size_t out_row0 = ((size_t)b * a.Hq + hq) * d;
  if (np == 0) {
    write_zero_rows(mg, out_row0, d);
    return;
  }

  __shared__ CL sm;
  const float* stage = reinterpret_cast<const float*>(sm.stage);
  const float* rec0 = a.ws + ((size_t)b * a.Hq + hq) * (size_t)a.P * RS;
  // kNPG * R <= kThreads (r = 48 leaves 16 threads without a group)
  const int pg = tid / R, j = tid - pg * R;
  const bool folds = pg < kNPG;
  float m = -FLT_MAX, L = 0.f, acc = 0.f;
  for (int p0 = 0; p0 < np; p0 += kChunk) {
    const int n4 = min(kChunk, np - p0) * RS / 4;  // float4 in this chunk
    if (p0 > 0) __syncthreads();                   // previous chunk consumed
    // 2. stage: every load of a thread is issued before the first LDS store
    constexpr int kPer = CL::kStage / 4 / kThreads;
    float4 v4[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kThreads;
      v4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < n4) v4[k] = reinterpret_cast<const float4*>(rec0 + (size_t)p0 * RS)[i];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid + k * kThreads;
      if (i < n4) sm.stage[i] = v4[k];
    }
    __syncthreads();
    // 3. fold this chunk's partitions pg, pg + NPG, ...
    const int pc = folds ? min(kChunk, np - p0) : 0;
    for (int pp = pg; pp < pc; pp += kNPG) {
      const float* rec = stage + pp * RS;
      const float mp = rec[R];
      const float nm = fmaxf(m, mp);
      const float fa = fast_exp2(m - nm), fb = fast_exp2(mp - nm);
      L = fmaf(L, fa, rec[R + 1] * fb);
      acc = fmaf(acc, fa, rec[j] * fb);
      m = nm;
    }
  }
  if (folds) {
    sm.m[tid] = m;
    sm.l[tid] = L;
    sm.v[tid] = acc;
  }
  __syncthreads();
  if (tid < R) {
#pragma unroll
    for (int q = 1; q < kNPG; ++q) {
      const int item = q * R + tid;
      const float mp = sm.m[item];
      const float nm = fmaxf(m, mp);
      const float fa = fast_exp2(m - nm), fb = fast_exp2(mp - nm);
      L = fmaf(L, fa, sm.l[item] * fb);
      acc = fmaf(acc, fa, sm.v[item] * fb);
      m = nm;
    }
    sm.vt[tid] = acc / L;
  }
  __syncthreads();

  // 4. row-block partial of out[i] = sum_j v~[j] * B_V[g][j][i]
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < RB) o = fmaf(sm.vt[jb * RB + k], bv[k], o);
  }
  sm.part[jb * d + i_col] = o;
  __syncthreads();
  if (tid < d) {
    float r = sm.part[tid];
    for (int q = 1; q < NB; ++q) r += sm.part[q * d + tid];
    const size_t oi = out_row0 + tid;
    if (mg.out_dtype == LRATTN_F32) static_cast<float*>(mg.out)[oi] = r;
    else static_cast<uint16_t*>(mg.out)[oi] = f32_to_bf16_rne(r);
  }
}

// ------------------------------------------------------------------ probes

// Streaming read: each workgroup reads one contiguous chunk with
// non-temporal 16-byte buffer loads, eight in flight per lane.
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const char* __restrict__ src,
                                                              size_t chunk, size_t total,
                                                              float* __restrict__ sink) {
  constexpr int kDepth = 8;
  const size_t beg = (size_t)blockIdx.x * chunk;
  uint32_t x = 0;
  if (beg < total) {
    const uint32_t n = (uint32_t)((beg + chunk < total ? beg + chunk : total) - beg);
    const auto r = make_rsrc(src + beg, n);
    for (uint32_t off = threadIdx.x * 16u; off < n; off += kThreads * 16u * kDepth) {
      u32x4 v[kDepth];
#pragma unroll
      for (int k = 0; k < kDepth; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + k * kThreads * 16u), 0, 2);
#pragma unroll
      for (int k = 0; k < kDepth; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
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

template <int R>
hipError_t launch_cg(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<R>), dim3(a.Hq, a.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
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
  (void)group;  // one workgroup per query head: the group size only maps h to g
  switch (a.r) {
    case 16: return launch_cg<16>(a, s);
    case 32: return launch_cg<32>(a, s);
    case 48: return launch_cg<48>(a, s);
    case 64: return launch_cg<64>(a, s);
    case 128: return launch_cg<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  // chunks of whole 4 KiB pages, each below 2^31 bytes (buffer addressing)
  size_t chunk = (bytes + kProbeBlocks - 1) / kProbeBlocks;
  chunk = (chunk + 4095) & ~(size_t)4095;
  if (chunk >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kThreads), 0, s,
                     static_cast<const char*>(src), chunk, bytes, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kThreads), 0, s,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace lrattn
