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
//   whole group.  Two kernel families: partition_mfma_kernel (bf16 latents,
//   4 or 8 heads per kv-head, r a multiple of 32: scores on the matrix cores)
//   and partition_kernel (everything else: scores on the VALU).
//   combine grid (Hq, B), 256 threads.
//
// Lane mapping inside a wave (the VALU kernel's hot loop; the matrix-core
// kernel keeps it for the value side):
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

#include "lrattn_device.hpp"
#include "lrattn_internal.hpp"

namespace lrattn {
namespace {

// ------------------------------------------------------------------ formats

struct LatF32 { static constexpr int kBytes = 4; };
struct LatBF16 { static constexpr int kBytes = 2; };
struct LatF16 { static constexpr int kBytes = 2; };
struct LatI8 { static constexpr int kBytes = 1; };

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

// ------------------------------------------------------------ partition
// Fixed launch-shape choices, each measured on MI355X:
//   kUnrollSmallG  rows per slot per step, 1-2 heads, 2- and 4-byte latents
//   kUnrollLargeG  rows per slot per step, 4-8 heads
//   kUnrollI8      rows per slot per step, 1-2 heads, int8 latents
//   kNonTemporal   cache-policy bits of the streaming latent loads: each
//                  latent byte is used once, so it should not displace
//                  reusable lines in L2
//   kMfmaTiles     16-token score tiles per wave per step in the
//                  matrix-core kernel
//   kValuAfter, kMfmaAfter  where a kernel issues its first latent loads in
//                  the prologue (prologue's kAfter): the VALU kernel once q
//                  is staged, the matrix-core kernel after the absorption,
//                  so every load the prologue waits for is served ahead of
//                  the grid's latent stream
constexpr int kUnrollSmallG = 4;
constexpr int kUnrollLargeG = 2;
constexpr int kUnrollI8 = 2;
constexpr int kNonTemporal = 2;
constexpr int kMfmaTiles = 2;
constexpr int kValuAfter = 1;
constexpr int kMfmaAfter = 2;


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
                           : G >= 4 ? kUnrollLargeG
                           : (LT::kBytes == 1 ? kUnrollI8 : kUnrollSmallG);
  static constexpr int kChunk = kU * kRPW;                // rows per wave per step
  // Occupancy target (waves per SIMD) the register allocation must meet:
  // 4 (<= 128 VGPRs) unless q~ plus accumulators alone need more than 64.
  static constexpr int kWavesPerEU =
      (kEPL * G <= 16 && kEPL * G * kU <= 32) || (kEPL * G <= 32 && R >= 64) ? 4 : 2;
  static_assert(kRowBytes % 16 == 0, "latent row must be whole 16-byte pieces");
  static_assert(kAct <= 16, "latent row wider than 16 lane loads");
};

// One lane load of kWords 32-bit words (16 or 8 bytes) with cache policy kAux:
// kNonTemporal for latents read once, 0 where other
// workgroups of the same XCD read the same latents (shared streams).
template <int kWords, int kAux = kNonTemporal>
__device__ __forceinline__ void load_words(uint32_t (&w)[kWords], __amdgpu_buffer_rsrc_t r,
                                           uint32_t off) {
  if constexpr (kWords == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAux);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAux);
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
  uint64_t low;  // adaptive rank: bit i set when the step's row cb + i is below the threshold
};

// Attention-aware rank: the importance scores of a step's rows cb .. cb +
// kChunk - 1, one per lane, loaded a step ahead of the rows' latents ...
template <class LT, int R, int G>
__device__ __forceinline__ float load_imp(int cb, __amdgpu_buffer_rsrc_t rimp) {
  constexpr int CH = Geo<LT, R, G>::kChunk;
  static_assert(CH <= 64, "one score per lane");
  const int lane = threadIdx.x & 63;
  return bload4f(rimp, lane < CH ? (uint32_t)(cb + lane) * 4u : kOffNone);
}

// ... and, once they have arrived, the step's rows below the threshold as one
// wave-uniform mask.
template <class LT, int R, int G>
__device__ __forceinline__ uint64_t low_mask(float imp, float thr) {
  const int lane = threadIdx.x & 63;
  return __builtin_amdgcn_ballot_w64(lane < Geo<LT, R, G>::kChunk && imp < thr);
}

// A step's latent loads.  With attention-aware rank (kAd) `low` marks the
// step's rows below the threshold: such a row keeps only coordinates
// [0, low_rank), so a lane whose whole piece lies past low_rank (`drop`)
// gives that row's loads an offset past the buffer, which fetches nothing
// and returns the zeros the masking would produce.
template <class LT, int R, int G, int kAux = kNonTemporal, bool kAd = false>
__device__ __forceinline__ void load_step(Step<LT, R, G>& st, int cb, int slot, uint32_t lane_off,
                                          __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          __amdgpu_buffer_rsrc_t rsk, __amdgpu_buffer_rsrc_t rsv,
                                          uint64_t low = 0, bool drop = false) {
  using Gm = Geo<LT, R, G>;
  constexpr int U = Gm::kU, RPW = Gm::kRPW;
  uint32_t off[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    off[u] = (uint32_t)(cb + u * RPW) * Gm::kRowBytes + lane_off;
    if constexpr (kAd) off[u] = drop && ((low >> (u * RPW + slot)) & 1u) ? kOffNone : off[u];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) load_words<Gm::kWords, kAux>(st.k[u], rk, off[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) load_words<Gm::kWords, kAux>(st.v[u], rv, off[u]);
  if constexpr (std::is_same<LT, LatI8>::value) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t so = (uint32_t)(cb + u * RPW + slot) * 4u;
      st.sk[u] = bload4f(rsk, so);
      st.sv[u] = bload4f(rsv, so);
    }
  }
  if constexpr (kAd) st.low = low;
}

// Attention-aware rank (AttentionPack page, section 2.B): a row whose
// importance is below the threshold keeps latent coordinates [0, low_rank);
// this lane's elements e >= keep are then zero (keep = low_rank - its first
// column, clamped to [0, EPL]).
struct AdaptiveRow {
  float thr;
  int keep;
  int col;       // this lane's place in its row (it stages heads col, col + LPR, ...)
  float* lds;    // the workgroup's LDS chunk of logits [row % valu_lg_rows][G]
  __amdgpu_buffer_rsrc_t rlg;  // the group's logits [token][G] from the partition start
};

// Rows of logits a workgroup of the adaptive VALU kernel stages in LDS (16 KB)
// before writing them out: stores mixed into the latent stream cost far more
// than their bytes, so they leave a chunk at a time.
template <int G>
constexpr int valu_lg_rows() {
  return 4096 / G;
}

// The logits of rows [c0, c1) from a VALU kernel's LDS chunk to HBM: 4 bytes
// per thread and instruction, 1 KB of consecutive bytes per instruction of
// the workgroup.  Between two barriers of the whole workgroup.
template <int G>
__device__ __forceinline__ void flush_valu_logits(const AdaptiveRow& ad, int c0, int c1) {
  const int n = (c1 - c0) * G;
  for (int i = threadIdx.x; i < n; i += kThreads)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ad.lds[i]), ad.rlg,
                                          (int)((uint32_t)(c0 * G + i) * 4u), 0, 0);
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

template <class LT, int R, int G, bool kMask, bool kAd = false>
__device__ __forceinline__ void compute_step(
    const Step<LT, R, G>& st, int cb, int ntok, int slot, const QtView<LT, R, G>& qt,
    float (&m)[G], float (&l)[G], float (&acc)[G][Geo<LT, R, G>::kEPL],
    const AdaptiveRow& ad = {}) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, U = Gm::kU, RPW = Gm::kRPW;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  // scores: s[u][h] = q~_h . Lk[row]   (base-2 logits)
  float s[U][G];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[EPL];
    Unpack<LT>::run(st.k[u], x);
    if constexpr (kAd) {
      const bool low = (st.low >> (u * RPW + slot)) & 1u;
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = (low && e >= ad.keep) ? 0.f : x[e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) t = fmaf(qt.at(h, e), x[e], t);
      t = group_sum<Gm::kLPR>(t);
      if constexpr (kInt8) t *= st.sk[u];
      if constexpr (kAd) {
        constexpr int kLg = valu_lg_rows<G>();
        if (h % Gm::kLPR == ad.col) ad.lds[((cb + u * RPW + slot) & (kLg - 1)) * G + h] = t;
      }
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
    if constexpr (kAd) {
      const bool low = (st.low >> (u * RPW + slot)) & 1u;
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = (low && e >= ad.keep) ? 0.f : x[e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w[u][h], x[e], acc[h][e]);
    }
  }
}

// Two factor sets (image block, then text) in one launch: partitions
// [0, P_img) cover the image tokens [0, n_img) in parts of S_img with B_K,
// the rest cover the text from n_img in parts of S with BK1, writing record
// slots P_img + .. .  Uniform per workgroup.
__device__ __forceinline__ void modal_segment(PartitionArgs& a, int& p) {
  if (p < a.P_img) {
    a.t_hi = a.n_img;
    a.S = a.S_img;
  } else {
    p -= a.P_img;
    a.p_off = a.P_img;
    a.t_lo = a.n_img;
    a.BK = a.BK1;
  }
}

// The workgroup's (partition p, head group hg, sequence b).  Normally the
// grid is (P, HG, B).  With a.xcd_group the grid is one-dimensional and the
// HG head groups of one (p, b) tile take linear ids 8 apart: workgroups are
// handed to the 8 XCDs in turn by linear id, so those groups run on one XCD,
// close in time, and the tile's latents (read by every head group of a shared
// stream) are fetched from HBM once and then served by that XCD's L2.
// Returns false for the padding workgroups of the last round of tiles.
template <bool kSeg = false>
__device__ __forceinline__ bool tile_of(const PartitionArgs& a, int& p, int& hg, int& b) {
  if constexpr (kSeg) {
    // two factor sets: grid (HG, B, P), partitions slowest, so the short
    // image partitions are dispatched first, one per CU, and the text
    // partitions then spread evenly over all CUs
    hg = blockIdx.x; b = blockIdx.y; p = blockIdx.z;
    return true;
  }
  if (!a.xcd_group) {
    p = blockIdx.x; hg = blockIdx.y; b = blockIdx.z;
    return true;
  }
  const int L = blockIdx.x, x = L & 7, k = L >> 3;
  hg = k % a.HG;
  const int t = 8 * (k / a.HG) + x;  // tile: p fastest
  p = t % a.P;
  b = t / a.P;
  return b < a.B;
}

// Sum of `x` over aligned groups of n lanes, n in {8, 16, 32} (runtime, uniform).
__device__ __forceinline__ float piece_sum(float x, int n) {
  if (n <= 8) return group_sum<8>(x);
  x = group_sum<16>(x);
  if (n > 16) x += __shfl_xor(x, 16);
  return x;
}

// ------------------------------------------------------------------ merge

// ------------------------------------------------------------ partition kernel

// Absorption for the G query heads of kv-head g of sequence b:
// qt_lds[h][j] = qscale * sum_i q[h][i] * B_K[g][j][i]  (fp32, G x R).
// Every product is exact in fp32 and the sums run in fp32.
//
// When q and B_K share a 2-byte format the product runs on the matrix cores
// (absorb_mfma_issue / absorb_mfma_finish below).  Otherwise on the VALU,
// in three steps, so that a
// kernel can place its first latent loads among them:
// absorb_issue loads this thread's q values and its first batch of B_K
// pieces (8 consecutive elements of one factor row) into registers;
// absorb_stage_q stages q in LDS; absorb_dot forms the dot products (a
// batch's loads are all in flight together) and leaves q~ in qt_lds.  Vector
// loads of a wave return in issue order, so loads issued before the latents
// are not held up by them, and the dot products overlap the first latent
// round trip.
template <int R, int G>
struct AbsorbIn {
  // q: G * d values of 2 or 4 bytes = at most 8 KiB = 2 x 16 bytes per thread
  static constexpr int kQLoads = (G * kMaxHeadDim * 4 / 16 + kThreads - 1) / kThreads;
  // B_K pieces per thread per batch: all of them for d = 128 and r <= 64
  static constexpr int kPieceBatch = R / 16 < 4 ? R / 16 : 4;
  u32x4 qw[kQLoads];
  u32x4 fw[kPieceBatch][2];  // a piece is 16 bytes (2-byte factors) or 32 bytes (fp32)
};

// 16 raw bytes -> x[0..8): eight values of a 2-byte format, or four fp32
// values (x[4..8) = 0).  Every conversion is exact; fixed indices and
// selects on the uniform format only.
__device__ __forceinline__ void words_to_floats(const u32x4& w, int dt, float* x) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t word = w[j >> 1];
    const float two = dt == LRATTN_BF16 ? ((j & 1) ? bf16_hi(word) : bf16_lo(word))
                                        : ((j & 1) ? f16_hi(word) : f16_lo(word));
    const float four = j < 4 ? __uint_as_float(w[j & 3]) : 0.f;
    x[j] = dt == LRATTN_F32 ? four : two;
  }
}

// The B_K[g] slice as a raw buffer resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t factor_rsrc(const PartitionArgs& a, int g, int R) {
  const uint32_t fes = a.f_dtype == LRATTN_F32 ? 4u : 2u;
  return make_rsrc(static_cast<const char*>(a.BK) + (size_t)g * R * a.d * fes,
                   (uint32_t)(R * a.d) * fes);
}

// Piece `it` of B_K[g] (8 consecutive elements of one row): one 16-byte load
// for 2-byte factors, two for fp32.  A piece past the factor loads zeros.
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t rf, int it, int npieces,
                                           bool f32, u32x4 (&w)[2]) {
  const uint32_t off = it < npieces ? (uint32_t)it * (f32 ? 32u : 16u) : kOffNone;
  w[0] = __builtin_amdgcn_raw_buffer_load_b128(rf, (int)off, 0, 0);
  w[1] = __builtin_amdgcn_raw_buffer_load_b128(rf, (int)(f32 ? off + 16u : kOffNone), 0, 0);
}

// Every load below is a raw buffer load bounded by its slice and every loaded
// value is used unconditionally, so no load sits behind a branch and all of a
// thread's loads are in flight together.
template <int R, int G>
__device__ __forceinline__ void absorb_issue(const PartitionArgs& a, int b, int g,
                                             AbsorbIn<R, G>& in) {
  using AI = AbsorbIn<R, G>;
  const int tid = threadIdx.x, d = a.d;
  const uint32_t qes = a.q_dtype == LRATTN_F32 ? 4u : 2u;
  const size_t q0 = ((size_t)b * a.Hq + (size_t)g * G) * d;  // the G*d values are contiguous
  const auto rq = make_rsrc(static_cast<const char*>(a.q) + q0 * qes, (uint32_t)(G * d) * qes);
#pragma unroll
  for (int k = 0; k < AI::kQLoads; ++k)
    in.qw[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)((tid + k * kThreads) * 16u), 0, 0);
  const auto rf = factor_rsrc(a, g, R);
#pragma unroll
  for (int k = 0; k < AI::kPieceBatch; ++k)
    load_piece(rf, tid + k * kThreads, R * (d >> 3), a.f_dtype == LRATTN_F32, in.fw[k]);
}

// q_lds holds G rows of kMaxHeadDim floats plus 8 floats of padding that
// absorbs the stores of threads without q values.
template <int R, int G>
__device__ __forceinline__ void absorb_stage_q(const PartitionArgs& a, AbsorbIn<R, G>& in,
                                               float* q_lds) {
  using AI = AbsorbIn<R, G>;
  const int tid = threadIdx.x, d = a.d;
  {
    const bool q32 = a.q_dtype == LRATTN_F32;
    const int epc = q32 ? 4 : 8;  // values per 16 bytes; divides d
#pragma unroll
    for (int k = 0; k < AI::kQLoads; ++k) {
      const int e0 = (tid + k * kThreads) * epc;
      const int h = e0 / d;
      float* dst = e0 < G * d ? q_lds + h * kMaxHeadDim + (e0 - h * d) : q_lds + G * kMaxHeadDim;
      float x[8];
      words_to_floats(in.qw[k], a.q_dtype, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = x[e];
      if (!q32) {
#pragma unroll
        for (int e = 4; e < 8; ++e) dst[e] = x[e];
      }
    }
  }
  __syncthreads();
}

// One batch of pieces (first piece index base + tid): q~ rows j of this
// batch's factor rows.  Pieces past the factor hold zeros and write nothing;
// the sums run in every lane (the cross-lane sum cannot sit under a branch).
template <int R, int G>
__device__ __forceinline__ void absorb_batch(const PartitionArgs& a, const AbsorbIn<R, G>& in,
                                             int base, const float* q_lds, float* qt_lds) {
  constexpr int PB = AbsorbIn<R, G>::kPieceBatch;
  const int tid = threadIdx.x;
  const int nch = a.d >> 3, npieces = R * nch;
  const bool f32 = a.f_dtype == LRATTN_F32;
#pragma unroll
  for (int k = 0; k < PB; ++k) {
    const int it = base + k * kThreads + tid;
    const int j = it / nch, c = it - j * nch;
    float f[8], f2[8];
    words_to_floats(in.fw[k][0], a.f_dtype, f);
    words_to_floats(in.fw[k][1], LRATTN_F32, f2);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 + e] = f32 ? f2[e] : f[4 + e];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t = fmaf(q_lds[h * kMaxHeadDim + c * 8 + e], f[e], t);
      t = piece_sum(t, nch);
      if (c == 0 && it < npieces) qt_lds[h * R + j] = t * a.qscale;
    }
  }
}

// The first batch was loaded by absorb_issue and is used in straight-line
// code: inside a loop whose body also loads, the hardware wait before its
// first use could not be told apart from waits on the later loads (the
// latents issued meanwhile included).  Later batches (d = 256 or r = 128)
// are loaded and used in the loop.
template <int R, int G>
__device__ __forceinline__ void absorb_dot(const PartitionArgs& a, int g, AbsorbIn<R, G>& in,
                                           const float* q_lds, float* qt_lds) {
  constexpr int PB = AbsorbIn<R, G>::kPieceBatch;
  const int tid = threadIdx.x;
  const int npieces = R * (a.d >> 3);
  const bool f32 = a.f_dtype == LRATTN_F32;
  absorb_batch<R, G>(a, in, 0, q_lds, qt_lds);
  if (npieces > PB * kThreads) {
    const auto rf = factor_rsrc(a, g, R);
    for (int base = PB * kThreads; base < npieces; base += PB * kThreads) {
#pragma unroll
      for (int k = 0; k < PB; ++k) load_piece(rf, base + tid + k * kThreads, npieces, f32, in.fw[k]);
      absorb_batch<R, G>(a, in, base, q_lds, qt_lds);
    }
  }
  __syncthreads();
}

// The matrix-core absorption: q and B_K both bf16 or both fp16 (exact
// products, fp32 sums, as on the VALU).  D = A . B with A = the G query rows
// (rows G..15 zero), B = B_K[g]^T, K = d in steps of 32
// (v_mfma_f32_16x16x32_{bf16,f16}); wave w forms the 16-column tiles
// nt = w, w + 4 of the r columns.  Lane l supplies row / column l % 16 and
// the 8 elements 8 * (l / 16) .. + 7 of each 32-element step: 16 contiguous
// bytes of q or of one B_K row, loaded straight into the operand register.
// The result, lane l register i = (head 4 * (l / 16) + i, column l % 16),
// goes to qt_lds.  All loads of a 4-step chunk are in flight together
// (d = 256 takes two chunks).  absorb_mfma_finish ends with a barrier.
__device__ __forceinline__ bool absorb_on_mfma(const PartitionArgs& a) {
  return a.q_dtype == a.f_dtype && a.q_dtype != LRATTN_F32;
}

// Operand registers of one 4-step chunk; absorb_mfma_issue loads the first
// chunk so that a kernel can issue its first latent loads before the MMAs
// wait (loads return in issue order: these come back first).
template <int R>
struct MfmaAbsorbIn {
  static constexpr int kNT = R / 16;                        // column tiles: 1, 2, 3, 4 or 8
  static constexpr int kTPW = (kNT + kWaves - 1) / kWaves;  // tiles per wave: 1 or 2
  u32x4 qa[4];
  u32x4 fb[kTPW][4];
};

template <int R, int G>
__device__ __forceinline__ void absorb_mfma_load(const PartitionArgs& a, int b, int g, int k0,
                                                 MfmaAbsorbIn<R>& in) {
  using AI = MfmaAbsorbIn<R>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, ksteps = d >> 5;  // 2, 4 or 8
  const int row = lane & 15, kg = lane >> 4;
  const size_t q0 = ((size_t)b * a.Hq + (size_t)g * G) * d;
  const auto rq = make_rsrc(static_cast<const uint16_t*>(a.q) + q0, (uint32_t)(G * d) * 2u);
  const auto rf = make_rsrc(static_cast<const uint16_t*>(a.BK) + (size_t)g * R * d,
                            (uint32_t)(R * d) * 2u);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ks = k0 + kk;
    const bool kv = ks < ksteps;
    const uint32_t qoff = row < G && kv ? (uint32_t)(row * d + 32 * ks + 8 * kg) * 2u : kOffNone;
    in.qa[kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qoff, 0, 0);
#pragma unroll
    for (int t = 0; t < AI::kTPW; ++t) {
      const int nt = wave + kWaves * t;
      const uint32_t foff =
          nt < AI::kNT && kv ? (uint32_t)((16 * nt + row) * d + 32 * ks + 8 * kg) * 2u : kOffNone;
      in.fb[t][kk] = __builtin_amdgcn_raw_buffer_load_b128(rf, (int)foff, 0, 0);
    }
  }
}

template <int R, int G>
__device__ __forceinline__ void absorb_mfma_issue(const PartitionArgs& a, int b, int g,
                                                  MfmaAbsorbIn<R>& in) {
  absorb_mfma_load<R, G>(a, b, g, 0, in);
}

template <int R, int G>
__device__ __forceinline__ void absorb_mfma_finish(const PartitionArgs& a, int b, int g,
                                                   MfmaAbsorbIn<R>& in, float* qt_lds) {
  using AI = MfmaAbsorbIn<R>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const bool bf = a.q_dtype == LRATTN_BF16;
  f32x4 acc[AI::kTPW];
#pragma unroll
  for (int t = 0; t < AI::kTPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&]() {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int t = 0; t < AI::kTPW; ++t) {
        if (bf)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, in.qa[kk]),
                                                           __builtin_bit_cast(bf16x8, in.fb[t][kk]),
                                                           acc[t], 0, 0, 0);
        else
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, in.qa[kk]),
                                                          __builtin_bit_cast(f16x8, in.fb[t][kk]),
                                                          acc[t], 0, 0, 0);
      }
    }
  };
  mma();                  // steps 0..3 (zero operands past d)
  if (a.d > 128) {        // d = 256: steps 4..7
    absorb_mfma_load<R, G>(a, b, g, 4, in);
    mma();
  }
#pragma unroll
  for (int t = 0; t < AI::kTPW; ++t) {
    const int nt = wave + kWaves * t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * kg + i;
      if (nt < AI::kNT && h < G) qt_lds[h * R + 16 * nt + row] = acc[t][i] * a.qscale;
    }
  }
  __syncthreads();
}

// Dense cache (no factors, r = d): q~ = qscale * q.  The loads are those of
// absorb_issue's q part; threads without q values store into qt_lds's
// padding, so no load sits behind a branch.
template <int R, int G>
__device__ __forceinline__ void identity_issue(const PartitionArgs& a, int b, int g,
                                               AbsorbIn<R, G>& in) {
  using AI = AbsorbIn<R, G>;
  const int tid = threadIdx.x, d = a.d;
  const uint32_t qes = a.q_dtype == LRATTN_F32 ? 4u : 2u;
  const size_t q0 = ((size_t)b * a.Hq + (size_t)g * G) * d;
  const auto rq = make_rsrc(static_cast<const char*>(a.q) + q0 * qes, (uint32_t)(G * d) * qes);
#pragma unroll
  for (int k = 0; k < AI::kQLoads; ++k)
    in.qw[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)((tid + k * kThreads) * 16u), 0, 0);
}

template <int R, int G>
__device__ __forceinline__ void identity_finish(const PartitionArgs& a, AbsorbIn<R, G>& in,
                                                float* qt_lds) {
  using AI = AbsorbIn<R, G>;
  const int tid = threadIdx.x, d = a.d;  // d == R
  const bool q32 = a.q_dtype == LRATTN_F32;
  const int epc = q32 ? 4 : 8;
#pragma unroll
  for (int k = 0; k < AI::kQLoads; ++k) {
    const int e0 = (tid + k * kThreads) * epc;
    float* dst = e0 < G * d ? qt_lds + e0 : qt_lds + G * R;  // rows of R == d: [h][j] is e0
    float x[8];
    words_to_floats(in.qw[k], a.q_dtype, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = x[e] * a.qscale;
    if (!q32) {
#pragma unroll
      for (int e = 4; e < 8; ++e) dst[e] = x[e] * a.qscale;
    }
  }
  __syncthreads();
}

// The partition prologue: q~ into qt_lds (fp32 [G][R]), with `issue` (the
// first latent loads) placed at position kAfter: 0 first, 1 once q is in
// flight / staged, 2 after the absorption.
// q~ absorbed beforehand (per-query-head factors): the G rows of heads
// hg * G .. + G - 1, fp32, straight into qt_lds.
template <int R, int G>
__device__ __forceinline__ u32x4 pre_issue(const PartitionArgs& a, int b, int hg) {
  const auto rq = make_rsrc(a.qt_pre + ((size_t)b * a.Hq + (size_t)hg * G) * R,
                            (uint32_t)(G * R) * 4u);
  return __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(threadIdx.x * 16u), 0, 0);
}

template <int R, int G>
__device__ __forceinline__ void pre_finish(const u32x4& w, float* qt_lds) {
  static_assert(G * R <= 4 * kThreads, "one 16-byte piece per thread");
  const int i = threadIdx.x * 4;
  // threads past the G * R values store into the padding
  float* dst = i < G * R ? qt_lds + i : qt_lds + G * R;
  dst[0] = __uint_as_float(w[0]);
  dst[1] = __uint_as_float(w[1]);
  dst[2] = __uint_as_float(w[2]);
  dst[3] = __uint_as_float(w[3]);
  __syncthreads();
}

template <int R, int G, int kAfter, class Issue>
__device__ __forceinline__ void prologue(const PartitionArgs& a, int b, int hg, int g,
                                         float* q_lds, float* qt_lds, Issue&& issue) {
  if (a.qt_pre != nullptr) {
    const u32x4 w = pre_issue<R, G>(a, b, hg);
    if constexpr (kAfter < 2) issue();
    pre_finish<R, G>(w, qt_lds);
  } else if (a.BK == nullptr) {
    AbsorbIn<R, G> in;
    identity_issue<R, G>(a, b, g, in);
    if constexpr (kAfter < 2) issue();
    identity_finish<R, G>(a, in, qt_lds);
  } else if (absorb_on_mfma(a)) {
    MfmaAbsorbIn<R> ai;
    absorb_mfma_issue<R, G>(a, b, g, ai);
    if constexpr (kAfter < 2) issue();
    absorb_mfma_finish<R, G>(a, b, g, ai, qt_lds);
  } else {
    AbsorbIn<R, G> ab;
    absorb_issue<R, G>(a, b, g, ab);
    if constexpr (kAfter == 0) issue();
    absorb_stage_q<R, G>(a, ab, q_lds);
    if constexpr (kAfter == 1) issue();
    absorb_dot<R, G>(a, g, ab, q_lds, qt_lds);
  }
  if constexpr (kAfter == 2) issue();
}

template <int R, int G>
struct PartLds {
  float q[G * kMaxHeadDim + 8];  // + padding for threads without q values
  float qt[G * R + 8];  // + padding (dense prologue)
  float acc[kWaves * G * R];
  float m[kWaves * G];
  float l[kWaves * G];
};

// Merges the kWaves per-wave partials (fixed order) and writes one record
// per query head of the group: acc[0..R), m, l.  red_acc [wave][h][R],
// red_m and red_l [wave][h] are in LDS; the caller has synchronized.
template <int R, int G, bool kSeg = false>
__device__ __forceinline__ void write_records(const PartitionArgs& a, int b, int hg, int p,
                                              const float* red_acc, const float* red_m,
                                              const float* red_l) {
  const int tid = threadIdx.x;
  // record slots: p of P, or (two factor sets) p_off + p of P_rec
  const int nrec = kSeg ? a.P_rec : a.P;
  if constexpr (kSeg) p += a.p_off;
  float* const rec0 = a.ws + ((size_t)b * a.Hq + (size_t)hg * G) * (size_t)nrec * (R + kRecPad);
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
    float* rec = rec0 + ((size_t)h * nrec + p) * (R + kRecPad);
    rec[j] = sacc;
    if (j == 0) {
      rec[R] = M;
      rec[R + 1] = L;
    }
  }
}

// Occupancy target of a VALU partition kernel: the geometry's, except that
// the two-segment form of fp32 latents with 8 heads needs a few registers
// more than 128 (one spilled at 4 waves per SIMD).
template <class LT, int R, int G, bool kSeg>
constexpr int valu_waves() {
  return kSeg && LT::kBytes == 4 && G == 8 ? 2 : Geo<LT, R, G>::kWavesPerEU;
}

template <class LT, int R, int G, int kAux = kNonTemporal, bool kAd = false, bool kSeg = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(valu_waves<LT, R, G, kSeg>())))
void partition_kernel(PartitionArgs a) {
  using Gm = Geo<LT, R, G>;
  constexpr int EPL = Gm::kEPL, LPR = Gm::kLPR, CH = Gm::kChunk;
  constexpr bool kInt8 = std::is_same<LT, LatI8>::value;

  // head group hg (its G query heads) reads latent stream g
  int p, hg, b;
  if (!tile_of<kSeg>(a, p, hg, b)) return;
  if constexpr (kSeg) modal_segment(a, p);
  const int g = hg * G / a.hps;
  // seq_lens[b] is one value for the whole workgroup; keeping it in a scalar
  // register keeps the buffer descriptors below scalar (a descriptor the
  // compiler must treat as per-lane costs a readfirstlane loop per load)
  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  const int t0 = (kSeg ? a.t_lo : 0) + p * a.S;
  const int t1 = min(t0 + a.S, kSeg ? min(len, a.t_hi) : len);
  if (t0 >= t1) return;  // partition past the sequence: nothing to write
  const int ntok = t1 - t0;

  __shared__ PartLds<R, G> lds;
  __shared__ float lg_lds[kAd ? valu_lg_rows<G>() * G : 1];  // adaptive rank: logits chunk
  float* q_lds = lds.q;
  float* qt_lds = lds.qt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, cc = lane % LPR;
  // first row of this wave's steps and the distance between its steps (the
  // four waves take the partition's steps in turn)
  constexpr int kStride = kWaves * CH;
  const int cb0 = wave * CH;
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
  // attention-aware rank: the partition's importance scores and logits
  __amdgpu_buffer_rsrc_t rimp = rk;
  AdaptiveRow ad{};
  if constexpr (kAd) {
    rimp = make_rsrc(a.imp + row0, (uint32_t)ntok * 4u);
    ad.thr = a.imp_thr;
    ad.keep = min(max(a.low_rank - cc * EPL, 0), EPL);
    ad.col = cc;
    ad.lds = lg_lds;
    ad.rlg = make_rsrc(a.logits + (((size_t)b * a.HG + hg) * (size_t)a.T + (size_t)t0) * G,
                       (uint32_t)ntok * G * 4u);
  }

  // q and B_K are requested first, then the first step's latents; the
  // absorption then runs while the latents are in flight.  Attention-aware
  // rank: the importance scores of each step's rows are requested a step
  // ahead (the first step's before q), so the loads of dropped latent
  // pieces can be left out.
  Step<LT, R, G> cur;
  float inx = 0.f;  // the next step's importance score of this lane's row
  const bool drop = kAd && ad.keep == 0;
  if constexpr (kAd) inx = load_imp<LT, R, G>(cb0, rimp);
  prologue<R, G, kValuAfter>(a, b, hg, g, q_lds, qt_lds, [&]() {
    const uint64_t low = kAd ? low_mask<LT, R, G>(inx, ad.thr) : 0;
    load_step<LT, R, G, kAux, kAd>(cur, cb0, slot, lane_off, rk, rv, rsk, rsv, low, drop);
    if constexpr (kAd) inx = load_imp<LT, R, G>(cb0 + kStride, rimp);
  });

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
  // one step in flight per wave: the next step's loads are issued once this
  // step's registers are free (past the partition they return zero without
  // touching memory)
  if constexpr (!kAd) {
    for (int cb = cb0; cb < ntok; cb += kStride) {
      if (cb + CH <= ntok)
        compute_step<LT, R, G, false, kAd>(cur, cb, ntok, slot, qt, m, l, acc, ad);
      else
        compute_step<LT, R, G, true, kAd>(cur, cb, ntok, slot, qt, m, l, acc, ad);
      load_step<LT, R, G, kAux, kAd>(cur, cb + kStride, slot, lane_off, rk, rv, rsk, rsv, 0,
                                     drop);
    }
  } else {
    // rounds of the four waves, the same count in every wave so that the
    // chunk flushes can synchronize the workgroup; a wave whose step lies
    // past the partition computes nothing in that round
    constexpr int kLg = valu_lg_rows<G>(), kRPC = kLg / kStride;
    static_assert(kLg % kStride == 0, "a chunk is whole rounds");
    const int nround = (ntok + kStride - 1) / kStride;
    for (int r = 0; r < nround; ++r) {
      const int cb = cb0 + r * kStride;
      if (cb + CH <= ntok)
        compute_step<LT, R, G, false, kAd>(cur, cb, ntok, slot, qt, m, l, acc, ad);
      else if (cb < ntok)
        compute_step<LT, R, G, true, kAd>(cur, cb, ntok, slot, qt, m, l, acc, ad);
      const uint64_t low = low_mask<LT, R, G>(inx, ad.thr);
      load_step<LT, R, G, kAux, kAd>(cur, cb + kStride, slot, lane_off, rk, rv, rsk, rsv, low,
                                     drop);
      inx = load_imp<LT, R, G>(cb + 2 * kStride, rimp);
      if ((r + 1) % kRPC == 0 || r + 1 == nround) {
        const int c0 = (r / kRPC) * kLg;
        __syncthreads();  // the chunk's rows are in LDS
        flush_valu_logits<G>(ad, c0, min(c0 + kLg, ntok));
        __syncthreads();  // and read before the next chunk's rows
      }
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

  write_records<R, G, kSeg>(a, b, hg, p, lds.acc, lds.m, lds.l);
}

// ------------------------------------------------ partition, matrix-core scores
// bf16 latents, 4 or 8 query heads per kv-head, r in {32, 64, 128}.
//
// The scores of a tile of 16 tokens are a dense product, D = A . B, taken on
// the matrix cores as r / 32 steps of v_mfma_f32_16x16x32_bf16 per term:
//   B[k][n] = Lk[token n][k]: the stored bf16 latents as they are.  Lane l
//             loads 16 bytes (8 columns) of token l % 16, column group
//             l / 16 of each 32-column step; that register is its B operand.
//   A[i][k] = q~[i % G][k]: rows repeat the G heads.  q~ is split exactly
//             into three bf16 terms (hi + mid + lo == q~ in fp32), each
//             multiplied into the same fp32 accumulator, so the scores are
//             fp32 products of the exact inputs, as on the VALU path.
// Lane l receives rows 4 * (l / 16) + i (i < 4) of column l % 16: the scores
// of token l % 16 for heads i (G = 4) or 4 * ((l / 16) % 2) + i (G = 8).
// One reference max per head serves the whole wave (moved lazily, as on the
// VALU path), so the exponentials computed in the score layout can be handed
// to the value side through a per-wave LDS tile [token][head]; the value side
// keeps the VALU path's slot layout: kLPR lanes per row, 8 columns per lane.
template <int R, int G, int NT = kMfmaTiles>
struct MGeo {
  static constexpr int kRowBytes = 2 * R;
  static constexpr int kKC = R / 32;           // 32-column MFMA steps per tile
  static constexpr int kTerms = 3;             // bf16 terms of q~
  static constexpr int kLPR = kRowBytes / 16;  // value lanes per row: 4, 8, 16
  static constexpr int kRPW = 64 / kLPR;       // rows per value load
  static constexpr int kVU = 16 / kRPW;        // value loads per tile
  static constexpr int kNT = NT;
  static constexpr int kChunk = 16 * kNT;      // tokens per wave per step
  static constexpr int kHL = G < 4 ? G : 4;    // distinct heads in a lane's 4 results
  // registers: q~ terms 12 * kKC, accumulators 8 * G, latents 4 * (kKC + kVU)
  // per tile
  static constexpr int kRegs = 12 * kKC + 8 * G + 4 * kNT * (kKC + kVU);
  static constexpr int kWavesPerEU = kRegs <= 80 ? 4 : kRegs <= 120 ? 3 : 2;
  static_assert(R % 32 == 0 && (G == 1 || G == 2 || G == 4 || G == 8), "matrix-core path shape");
};

template <int R, int G, int NT = kMfmaTiles>
struct MStep {
  uint32_t k[NT][MGeo<R, G, NT>::kKC][4];
  uint32_t v[NT][MGeo<R, G, NT>::kVU][4];
};

// Attention-aware rank on the matrix-core kernel (AttentionPack page, section
// 2.B).  A row below the threshold keeps latent columns [0, low_rank).  A
// 16-byte piece a lane loads that lies wholly past low_rank is simply not
// fetched for such a row (an offset past the buffer returns the zeros the
// reduced rank means).  When low_rank is not a multiple of 8 (the kernel's
// kCut form) one piece per row is cut: its columns past low_rank are
// cleared in registers.  dropk bit c: this lane's piece of 32-column step c
// (score layout) lies past low_rank; dropv: its value piece does.
struct MAdaptive {
  float thr;
  uint32_t dropk;
  bool dropv;
  int pk;      // the 32-column step whose piece of this lane is cut, or -1
  int keepk;   // columns that piece keeps (1..7)
  int keepv;   // columns this lane's value piece keeps (8 when it is not cut)
  __amdgpu_buffer_rsrc_t rlg;  // the group's logits [token][G] from the partition start
  float* lgs;  // the workgroup's LDS chunk of logits [row % lg_rows][G]
};

// Rows of logits a workgroup of the adaptive matrix-core kernel stages in LDS
// before writing them out (a power of two, a multiple of the 128 rows of a
// round of the four waves), sized so that the chunk does not lower the
// kernel's occupancy: 32 or 64 KB, over the LDS of the prologue and epilogue.
template <int R, int G>
constexpr int lg_rows() {
  return G == 8 ? (R == 128 ? 2048 : 1024) : (R == 128 ? 4096 : 2048);
}

// The logits of rows [c0, c1) from the LDS chunk to HBM: 16 bytes per thread
// and instruction, every instruction of the workgroup 4 KB of consecutive
// bytes.  Between two barriers of the whole workgroup.
template <int G>
__device__ __forceinline__ void flush_logits(const MAdaptive& ad, int c0, int c1) {
  const int n4 = (c1 - c0) * G / 4;  // 16-byte pieces
  const float4* src = reinterpret_cast<const float4*>(ad.lgs);
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const float4 v = src[i];
    const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(w, ad.rlg, (int)((uint32_t)(c0 * G + 4 * i) * 4u), 0, 0);
  }
}

// Latent word holding elements e0 (low half) and e0 + 1 (high half): the
// elements at or past `keep` become zero.
__device__ __forceinline__ uint32_t keep_word(uint32_t w, int keep, int e0) {
  return w & (keep > e0 + 1 ? 0xffffffffu : keep > e0 ? 0x0000ffffu : 0u);
}

// The importance scores of a wave's step (rows cb .. cb + CH - 1), one per
// lane, requested a step ahead of the rows' latents ...
template <int CH>
__device__ __forceinline__ float load_step_imp(__amdgpu_buffer_rsrc_t rimp, int cb, int lane) {
  static_assert(CH <= 64, "one score per lane");
  return bload4f(rimp, lane < CH ? (uint32_t)(cb + lane) * 4u : kOffNone);
}

// ... and, when they have arrived, the step's low rows as one wave-uniform
// mask (bit i: row cb + i is below the threshold).  Rows past the partition
// read 0; their latents lie past the buffer whatever the mask says.
template <int CH>
__device__ __forceinline__ uint32_t low_rows(float imp, int lane, float thr) {
  static_assert(CH <= 32, "one mask bit per row of the step");
  return (uint32_t)__builtin_amdgcn_ballot_w64(lane < CH && imp < thr);
}

// A step's latent loads.  With attention-aware rank (kAd) `low` marks the
// step's rows below the threshold: their pieces past low_rank get an offset
// past the buffer, so they are not fetched and arrive as zeros.
template <int R, int G, int NT, int kAux = kNonTemporal, bool kAd = false>
__device__ __forceinline__ void load_mstep(MStep<R, G, NT>& st, int cb, uint32_t koff,
                                           uint32_t voff, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, uint32_t low = 0,
                                           const MAdaptive* ad = nullptr) {
  using Mg = MGeo<R, G, NT>;
  const int lane = threadIdx.x & 63, slot = lane / Mg::kLPR;
#pragma unroll
  for (int t = 0; t < Mg::kNT; ++t) {
    const uint32_t base = (uint32_t)(cb + 16 * t) * Mg::kRowBytes;
    const bool lowk = kAd && ((low >> (16 * t + (lane & 15))) & 1u);
#pragma unroll
    for (int c = 0; c < Mg::kKC; ++c) {
      // only the lane's part is selected, so the step base and the piece
      // offset stay scalar and immediate (kOffNone plus them is still past
      // the buffer)
      uint32_t lo = koff;
      if constexpr (kAd) lo = lowk && ((ad->dropk >> c) & 1u) ? kOffNone : lo;
      load_words<4, kAux>(st.k[t][c], rk, base + lo + 64u * c);
    }
  }
#pragma unroll
  for (int t = 0; t < Mg::kNT; ++t) {
    const uint32_t base = (uint32_t)(cb + 16 * t) * Mg::kRowBytes;
#pragma unroll
    for (int u = 0; u < Mg::kVU; ++u) {
      uint32_t lo = voff;
      if constexpr (kAd) {
        const bool lowv = (low >> (16 * t + slot + Mg::kRPW * u)) & 1u;
        lo = lowv && ad->dropv ? kOffNone : lo;
      }
      load_words<4, kAux>(st.v[t][u], rv, base + lo + (uint32_t)(u * Mg::kRPW) * Mg::kRowBytes);
    }
  }
}

// Scores of the step's tiles: s[t][i] = base-2 logit of token 16 t + l % 16
// for this lane's head i (rows 4 * (l / 16) + i of the product).
template <int R, int G, int NT, bool kMask, bool kAd = false, bool kCut = false>
__device__ __forceinline__ void mfma_scores(const MStep<R, G, NT>& st, int cb, int ntok, int lane,
                                            const bf16x8 (&qa)[3][MGeo<R, G, NT>::kKC],
                                            float (&s)[NT][4], uint32_t low = 0,
                                            const MAdaptive* ad = nullptr) {
  constexpr int KC = MGeo<R, G, NT>::kKC;
  const int tok = lane & 15;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    u32x4 kw[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      kw[c] = u32x4{st.k[t][c][0], st.k[t][c][1], st.k[t][c][2], st.k[t][c][3]};
    }
    if constexpr (kCut) {
      const bool lowk = (low >> (16 * t + tok)) & 1u;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          kw[c][j] = lowk && c == ad->pk ? keep_word(kw[c][j], ad->keepk, 2 * j) : kw[c][j];
      }
    }
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int term = 2; term >= 0; --term) {  // smallest term first
#pragma unroll
      for (int c = 0; c < KC; ++c)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[term][c], __builtin_bit_cast(bf16x8, kw[c]),
                                                    d, 0, 0, 0);
    }
    if constexpr (kAd) {
      // the logits into the LDS chunk, token-major per head group: lanes
      // 0-15 hold heads 0-3 of their token, lanes 16-31 heads 4-7 (G = 8);
      // rows past the partition are staged but never written out
      constexpr int kLg = lg_rows<R, G>();
      const int row = (cb + 16 * t + tok) & (kLg - 1);
      if (lane < (G == 8 ? 32 : 16))
        *reinterpret_cast<float4*>(ad->lgs + row * G + 4 * ((lane >> 4) & 1)) =
            make_float4(d[0], d[1], d[2], d[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[t][i] = d[i];
      if constexpr (kMask) {
        if (cb + 16 * t + tok >= ntok) s[t][i] = -INFINITY;
      }
    }
  }
}

// Online softmax on scores in the matrix-core result layout, then the
// latent-space value accumulation in the slot layout.  Lane l's result i is
// head (4 * (l / 16) + i) % G: with G < 4 results i >= G repeat heads and are
// not used.
template <int R, int G, int NT, bool kCut = false>
__device__ __forceinline__ void softmax_values(const float (&s)[NT][4], const MStep<R, G, NT>& st,
                                               int lane, float (&mm)[4], float (&ll)[4],
                                               float (&acc)[G][8], float* wl, uint32_t low = 0,
                                               const MAdaptive* ad = nullptr) {
  using Mg = MGeo<R, G, NT>;
  constexpr int VU = Mg::kVU, RPW = Mg::kRPW, HL = Mg::kHL;
  const int tok = lane & 15;
  const bool hi_half = G == 8 && ((lane >> 4) & 1);  // this lane's results are heads 4..7

  // Lazily moved reference max per head, the same in every lane holding the
  // head (lanes of the same row parity hold identical rows): mm[i] belongs to
  // this lane's head i.  A 16-lane row max is the wave max of that head.
  bool need = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < HL; ++i) need |= s[t][i] > mm[i] + kLazyLog2;
  }
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int i = 0; i < HL; ++i) {
      float x = s[0][i];
#pragma unroll
      for (int t = 1; t < NT; ++t) x = fmaxf(x, s[t][i]);
      x = row_max16(x);
      const float nm = x > mm[i] + kLazyLog2 ? x : mm[i];
      const float corr = fast_exp2(mm[i] - nm);
      mm[i] = nm;
      ll[i] *= corr;
      // the value side holds every head: heads i (lane 0) and 4 + i (lane 16)
      const float c0 = readlane_f(corr, 0);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= c0;
      if constexpr (G == 8) {
        const float c1 = readlane_f(corr, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[4 + i][e] *= c1;
      }
    }
  }

  // weights 2^(s - m) into the wave's [token][head] tile
  float e[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < HL; ++i) {
      e[t][i] = fast_exp2(s[t][i] - mm[i]);
      ll[i] += e[t][i];
    }
  }
  if (lane < (G == 8 ? 32 : 16)) {  // the lanes holding distinct (token, head) results
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float* dst = wl + (16 * t + tok) * G + (hi_half ? 4 : 0);
      if constexpr (HL == 4) *reinterpret_cast<float4*>(dst) = make_float4(e[t][0], e[t][1], e[t][2], e[t][3]);
      else if constexpr (HL == 2) *reinterpret_cast<float2*>(dst) = make_float2(e[t][0], e[t][1]);
      else dst[0] = e[t][0];
    }
  }
  // the other lanes' weights are read below
  wave_sync();

  // latent-space value accumulation, slot layout
  const int slot = lane / Mg::kLPR;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const float* wr = wl + (16 * t + slot + RPW * u) * G;
      float w[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < G; h4 += 4) {
          const float4 w4 = *reinterpret_cast<const float4*>(wr + h4);
          w[h4] = w4.x; w[h4 + 1] = w4.y; w[h4 + 2] = w4.z; w[h4 + 3] = w4.w;
        }
      } else if constexpr (G == 2) {
        const float2 w2 = *reinterpret_cast<const float2*>(wr);
        w[0] = w2.x; w[1] = w2.y;
      } else {
        w[0] = wr[0];
      }
      float x[8];
      Unpack<LatBF16>::run(st.v[t][u], x);
      if constexpr (kCut) {
        const bool lowv = (low >> (16 * t + slot + RPW * u)) & 1u;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = lowv && j >= ad->keepv ? 0.f : x[j];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(w[h], x[j], acc[h][j]);
      }
    }
  }
  // the tile's reads are done before the next step writes it
  wave_sync();
}

template <int R, int G, bool kMask, bool kAd = false, bool kCut = false>
__device__ __forceinline__ void compute_mstep(
    const MStep<R, G>& st, int cb, int ntok, int lane, const bf16x8 (&qa)[3][MGeo<R, G>::kKC],
    float (&mm)[4], float (&ll)[4], float (&acc)[G][8], float* wl, uint32_t low = 0,
    const MAdaptive* ad = nullptr) {
  float s[MGeo<R, G>::kNT][4];
  mfma_scores<R, G, MGeo<R, G>::kNT, kMask, kAd, kCut>(st, cb, ntok, lane, qa, s, low, ad);
  softmax_values<R, G, MGeo<R, G>::kNT, kCut>(s, st, lane, mm, ll, acc, wl, low, ad);
}

// End of a matrix-core partition: the wave's exp-sums over its 16 token
// lanes, its accumulators over the slots (one reference per head for the
// whole wave: plain sums), then the fixed-order merge of the waves.
template <int R, int G, int NT, bool kSeg = false>
__device__ __forceinline__ void mfma_epilogue(const PartitionArgs& a, int b, int hg, int p,
                                              const float (&mm)[4], const float (&ll)[4],
                                              float (&acc)[G][8], PartLds<R, G>& lds) {
  using Mg = MGeo<R, G, NT>;
  constexpr int LPR = Mg::kLPR, HL = Mg::kHL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPR, cc = lane % LPR;
  float m[G], l[G];
#pragma unroll
  for (int i = 0; i < HL; ++i) {
    const float x = group_sum<16>(ll[i]);
    l[i] = readlane_f(x, 0);
    m[i] = readlane_f(mm[i], 0);
    if constexpr (G == 8) {
      l[4 + i] = readlane_f(x, 16);
      m[4 + i] = readlane_f(mm[i], 16);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lds.acc[(wave * G + h) * R + cc * 8 + e] = acc[h][e];
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
  write_records<R, G, kSeg>(a, b, hg, p, lds.acc, lds.m, lds.l);
}

template <int R, int G>
struct MPartLds {
  PartLds<R, G> base;
  float w[kWaves * MGeo<R, G>::kChunk * G];
};

// The adaptive form: the LDS chunk of logits overlays the query staging and
// the merge area, which are idle while the partition streams.
template <int R, int G>
struct MPartLdsAd {
  union {
    PartLds<R, G> base;
    float lg[lg_rows<R, G>() * G];
  };
  float w[kWaves * MGeo<R, G>::kChunk * G];
};

// Occupancy targets (waves per SIMD) of the attention-aware forms, each the
// highest without spills: with 8 heads the adaptive form needs more registers
// than three waves per SIMD allow; with 4 heads it fits the plain form's;
// the plain form does; the kCut form with 8 heads at r = 128 needs more than
// 256 registers.
template <int R, int G, bool kAd, bool kCut>
constexpr int mfma_waves() {
  if constexpr (kCut && G == 8 && R == 128) return 1;
  else if constexpr (kAd && G == 8 && MGeo<R, G>::kWavesPerEU > 2) return 2;
  else return MGeo<R, G>::kWavesPerEU;
}

template <int R, int G, int kAux = kNonTemporal, bool kSeg = false, bool kAd = false,
          bool kCut = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(mfma_waves<R, G, kAd, kCut>())))
void partition_mfma_kernel(PartitionArgs a) {
  static_assert(kAd || !kCut, "a cut piece only exists with attention-aware rank");
  using Mg = MGeo<R, G>;
  constexpr int KC = Mg::kKC, LPR = Mg::kLPR, CH = Mg::kChunk;

  // head group hg (its G query heads) reads latent stream g
  int p, hg, b;
  if (!tile_of<kSeg>(a, p, hg, b)) return;
  if constexpr (kSeg) modal_segment(a, p);
  const int g = hg * G / a.hps;
  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  const int t0 = (kSeg ? a.t_lo : 0) + p * a.S;
  const int t1 = min(t0 + a.S, kSeg ? min(len, a.t_hi) : len);
  if (t0 >= t1) return;  // partition past the sequence: nothing to write
  const int ntok = t1 - t0;

  __shared__ std::conditional_t<kAd, MPartLdsAd<R, G>, MPartLds<R, G>> lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, cc = lane % LPR;

  const size_t row0 = ((size_t)b * a.Hkv + g) * (size_t)a.T + (size_t)t0;
  const uint32_t nbytes = (uint32_t)ntok * Mg::kRowBytes;
  const auto rk = make_rsrc(static_cast<const char*>(a.LK) + row0 * Mg::kRowBytes, nbytes);
  const auto rv = make_rsrc(static_cast<const char*>(a.LV) + row0 * Mg::kRowBytes, nbytes);
  // score layout: token lane % 16, 16-byte column group lane / 16 of each
  // 64-byte (32-column) step; value layout: slot rows, 16 bytes per lane
  const uint32_t koff = (uint32_t)((lane & 15) * Mg::kRowBytes + (lane >> 4) * 16);
  const uint32_t voff = (uint32_t)(slot * Mg::kRowBytes + cc * 16);
  // attention-aware rank: the partition's importance scores and logits (the
  // logits are staged in LDS and written out a chunk at a time: stores mixed
  // into the latent stream cost far more than their bytes)
  __amdgpu_buffer_rsrc_t rimp = rk;
  MAdaptive ad{};
  if constexpr (kAd) {
    rimp = make_rsrc(a.imp + row0, (uint32_t)ntok * 4u);
    ad.thr = a.imp_thr;
#pragma unroll
    for (int c = 0; c < KC; ++c) ad.dropk |= (32 * c + 8 * (lane >> 4) >= a.low_rank ? 1u : 0u) << c;
    ad.dropv = cc * 8 >= a.low_rank;
    ad.pk = -1;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int keep = a.low_rank - (32 * c + 8 * (lane >> 4));
      if (keep > 0 && keep < 8) {
        ad.pk = c;
        ad.keepk = keep;
      }
    }
    ad.keepv = min(max(a.low_rank - cc * 8, 0), 8);
    ad.rlg = make_rsrc(a.logits + (((size_t)b * a.HG + hg) * (size_t)a.T + (size_t)t0) * G,
                       (uint32_t)ntok * G * 4u);
    if constexpr (kAd) ad.lgs = lds.lg;
  }

  // attention-aware rank: the importance scores of each step's rows are
  // requested a step ahead of its latents (the first step's before the
  // prologue), so the loads of dropped latent pieces can be left out
  MStep<R, G> cur;
  float imp_next = 0.f;
  uint32_t low = 0;  // the low rows of the step in `cur`
  if constexpr (kAd) imp_next = load_step_imp<CH>(rimp, wave * CH, lane);
  prologue<R, G, kMfmaAfter>(a, b, hg, g, lds.base.q, lds.base.qt, [&]() {
    if constexpr (kAd) low = low_rows<CH>(imp_next, lane, ad.thr);
    load_mstep<R, G, Mg::kNT, kAux, kAd>(cur, wave * CH, koff, voff, rk, rv, low, &ad);
    if constexpr (kAd) imp_next = load_step_imp<CH>(rimp, wave * CH + kWaves * CH, lane);
  });

  // A operands: row lane % 16 is head (lane % 16) % G; k-group lane / 16
  bf16x8 qa[3][KC];
  {
    const float* qrow = lds.base.qt + ((lane & 15) % G) * R + 8 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = qrow[32 * c + j];
      bf16x8 t[3];
      split3x8(x, t);
#pragma unroll
      for (int term = 0; term < 3; ++term) qa[term][c] = t[term];
    }
  }
  // the logits chunk overlays q~, which every wave has read above
  if constexpr (kAd) __syncthreads();

  float mm[4], ll[4], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mm[i] = -FLT_MAX;
    ll[i] = 0.f;
  }
  float* wl = lds.w + wave * CH * G;
  if constexpr (!kAd) {
    for (int cb = wave * CH; cb < ntok; cb += kWaves * CH) {
      if (cb + CH <= ntok)
        compute_mstep<R, G, false>(cur, cb, ntok, lane, qa, mm, ll, acc, wl);
      else
        compute_mstep<R, G, true>(cur, cb, ntok, lane, qa, mm, ll, acc, wl);
      load_mstep<R, G, Mg::kNT, kAux>(cur, cb + kWaves * CH, koff, voff, rk, rv);
    }
  } else {
    // rounds of the four waves (128 rows), the same count in every wave so
    // that the chunk flushes can synchronize the workgroup; a wave whose
    // step lies past the partition computes nothing in that round
    constexpr int kRound = kWaves * CH, kLg = lg_rows<R, G>(), kRPC = kLg / kRound;
    static_assert(kLg % kRound == 0, "a chunk is whole rounds");
    const int nround = (ntok + kRound - 1) / kRound;
    for (int r = 0; r < nround; ++r) {
      const int cb = wave * CH + r * kRound;
      if (cb + CH <= ntok)
        compute_mstep<R, G, false, kAd, kCut>(cur, cb, ntok, lane, qa, mm, ll, acc, wl, low, &ad);
      else if (cb < ntok)
        compute_mstep<R, G, true, kAd, kCut>(cur, cb, ntok, lane, qa, mm, ll, acc, wl, low, &ad);
      low = low_rows<CH>(imp_next, lane, ad.thr);
      load_mstep<R, G, Mg::kNT, kAux, kAd>(cur, cb + kRound, koff, voff, rk, rv, low, &ad);
      imp_next = load_step_imp<CH>(rimp, cb + 2 * kRound, lane);
      if ((r + 1) % kRPC == 0 || r + 1 == nround) {
        const int c0 = (r / kRPC) * kLg;
        __syncthreads();  // the chunk's rows are in LDS
        flush_logits<G>(ad, c0, min(c0 + kLg, ntok));
        __syncthreads();  // and read before the next chunk's rows
      }
    }
  }

  mfma_epilogue<R, G, Mg::kNT, kSeg>(a, b, hg, p, mm, ll, acc, lds.base);
}

// --------------------------------------- partition, rebuilt (and rotated) keys
// WSVD page, section 2.C: the decode kernel rebuilds the keys from the
// latents on chip and scores the rebuilt keys.  This kernel does so for a
// tile of 16 keys per wave on the matrix cores, can rotate the rebuilt keys
// by position before scoring (a position-dependent rotation is what the
// absorbed form q . B_K^T cannot carry), and scores them against the query
// rotated by its own position.  Values are not rotated, so they stay in the
// latent space: the value side and the records are those of the absorbed
// path.  bf16 q, latents and factors; d in {64, 128}; r in {32, 64}.
//
//   rebuild  K^T (d x 16) = B_K^T (d x r) . L_K^T (r x 16): per 16-row block n
//            of d and 32-row step c of r one v_mfma_f32_16x16x32_bf16.
//            A = B_K^T fragments (arranged in LDS once per workgroup),
//            B = the latent tile as loaded (lane l: token l % 16, latents
//            32 c + 8 (l / 16) .. + 7).  Lane l's result register i of block
//            n is d = 16 n + 4 (l / 16) + i of token l % 16: exact bf16
//            products, fp32 sums.
//   rotate   pairs (j, j + d/2) are blocks n and n + d/32 of one lane and
//            register; the cosines and sines of the token's position come
//            from the caller's table.
//   score    S = Q' . K'^T in fp32 on the matrix cores with the 16-block
//            4 x 4 instruction (v_mfma_f32_4x4x1_16b_f32), q' = qscale *
//            rotate(q, seq_len - 1).  Block l / 4 pairs a quad of 4 heads
//            (rows, from the query operand) with the 4 tokens of lanes
//            4 (l / 4) .. + 3 (columns); lane l's rebuilt value for block n,
//            register i is its column's entry as it stands.  The 16 x 16
//            instruction would spend 12 of its 16 rows on repeats when 4 heads
//            share a key; the 4 x 4 one has the same rate per product and no
//            repeats.  Each block sums one quarter of d; two lane swaps add
//            the quarters.  No conversion, fp32 products and sums.  The result
//            layout is that of partition_mfma_kernel, whose softmax and value
//            code follow.
//
// Work split: the rotation table is the same for every sequence and head,
// and per token it is larger than the latents (512 bytes for d = 128 against
// 2 r bf16 values, twice).  So the four waves of a workgroup take four
// sequences (b = 4 z + wave) of one kv-head over the same positions: each
// tile's table rows are loaded once, by all four waves together, into LDS
// (two buffers, one barrier per tile), and each wave owns its sequence's
// partition and writes its own records.  The B_K^T fragments serve all four.

template <int R, int D>
struct RGeo {
  static constexpr int kNB = D / 16;   // 16-row blocks of d
  static constexpr int kKC = R / 32;   // 32-row steps of r
  static constexpr int kHalf = D / 32; // blocks per half of d (rotation pairs)
  static constexpr int kRopeEntries = D / 16 * 64;  // 16-byte table pieces per tile
};

// No rotation.
struct RopeNone {};

// A tile's table values in LDS, [pair n][cos, sin][lane]: lane l's cosines
// (sines) of d = 16 n + 4 (l / 16) + i, i < 4, for its token l % 16.
struct RopeLds {
  const u32x4* base;
  int lane;
  __device__ u32x4 cos(int n) const { return base[(2 * n) * 64 + lane]; }
  __device__ u32x4 sin(int n) const { return base[(2 * n + 1) * 64 + lane]; }
};

// head quads of the score instruction: heads 0..3, and 4..7 for G = 8
template <int G>
struct RQuads {
  static constexpr int kQ = G == 8 ? 2 : 1;
};

// B_K^T fragment (n, c) of this lane: held in registers (64 for r = 64,
// d = 128) so the rebuild reads no LDS per tile, or, with 8 heads, whose
// accumulators leave no room for them, read from the LDS copy.
template <int R, int D>
struct FragRegs {
  u32x4 r[D / 16][R / 32];
  __device__ u32x4 at(int n, int c) const { return r[n][c]; }
};
struct FragLds {
  const u32x4* base;
  int lane;
  int kc;
  __device__ u32x4 at(int n, int c) const { return base[(n * kc + c) * 64 + lane]; }
};

// The query operand of the score instruction, q'[head][16 n + 4 (l / 16) + i]
// for quad qh: held in registers, or, with 8 heads (whose accumulators and
// fragments leave no room for them), read from the wave's LDS copy of q'.
template <int G, int D>
struct QfRegs {
  float v[RQuads<G>::kQ][D / 16][4];
  __device__ float at(int qh, int n, int i) const { return v[qh][n][i]; }
};
struct QfLds {
  const float* row[2];  // the lane's q' row of each quad, from column 4 (l / 16)
  __device__ float at(int qh, int n, int i) const { return row[qh][16 * n + i]; }
};

template <int R, int G, int D, class Rope, class Frag, class Qf>
__device__ __forceinline__ void rebuild_scores(const MStep<R, G, 1>& lat, const Rope& rope,
                                               int cb, int ntok, int lane, const Frag& fr,
                                               const Qf& qf, float (&s)[1][4]) {
  using Rg = RGeo<R, D>;
  constexpr int KC = Rg::kKC, NH = Rg::kHalf, QH = RQuads<G>::kQ;
  constexpr bool kRot = !std::is_same<Rope, RopeNone>::value;
  // Per rotary pair of 16-row blocks (n, n + d/32): rebuild both blocks of
  // the tile's keys, transposed, rotate them, and add them into the scores.
  //
  // Scores on v_mfma_f32_4x4x1_16b_f32: block l / 4 is token quad (l % 16) / 4
  // of d-quarter l / 16; its rows are the 4 heads of a quad, its columns the
  // quad's tokens, and each instruction adds one d of the quarter
  // (d = 16 n + 4 (l / 16) + i, lane l's own rebuilt value); then the four
  // quarters are added across lanes.
  // two accumulators per quad (first and second half of each rotary pair),
  // so consecutive score instructions do not wait on each other's results
  f32x4 sd[QH][2];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) sd[qh][0] = sd[qh][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < NH; ++n) {
    f32x4 kd[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int nb = n + hf * NH;
      kd[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 bk = fr.at(nb, c);
        const u32x4 lk = {lat.k[0][c][0], lat.k[0][c][1], lat.k[0][c][2], lat.k[0][c][3]};
        kd[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bk),
                                                         __builtin_bit_cast(bf16x8, lk), kd[hf], 0, 0, 0);
      }
    }
    if constexpr (kRot) {
      const u32x4 cw = rope.cos(n), sw = rope.sin(n);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = __uint_as_float(cw[i]), sn = __uint_as_float(sw[i]);
        const float x = kd[0][i], y = kd[1][i];
        kd[0][i] = x * c - y * sn;
        kd[1][i] = x * sn + y * c;
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int qh = 0; qh < QH; ++qh)
          sd[qh][hf] = __builtin_amdgcn_mfma_f32_4x4x1f32(qf.at(qh, n + hf * NH, i), kd[hf][i], sd[qh][hf], 0, 0, 0);
      }
    }
  }
  float sq[QH][4];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sq[qh][i] = sum_quarters(sd[qh][0][i] + sd[qh][1][i]);
  }
  // lane l keeps heads 4 (l / 16 % 2) + i for G = 8 (the score layout of
  // partition_mfma_kernel), heads i % G otherwise
  const bool hi_half = G == 8 && ((lane >> 4) & 1);
  const int tok = lane & 15;
  const bool masked = cb + tok >= ntok;  // a select, not a branch
  // a select on the two values (a conditional over the two array elements
  // would pick an address at run time and put sq in scratch memory)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x0 = __float_as_uint(sq[0][i]), x1 = __float_as_uint(sq[QH - 1][i]);
    const float x = __uint_as_float(QH == 2 && hi_half ? x1 : x0);
    s[0][i] = masked ? -INFINITY : x;
  }
}

template <int R, int G, int D>
struct RPartLds {
  union {
    uint16_t stage[R * D];                         // B_K[g] as stored, for the gather
    u32x4 rope[2][RGeo<R, D>::kRopeEntries / 64][64];  // table tiles, two buffers
  };
  u32x4 frag[D * R / 8];       // B_K^T fragments [n][c][lane]
  float q[kWaves][G * D];      // q' = qscale * rotate(q, seq_len - 1) of each wave's sequence
  float w[kWaves * 16 * G];
};

template <int R, int G, int D, bool kRot>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void partition_rebuild_kernel(PartitionArgs a) {
  using Mg = MGeo<R, G, 1>;
  using Rg = RGeo<R, D>;
  constexpr int LPR = Mg::kLPR, KC = R / 32, CH = 16;
  constexpr int EPT = Rg::kRopeEntries / kThreads;  // table pieces per thread and tile
  static_assert(Rg::kRopeEntries % kThreads == 0, "table tile split");

  // workgroup: kv-head group hg, partition p, sequences 4 z .. 4 z + 3
  const int p = blockIdx.x, hg = blockIdx.y, z = blockIdx.z;
  const int g = hg * G / a.hps;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = p * a.S;
  int nmax = 0, len = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int bw = kWaves * z + w;
    const int lw = bw < a.B ? min(max(a.seq_lens[bw], 0), a.T) : 0;
    nmax = max(nmax, min(t0 + a.S, lw) - t0);
    len = w == wave ? lw : len;
  }
  if (nmax <= 0) return;  // every sequence of the quad ends before this partition
  len = __builtin_amdgcn_readfirstlane(len);
  const int b = kWaves * z + wave;
  const int bs = min(b, a.B - 1);                  // in range for the address arithmetic
  const int ntok = max(min(t0 + a.S, len) - t0, 0);  // 0: the wave adds and writes nothing

  __shared__ RPartLds<R, G, D> lds;
  const int slot = lane / LPR, cc = lane % LPR;

  const size_t row0 = ((size_t)bs * a.Hkv + g) * (size_t)a.T + (size_t)t0;
  const uint32_t nbytes = (uint32_t)ntok * Mg::kRowBytes;
  const auto rk = make_rsrc(static_cast<const char*>(a.LK) + row0 * Mg::kRowBytes, nbytes);
  const auto rv = make_rsrc(static_cast<const char*>(a.LV) + row0 * Mg::kRowBytes, nbytes);
  const uint32_t koff = (uint32_t)((lane & 15) * Mg::kRowBytes + (lane >> 4) * 16);
  const uint32_t voff = (uint32_t)(slot * Mg::kRowBytes + cc * 16);
  const auto rr = kRot ? make_rsrc(a.rope, (uint32_t)a.T * D * 4u) : make_rsrc(nullptr, 0u);
  // this thread's table pieces e = tid + k * kThreads of a tile: pair n,
  // cos|sin part cs, reader lane l -> row t0 + cb + l % 16, column
  // cs * d/2 + 16 n + 4 (l / 16); rows past the table load zeros
  uint32_t roff[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * kThreads, j = e >> 6, l = e & 63;
    roff[k] = (uint32_t)(((t0 + (l & 15)) * D + (j & 1) * (D / 2) + 16 * (j >> 1) + 4 * (l >> 4)) * 4);
  }

  // ---- prologue: B_K[g] (all threads) and q' of this wave's sequence
  {
    const auto rf = make_rsrc(static_cast<const uint16_t*>(a.BK) + (size_t)g * R * D,
                              (uint32_t)(R * D) * 2u);
    constexpr int kF = R * D / 8 / kThreads;  // 16-byte pieces of B_K per thread
    u32x4 fw[kF];
#pragma unroll
    for (int k = 0; k < kF; ++k)
      fw[k] = __builtin_amdgcn_raw_buffer_load_b128(rf, (int)((tid + k * kThreads) * 16u), 0, 0);
    const size_t q0 = ((size_t)bs * a.Hq + (size_t)hg * G) * D;
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.q) + q0, (uint32_t)(G * D) * 2u);
    // pairs (j, j + D/2) of head h: lane handles pair index lane + 64 k
    constexpr int kPairs = G * D / 2, kPP = (kPairs + 63) / 64;
    uint32_t qlo[kPP], qhi[kPP];
    float rc[kPP], rs[kPP];
#pragma unroll
    for (int k = 0; k < kPP; ++k) {
      const int pi = lane + 64 * k;
      const int h = pi / (D / 2), j = pi - h * (D / 2);
      const bool ok = pi < kPairs;
      qlo[k] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)(ok ? (h * D + j) * 2u & ~3u : kOffNone), 0, 0);
      qhi[k] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)(ok ? (h * D + j + D / 2) * 2u & ~3u : kOffNone), 0, 0);
      rc[k] = 1.f;
      rs[k] = 0.f;
      if constexpr (kRot) {
        const uint32_t row = (uint32_t)max(len - 1, 0) * D * 4u;
        rc[k] = bload4f(rr, row + 4u * j);
        rs[k] = bload4f(rr, row + 4u * (D / 2 + j));
      }
    }
#pragma unroll
    for (int k = 0; k < kF; ++k)
      *reinterpret_cast<u32x4*>(&lds.stage[(tid + k * kThreads) * 8]) = fw[k];
    float* qw = lds.q[wave];
#pragma unroll
    for (int k = 0; k < kPP; ++k) {
      const int pi = lane + 64 * k;
      if (pi < kPairs) {
        const int h = pi / (D / 2), j = pi - h * (D / 2);
        const float x = (j & 1) ? bf16_hi(qlo[k]) : bf16_lo(qlo[k]);
        const float y = (j & 1) ? bf16_hi(qhi[k]) : bf16_lo(qhi[k]);
        qw[h * D + j] = (x * rc[k] - y * rs[k]) * a.qscale;
        qw[h * D + j + D / 2] = (x * rs[k] + y * rc[k]) * a.qscale;
      }
    }
  }
  __syncthreads();
  // B_K^T fragments: fragment (n, c) of lane l = B_K[32 c + 8 (l / 16) + j][16 n + l % 16]
  for (int f = tid; f < D * R / 8; f += kThreads) {
    const int fl = f & 63, nc = f >> 6;
    const int n = nc / KC, c = nc - n * KC;
    const int col = 16 * n + (fl & 15), k0 = 32 * c + 8 * (fl >> 4);
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)lds.stage[(k0 + 2 * j) * D + col] |
             ((uint32_t)lds.stage[(k0 + 2 * j + 1) * D + col] << 16);
    lds.frag[f] = w;
  }
  // query operand of the score instruction: lane l is row l % 4 of its block,
  // head (l % 4) % G of quad qh; instruction (n, i) takes d = 16 n + 4 (l / 16) + i
  using Qf = std::conditional_t<(G < 8), QfRegs<G, D>, QfLds>;
  Qf qf;
  if constexpr (G < 8) {
#pragma unroll
    for (int qh = 0; qh < RQuads<G>::kQ; ++qh) {
      const float* qrow = lds.q[wave] + (4 * qh + (lane & 3) % G) * D + 4 * (lane >> 4);
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qf.v[qh][n][i] = qrow[16 * n + i];
      }
    }
  } else {
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) qf.row[qh] = lds.q[wave] + (4 * qh + (lane & 3)) * D + 4 * (lane >> 4);
  }
  __syncthreads();  // the stage is free: its space holds the table tiles
  using Frag = std::conditional_t<(G < 8), FragRegs<R, D>, FragLds>;
  Frag fr;
  if constexpr (G < 8) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int c = 0; c < KC; ++c) fr.r[n][c] = lds.frag[(n * KC + c) * 64 + lane];
  } else {
    fr = FragLds{lds.frag, lane, KC};
  }

  // ---- the tiles.  Two tiles of latents in flight per wave: the loads of
  // tile k + 2 are issued as soon as tile k is done, so each tile's latency is
  // covered by a whole tile of work.  The table tile k + 1 is loaded into
  // registers during tile k and written to the other LDS buffer at its end.
  // The loop runs to the quad's longest partition (every wave takes part in
  // every barrier); a wave past its own end, or an odd last tile, sees loads
  // that return zeros (outside its buffer's range) and scores masked to -inf,
  // and adds nothing.  The scheduling barriers keep the issue order, which
  // the waits on in-order load returns rely on.
  u32x4 rp[EPT];
  if constexpr (kRot) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) rp[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (int)roff[k], 0, 0);
#pragma unroll
    for (int k = 0; k < EPT; ++k) (&lds.rope[0][0][0])[tid + k * kThreads] = rp[k];
  }
  MStep<R, G, 1> l0, l1;
  load_mstep<R, G, 1>(l0, 0, koff, voff, rk, rv);
  if constexpr (kRot) {
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      rp[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (int)(roff[k] + CH * D * 4u), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_mstep<R, G, 1>(l1, CH, koff, voff, rk, rv);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kRot) __syncthreads();

  float mm[4], ll[4], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mm[i] = -FLT_MAX;
    ll[i] = 0.f;
  }
  float* wl = lds.w + wave * CH * G;
  // one tile: scores, softmax and values; then the next table tile into the
  // other buffer, the loads two tiles ahead, and the barrier
  auto tile = [&](MStep<R, G, 1>& lt, int cb, int buf) {
    float s[1][4];
    if constexpr (kRot)
      rebuild_scores<R, G, D>(lt, RopeLds{&lds.rope[buf][0][0], lane}, cb, ntok, lane, fr, qf, s);
    else
      rebuild_scores<R, G, D>(lt, RopeNone{}, cb, ntok, lane, fr, qf, s);
    softmax_values<R, G, 1>(s, lt, lane, mm, ll, acc, wl);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kRot) {
#pragma unroll
      for (int k = 0; k < EPT; ++k) (&lds.rope[buf ^ 1][0][0])[tid + k * kThreads] = rp[k];
#pragma unroll
      for (int k = 0; k < EPT; ++k)
        rp[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (int)(roff[k] + (uint32_t)(cb + 2 * CH) * D * 4u), 0, 0);
    }
    load_mstep<R, G, 1>(lt, cb + 2 * CH, koff, voff, rk, rv);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kRot) __syncthreads();
  };
  for (int cb = 0; cb < nmax; cb += 2 * CH) {
    tile(l0, cb, 0);
    tile(l1, cb + CH, 1);
  }

  // ---- this wave's records: (acc, m, l) of its G heads
  float m[G], l[G];
#pragma unroll
  for (int i = 0; i < Mg::kHL; ++i) {
    const float x = group_sum<16>(ll[i]);
    l[i] = readlane_f(x, 0);
    m[i] = readlane_f(mm[i], 0);
    if constexpr (G == 8) {
      l[4 + i] = readlane_f(x, 16);
      m[4 + i] = readlane_f(mm[i], 16);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  }
  if (ntok > 0) {
    float* const rec0 = a.ws + ((size_t)b * a.Hq + (size_t)hg * G) * (size_t)a.P * (R + kRecPad);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* rec = rec0 + ((size_t)h * a.P + p) * (R + kRecPad);
      if (slot == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rec[cc * 8 + e] = acc[h][e];
      }
      if (lane == 0) {
        rec[R] = m[h];
        rec[R + 1] = l[h];
      }
    }
  }
}

// ------------------------------------------------------------------ combine
// Second kernel of the decode step: one workgroup per (b, query head) merges
// that head's partial records and projects through B_V.  The kernel boundary
// is what makes every partition's records visible to it: on this multi-XCD
// part an in-kernel hand-off (last-arriving workgroup merges) needs an
// agent-scope fence per workgroup, i.e. an L2 writeback each, which measured
// several times slower than the second launch; records stored write-through
// (device-scope stores, no writeback) with a counter per head still cost
// each workgroup two round trips at its end, 14% on the 256-partition
// long-context workload before any merging.
//
// The kernel is latency-bound, so its loads are issued together, before
// anything waits, as raw buffer loads bounded by their slices with no branch
// around any of them (a load past a slice returns zero):
//   1. each thread loads its pieces of B_V[g] (16 bytes each: a column
//      chunk of every NG-th row, ProjTile below) and its share of the first
//      chunk of the head's records (16 bytes per load) -- speculatively, as
//      the records past seq_len's last partition are never folded;
//   2. the chunk is staged in LDS (further chunks: one round trip each);
//   3. the chunk's reference M (the maximum of the running reference and
//      the chunk's partition maxima; the running sums are rescaled when it
//      moves) and each partition's weight 2^(m_p - M), once per partition;
//      thread (pg, j) then adds w_p acc_p[j] and w_p l_p over partitions
//      pg, pg + NPG, ... in ascending order (NPG = kThreads / r groups),
//      and the NPG group sums, which share M, are added in ascending
//      order: v~ = acc / l;
//   4. thread (rg, c) forms the partial of its column chunk over its rows
//      and the NG partials of each column are added in ascending order.
// Every order is fixed, so results are bitwise reproducible.

// kStage floats of records are staged per round trip: 4096 (16 KB), or
// 16384 (64 KB) for a head with more records than that (a long context cut
// into hundreds of partitions), so that every record of the head arrives in
// one round trip instead of one per 16 KB chunk.
constexpr int kStageSmall = 4096;
constexpr int kStageLarge = 16384;

template <int R, int kStageFloats = kStageSmall>
struct CombineLds {
  static constexpr int kNPG = kThreads / R;                 // partition groups
  static constexpr int kStage = kStageFloats;               // staged floats
  static constexpr int kChunk = kStage / (R + kRecPad);     // partitions per chunk
  float4 stage[kStage / 4];
  float w[kChunk];     // weight 2^(m_p - M) of each staged partition
  float red[kWaves];   // per-wave maxima
  float l[kNPG];
  float v[kNPG * R];
  float vt[R];
};

// Maximum of x over the workgroup (every thread gets it).  `red` is free
// on entry; the caller synchronizes before writing it again.
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  return r;
}

// The projection out[i] = sum_j v~[j] B_V[g][j][i] in 16-byte pieces of B_V
// (ES bytes per element: EPP = 16 / ES columns a piece): thread (rg, c)
// takes column chunk c of rows rg, rg + NG, ... (each set), so a wave's
// loads cover whole consecutive rows; the NG partials of a column are added
// in ascending rg.  Rows past r load zeros (buffer bounds) and are skipped.
template <int R, int D, int ES, int NSET>
struct ProjTile {
  static constexpr int kEPP = 16 / ES;              // columns per piece
  static constexpr int kCPR = D / kEPP;             // pieces per row
  static constexpr int kNG = kThreads / kCPR;       // row groups
  static constexpr int kRPT = (R + kNG - 1) / kNG;  // rows per thread (a set)
  static constexpr int kTP = kRPT * NSET;           // pieces per thread
  static constexpr int kPB = kTP < 16 ? kTP : 16;   // pieces per batch in flight
  static_assert(kCPR * kNG == kThreads && kTP % kPB == 0, "projection tiling");

  __device__ static void load(const __amdgpu_buffer_rsrc_t (&rbv)[NSET], int tid, int bt,
                              u32x4 (&bw)[kPB]) {
    const int c = tid % kCPR, rg = tid / kCPR;
#pragma unroll
    for (int q = 0; q < kPB; ++q) {
      const int qq = bt * kPB + q, st = qq / kRPT, row = rg + kNG * (qq % kRPT);
      bw[q] = __builtin_amdgcn_raw_buffer_load_b128(rbv[st], row * D * ES + c * 16, 0, 0);
    }
  }

  __device__ static void fma(const float* const (&vts)[2], int tid, int bt,
                             const u32x4 (&bw)[kPB], int fdt, float (&o)[kEPP]) {
    const int rg = tid / kCPR;
#pragma unroll
    for (int q = 0; q < kPB; ++q) {
      const int qq = bt * kPB + q, st = qq / kRPT, row = rg + kNG * (qq % kRPT);
      if (row < R) {
        const float v = vts[st][row];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t w = bw[q][k];
          if constexpr (ES == 4) {
            o[k] = fmaf(v, __uint_as_float(w), o[k]);
          } else {
            const bool bf = fdt == LRATTN_BF16;
            o[2 * k] = fmaf(v, bf ? bf16_lo(w) : f16_lo(w), o[2 * k]);
            o[2 * k + 1] = fmaf(v, bf ? bf16_hi(w) : f16_hi(w), o[2 * k + 1]);
          }
        }
      }
    }
  }
};

// 16-byte loads of records [p0, p0 + n) of one head into this thread's
// share of the stage (slots tid + k * kThreads).
template <int R, int kStageFloats>
__device__ __forceinline__ void load_chunk(const float* rec0, int p0, int n,
                                           float4 (&v4)[kStageFloats / 4 / kThreads]) {
  constexpr int RS = R + kRecPad;
  const auto rr = make_rsrc(rec0 + (size_t)p0 * RS, (uint32_t)n * RS * 4u);
#pragma unroll
  for (int k = 0; k < kStageFloats / 4 / kThreads; ++k) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rr, (int)((threadIdx.x + k * kThreads) * 16u), 0, 0);
    v4[k] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                        __uint_as_float(w[3]));
  }
}

// Two factor sets (kModal: image block, then text; AttentionPack page,
// section 2.A compresses the modalities apart): the records of each set fold
// into their own latent-space sum under the common running max and
// denominator, and out = (acc_img . B_V_img[g] + acc_txt . B_V_txt[g]) / L.
template <int R, int D, bool kModal, int ES, int kStageFloats = kStageSmall>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void combine_kernel(CombineArgs a) {
  using CL = CombineLds<R, kStageFloats>;
  constexpr int RS = R + kRecPad;
  constexpr int kNPG = CL::kNPG, kChunk = CL::kChunk;
  constexpr int kPer = CL::kStage / 4 / kThreads;
  constexpr int NSET = kModal ? 2 : 1;
  using PT = ProjTile<R, D, ES, NSET>;
  static_assert(PT::kNG * D <= CL::kStage, "projection partials fit the stage");
  const int hq = blockIdx.x, b = blockIdx.y;
  // B_V block: per kv-head, or per query head (shared latent streams)
  const int g = a.factor_per_head ? hq : hq / (a.Hq / a.Hkv);
  const int tid = threadIdx.x;
  const MergeArgs& mg = a.merge;

  // 1. B_V[g] pieces of this thread (PT::load): 16-byte pieces, column
  //    chunk c of rows rg, rg + NG, ...
  const int fdt = mg.f_dtype;
  // dense cache (no B_V, r == d): an empty resource, every load returns zero
  const bool dense = mg.BV == nullptr;
  __amdgpu_buffer_rsrc_t rbv[NSET];
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    const void* bv = st == 0 ? mg.BV : a.BV1;
    rbv[st] = dense ? make_rsrc(nullptr, 0u)
                    : make_rsrc(static_cast<const char*>(bv) + (size_t)g * R * D * ES,
                                (uint32_t)(R * D * ES));
  }
  u32x4 bw[PT::kPB];
  PT::load(rbv, tid, 0, bw);
  const float* rec0 = a.ws + ((size_t)b * a.Hq + hq) * (size_t)a.P * RS;
  float4 v4[kPer];
  load_chunk<R, kStageFloats>(rec0, 0, min(kChunk, a.P), v4);

  // No early exit for an empty sequence (np == 0): it runs the same steps
  // with nothing to fold and writes a zero row.  A branch here would let the
  // compiler move the loads above behind the seq_lens round trip.
  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  // record ranges [beg, beg + cnt) of each set
  int beg[NSET], cnt[NSET];
  if constexpr (kModal) {
    const int ni = min(len, a.n_img);
    beg[0] = 0;
    cnt[0] = (ni + a.S_img - 1) / a.S_img;
    beg[1] = a.P_img;
    cnt[1] = (max(len - a.n_img, 0) + a.S - 1) / a.S;
  } else {
    beg[0] = 0;
    cnt[0] = (len + a.S - 1) / a.S;
  }
  int np = 0;
#pragma unroll
  for (int st = 0; st < NSET; ++st) np += cnt[st];
  const size_t out_row0 = ((size_t)b * a.Hq + hq) * D;

  __shared__ CL sm;
  __shared__ float vt1[kModal ? kNPG * R + R : 1];  // second set: group sums, then v~
  const float* stage = reinterpret_cast<const float*>(sm.stage);
  // kNPG * R <= kThreads (r = 48 leaves 16 threads without a group)
  const int pg = tid / R, j = tid - pg * R;
  const bool folds = pg < kNPG;
  // One reference M for every partial of a staged chunk: the running
  // maximum of the partitions' maxima, moved (and the sums rescaled) only
  // between chunks.  Within a chunk each partition's weight 2^(m_p - M) is
  // computed once, and the sums are plain weighted sums in a fixed order.
  float M = -FLT_MAX, L = 0.f, acc[NSET];
#pragma unroll
  for (int st = 0; st < NSET; ++st) acc[st] = 0.f;
#pragma unroll
  for (int st = 0; st < NSET; ++st) {
    for (int p0 = 0; p0 < cnt[st]; p0 += kChunk) {
      if (st > 0 || p0 > 0) {
        __syncthreads();  // previous chunk consumed
        load_chunk<R, kStageFloats>(rec0, beg[st] + p0, min(kChunk, cnt[st] - p0), v4);
      }
      // 2. stage (every slot is written: zeros past the chunk)
#pragma unroll
      for (int k = 0; k < kPer; ++k) sm.stage[tid + k * kThreads] = v4[k];
      __syncthreads();
      // 3. the chunk's reference, its weights, then the weighted sums of
      //    partitions pg, pg + NPG, ... into set st
      const int pc = min(kChunk, cnt[st] - p0);
      float mx = -FLT_MAX;
      for (int i = tid; i < pc; i += kThreads) mx = fmaxf(mx, stage[i * RS + R]);
      const float Mn = fmaxf(M, block_max(mx, sm.red));
      for (int i = tid; i < pc; i += kThreads) sm.w[i] = fast_exp2(stage[i * RS + R] - Mn);
      __syncthreads();
      const float sc = fast_exp2(M - Mn);  // 0 on the first chunk
      L *= sc;
#pragma unroll
      for (int u = 0; u < NSET; ++u) acc[u] *= sc;
      M = Mn;
      if (folds) {
#pragma unroll 4
        for (int pp = pg; pp < pc; pp += kNPG) {
          const float wp = sm.w[pp];
          const float* rec = stage + pp * RS;
          acc[st] = fmaf(wp, rec[j], acc[st]);
          L = fmaf(wp, rec[R + 1], L);
        }
      }
    }
  }
  // the groups' sums share M: the row is their plain sum, in ascending group
  if (folds) {
    sm.v[tid] = acc[0];
    if constexpr (kModal) vt1[tid] = acc[1];
    if (j == 0) sm.l[pg] = L;
  }
  __syncthreads();
  if (tid < R) {
    float s0 = sm.v[tid], s1 = 0.f, Lt = sm.l[0];
    if constexpr (kModal) s1 = vt1[tid];
#pragma unroll
    for (int q = 1; q < kNPG; ++q) {
      s0 += sm.v[q * R + tid];
      if constexpr (kModal) s1 += vt1[q * R + tid];
      Lt += sm.l[q];
    }
    sm.vt[tid] = np > 0 ? s0 / Lt : 0.f;
    if constexpr (kModal) vt1[kNPG * R + tid] = np > 0 ? s1 / Lt : 0.f;
    // the row's final reference and denominator (attention weights of the
    // step: 2^(logit - M) / L)
    if (a.stats != nullptr && tid == 0) {
      a.stats[((size_t)b * a.Hq + hq) * 2] = M;
      a.stats[((size_t)b * a.Hq + hq) * 2 + 1] = Lt;
    }
  }
  __syncthreads();

  // 4. partial of out[c EPP .. + EPP) over the thread's rows (each set), in
  //    the stage (free after the fold): part[rg][column]
  float* part = reinterpret_cast<float*>(sm.stage);
  {
    const float* vts[2] = {sm.vt, kModal ? vt1 + kNPG * R : sm.vt};
    float o[PT::kEPP];
#pragma unroll
    for (int e = 0; e < PT::kEPP; ++e) o[e] = 0.f;
#pragma unroll
    for (int bt = 0; bt < PT::kTP / PT::kPB; ++bt) {
      if (bt > 0) {
        __syncthreads();  // a scheduling boundary: the batches never overlap in registers
        PT::load(rbv, tid, bt, bw);
      }
      PT::fma(vts, tid, bt, bw, fdt, o);
    }
    const int c = tid % PT::kCPR, rg = tid / PT::kCPR;
#pragma unroll
    for (int e = 0; e < PT::kEPP; e += 4)
      *reinterpret_cast<float4*>(part + rg * D + c * PT::kEPP + e) =
          make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
  }
  __syncthreads();
  if (tid < D) {
    float r = part[tid];
#pragma unroll
    for (int q = 1; q < PT::kNG; ++q) r += part[q * D + tid];
    if (dense) r = tid < R ? sm.vt[tid] : 0.f;  // r == d: v~ is the output row
    if (np == 0) r = 0.f;       // attention over no tokens: zero output
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

// The matrix-core score kernel serves bf16 latents, r a multiple of 32 and
// 4 or 8 heads per kv-head.
constexpr bool mfma_scores(int latent_dtype, int rank, int group) {
  return latent_dtype == LRATTN_BF16 && rank % 32 == 0 &&
         (group == 4 || group == 8);
}

// Head groups sharing a latent stream (a.xcd_group) keep the latents in L2
// for each other: cache policy 0 instead of non-temporal, for groups of 4 or
// 8 heads (the shared-stream groups; smaller groups keep the default).
template <class LT, int R>
hipError_t launch_pg(int group, const PartitionArgs& a, hipStream_t s) {
  const dim3 block(kThreads);
  if (a.BK1 != nullptr) {
    // two factor sets: grid (HG, B, P), see tile_of
    const dim3 grid(a.HG, a.B, a.P);
    constexpr int X = kNonTemporal;
    if constexpr (mfma_scores(std::is_same<LT, LatBF16>::value ? LRATTN_BF16 : -1, R, 4)) {
      if (group == 4) {
        hipLaunchKernelGGL((partition_mfma_kernel<R, 4, X, true>), grid, block, 0, s, a);
        return hipGetLastError();
      }
      if (group == 8) {
        hipLaunchKernelGGL((partition_mfma_kernel<R, 8, X, true>), grid, block, 0, s, a);
        return hipGetLastError();
      }
    }
    switch (group) {
      case 1: hipLaunchKernelGGL((partition_kernel<LT, R, 1, X, false, true>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((partition_kernel<LT, R, 2, X, false, true>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((partition_kernel<LT, R, 4, X, false, true>), grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL((partition_kernel<LT, R, 8, X, false, true>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid = a.xcd_group ? dim3(8 * a.HG * ((a.P * a.B + 7) / 8)) : dim3(a.P, a.HG, a.B);
  const bool keep = a.xcd_group != 0;
  if constexpr (mfma_scores(std::is_same<LT, LatBF16>::value ? LRATTN_BF16 : -1, R, 4)) {
    if (group == 4) {
      if (keep) hipLaunchKernelGGL((partition_mfma_kernel<R, 4, 0>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_mfma_kernel<R, 4>), grid, block, 0, s, a);
      return hipGetLastError();
    }
    if (group == 8) {
      if (keep) hipLaunchKernelGGL((partition_mfma_kernel<R, 8, 0>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_mfma_kernel<R, 8>), grid, block, 0, s, a);
      return hipGetLastError();
    }
  }
  switch (group) {
    case 1: hipLaunchKernelGGL((partition_kernel<LT, R, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((partition_kernel<LT, R, 2>), grid, block, 0, s, a); break;
    case 4:
      if (keep) hipLaunchKernelGGL((partition_kernel<LT, R, 4, 0>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_kernel<LT, R, 4>), grid, block, 0, s, a);
      break;
    case 8:
      if (keep) hipLaunchKernelGGL((partition_kernel<LT, R, 8, 0>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_kernel<LT, R, 8>), grid, block, 0, s, a);
      break;
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

// Attention-aware rank: the VALU partition kernel with per-row rank masks
// and logits output, for the shapes of adaptive_supported.
template <class LT, int R>
hipError_t launch_ag(int group, const PartitionArgs& a, hipStream_t s) {
  const dim3 grid(a.P, a.HG, a.B), block(kThreads);
  // bf16 latents with 4 or 8 heads per kv-head and r a multiple of 32: the
  // matrix-core kernel, as for the plain decode (the kCut form when low_rank
  // splits a 16-byte piece)
  if constexpr (mfma_scores(std::is_same<LT, LatBF16>::value ? LRATTN_BF16 : -1, R, 4)) {
    constexpr int X = kNonTemporal;
    const bool cut = a.low_rank % 8 != 0;
    if (group == 4) {
      if (cut) hipLaunchKernelGGL((partition_mfma_kernel<R, 4, X, false, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_mfma_kernel<R, 4, X, false, true>), grid, block, 0, s, a);
      return hipGetLastError();
    }
    if (group == 8) {
      if (cut) hipLaunchKernelGGL((partition_mfma_kernel<R, 8, X, false, true, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_mfma_kernel<R, 8, X, false, true>), grid, block, 0, s, a);
      return hipGetLastError();
    }
  }
  // the VALU form for the other shapes only: where the matrix-core kernel
  // takes 4 and 8 heads, the VALU form of those groups is not built
  constexpr bool kMfmaShape =
      mfma_scores(std::is_same<LT, LatBF16>::value ? LRATTN_BF16 : -1, R, 4);
  switch (group) {
    case 1: hipLaunchKernelGGL((partition_kernel<LT, R, 1, kNonTemporal, true>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((partition_kernel<LT, R, 2, kNonTemporal, true>), grid, block, 0, s, a); break;
    case 4:
      if constexpr (!kMfmaShape) {
        hipLaunchKernelGGL((partition_kernel<LT, R, 4, kNonTemporal, true>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case 8:
      if constexpr (!kMfmaShape) {
        hipLaunchKernelGGL((partition_kernel<LT, R, 8, kNonTemporal, true>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int R, int D>
hipError_t launch_rg(int group, bool rot, const PartitionArgs& a, hipStream_t s) {
  // partitions x kv-head groups x quads of sequences (one wave per sequence)
  const dim3 grid(a.P, a.HG, (a.B + kWaves - 1) / kWaves);
  const dim3 block(kThreads);
  switch (group) {
    case 1:
      if (rot) hipLaunchKernelGGL((partition_rebuild_kernel<R, 1, D, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_rebuild_kernel<R, 1, D, false>), grid, block, 0, s, a);
      break;
    case 2:
      if (rot) hipLaunchKernelGGL((partition_rebuild_kernel<R, 2, D, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_rebuild_kernel<R, 2, D, false>), grid, block, 0, s, a);
      break;
    case 4:
      if (rot) hipLaunchKernelGGL((partition_rebuild_kernel<R, 4, D, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_rebuild_kernel<R, 4, D, false>), grid, block, 0, s, a);
      break;
    case 8:
      if (rot) hipLaunchKernelGGL((partition_rebuild_kernel<R, 8, D, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((partition_rebuild_kernel<R, 8, D, false>), grid, block, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int R, int ES>
hipError_t launch_cge(const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.Hq, a.B), block(kThreads);
  // two factor sets: d <= 128 and r <= 64 (modal_supported)
  if (a.BV1 != nullptr) {
    if constexpr (R <= 64) {
      switch (a.d) {
        case 64: hipLaunchKernelGGL((combine_kernel<R, 64, true, ES>), grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL((combine_kernel<R, 128, true, ES>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if ((int64_t)a.P * (R + kRecPad) > kStageSmall) {
    // every record of a head in one round trip (64 KB stage)
    constexpr int K = kStageLarge;
    switch (a.d) {
      case 64: hipLaunchKernelGGL((combine_kernel<R, 64, false, ES, K>), grid, block, 0, s, a); break;
      case 128: hipLaunchKernelGGL((combine_kernel<R, 128, false, ES, K>), grid, block, 0, s, a); break;
      case 256: hipLaunchKernelGGL((combine_kernel<R, 256, false, ES, K>), grid, block, 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.d) {
    case 64: hipLaunchKernelGGL((combine_kernel<R, 64, false, ES>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((combine_kernel<R, 128, false, ES>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((combine_kernel<R, 256, false, ES>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// factor element size: 4 bytes (fp32) or 2 (bf16, fp16)
template <int R>
hipError_t launch_cg(const CombineArgs& a, hipStream_t s) {
  return a.merge.f_dtype == LRATTN_F32 ? launch_cge<R, 4>(a, s) : launch_cge<R, 2>(a, s);
}

}  // namespace

bool modal_supported(int head_dim, int rank) {
  return (head_dim == 64 || head_dim == 128) && rank <= 64;
}

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

const char* partition_kernel_name(int latent_dtype, int rank, int group) {
  if (!partition_supported(latent_dtype, rank, group)) return "";
  return mfma_scores(latent_dtype, rank, group) ? "partition_mfma_kernel" : "partition_kernel";
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

bool adaptive_supported(int latent_dtype, int rank, int group) {
  const bool g = group == 1 || group == 2 || group == 4 || group == 8;
  switch (latent_dtype) {
    case LRATTN_F32: return rank == 16 && group == 1;
    case LRATTN_BF16: return (rank == 32 || rank == 48 || rank == 64 || rank == 128) && g;
    case LRATTN_I8: return rank == 32 && (group == 1 || group == 4);
    default: return false;
  }
}

const char* adaptive_kernel_name(int latent_dtype, int rank, int group) {
  if (!adaptive_supported(latent_dtype, rank, group)) return "";
  return mfma_scores(latent_dtype, rank, group) ? "partition_mfma_kernel" : "partition_kernel";
}

hipError_t launch_adaptive(int latent_dtype, int rank, int group, const PartitionArgs& a,
                           hipStream_t s) {
  if (!adaptive_supported(latent_dtype, rank, group)) return hipErrorInvalidValue;
  if (latent_dtype == LRATTN_F32) return launch_ag<LatF32, 16>(1, a, s);
  if (latent_dtype == LRATTN_I8) return launch_ag<LatI8, 32>(group, a, s);
  switch (rank) {
    case 32: return launch_ag<LatBF16, 32>(group, a, s);
    case 48: return launch_ag<LatBF16, 48>(group, a, s);
    case 128: return launch_ag<LatBF16, 128>(group, a, s);
    default: return launch_ag<LatBF16, 64>(group, a, s);
  }
}

bool rebuild_supported(int head_dim, int rank, int group) {
  return (head_dim == 64 || head_dim == 128) && (rank == 32 || rank == 64) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_rebuild(int head_dim, int rank, int group, const PartitionArgs& a,
                          hipStream_t s) {
  const bool rot = a.rope != nullptr;
  if (head_dim == 64 && rank == 32) return launch_rg<32, 64>(group, rot, a, s);
  if (head_dim == 64 && rank == 64) return launch_rg<64, 64>(group, rot, a, s);
  if (head_dim == 128 && rank == 32) return launch_rg<32, 128>(group, rot, a, s);
  if (head_dim == 128 && rank == 64) return launch_rg<64, 128>(group, rot, a, s);
  return hipErrorInvalidValue;
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
