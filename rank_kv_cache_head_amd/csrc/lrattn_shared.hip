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
// is streamed once per thread, 256 bytes per round, and reused across those
// sequences; the query rows sit in LDS.  Every product is exact in fp32 and
// the sums run over i in increasing order.
#include <float.h>

#include "lrattn.h"
#include "lrattn_device.hpp"
#include "lrattn_internal.hpp"
#include "lrattn_shared.hpp"

namespace lrattn {
namespace {

constexpr int kAbsorbPieces = 16;  // 16-byte pieces of a factor row per round

// The elements of one 16-byte piece as fp32 (4 for fp32, 8 for 16-bit types).
template <int DT>
__device__ __forceinline__ void unpack_piece(const u32x4& w, float (&f)[DT == LRATTN_F32 ? 4 : 8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (DT == LRATTN_F32) {
      f[k] = __uint_as_float(w[k]);
    } else if constexpr (DT == LRATTN_BF16) {
      f[2 * k] = __uint_as_float(w[k] << 16);
      f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    } else {
      f[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xffffu));
      f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
    }
  }
}

template <int DT>
__device__ __forceinline__ void stage_q_piece(const u32x4& w, float* dst) {
  float f[DT == LRATTN_F32 ? 4 : 8];
  unpack_piece<DT>(w, f);
#pragma unroll
  for (int e = 0; e < (DT == LRATTN_F32 ? 4 : 8); ++e) dst[e] = f[e];
}

// Every load is issued before anything waits: the first round of the
// factor row, then the block's query rows (16-byte pieces, at most two per
// thread), so the kernel costs about one memory round trip.  Query rows
// past the batch load zeros (buffer bounds); pieces past a factor row are
// loaded (the next row, or zeros past the block) and never used.
template <int R, int FT>
__device__ __forceinline__ void absorb_body(const AbsorbHeadsArgs& a) {
  constexpr int SB = 8;                      // sequences per workgroup
  constexpr int TPJ = kThreads / R;          // threads per latent coordinate
  constexpr int KPT = (SB + TPJ - 1) / TPJ;  // sequences per thread
  constexpr int ES = FT == LRATTN_F32 ? 4 : 2;
  constexpr int EPP = 16 / ES;  // factor elements per piece
  const int h = blockIdx.x, b0 = blockIdx.y * SB;
  const int tid = threadIdx.x, j = tid % R, s0 = tid / R;
  const int d = a.d, npieces = d / EPP;
  // the head's factor block (a wave-uniform resource); row j at j d ES bytes
  const auto rb = make_rsrc(static_cast<const char*>(a.BK) + (size_t)h * R * d * ES,
                            (uint32_t)(R * d * ES));
  u32x4 w[kAbsorbPieces];
  auto load_round = [&](int r0) {
#pragma unroll
    for (int k = 0; k < kAbsorbPieces; ++k)
      w[k] = __builtin_amdgcn_raw_buffer_load_b128(
          rb, j * d * ES + (r0 * kAbsorbPieces + k) * 16, 0, 0);
  };
  load_round(0);

  __shared__ float qs[SB][kMaxHeadDim];
  {
    const int qes = a.q_dtype == LRATTN_F32 ? 4 : 2;
    const int qpr = d * qes / 16;  // pieces per query row
    const int nb = min(SB, a.B - b0);
    const uint32_t qrow = (uint32_t)a.Hq * d * qes;  // bytes between sequences
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + ((size_t)b0 * a.Hq + h) * d * qes,
                              (uint32_t)(nb - 1) * qrow + (uint32_t)(d * qes));
    u32x4 qw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + k * kThreads, sq = e / qpr, c = e - sq * qpr;
      const uint32_t off = sq < nb ? (uint32_t)sq * qrow + (uint32_t)c * 16u : kOffNone;
      qw[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + k * kThreads, sq = e / qpr, c = e - sq * qpr;
      if (sq < SB) {
        if (a.q_dtype == LRATTN_F32) stage_q_piece<LRATTN_F32>(qw[k], &qs[sq][4 * c]);
        else if (a.q_dtype == LRATTN_BF16) stage_q_piece<LRATTN_BF16>(qw[k], &qs[sq][8 * c]);
        else stage_q_piece<LRATTN_F16>(qw[k], &qs[sq][8 * c]);
      }
    }
  }
  __syncthreads();
  if (s0 >= TPJ) return;  // r = 48: 16 threads without a coordinate

  // acc[m] = sum_i qs[s0 + m TPJ][i] * B_K[h][j][i], i in increasing order
  float acc[KPT];
#pragma unroll
  for (int m = 0; m < KPT; ++m) acc[m] = 0.f;
  for (int r0 = 0; r0 * kAbsorbPieces < npieces; ++r0) {
    if (r0 > 0) {
      load_round(r0);
      __builtin_amdgcn_sched_barrier(0);  // the round's loads ahead of its arithmetic
    }
#pragma unroll
    for (int k = 0; k < kAbsorbPieces; ++k) {
      const int pc = r0 * kAbsorbPieces + k;
      if (pc < npieces) {
        float f[EPP];
        unpack_piece<FT>(w[k], f);
#pragma unroll
        for (int m = 0; m < KPT; ++m) {
          const int sq = s0 + m * TPJ;
          if (sq < SB) {
#pragma unroll
            for (int e = 0; e < EPP; ++e) acc[m] = fmaf(qs[sq][pc * EPP + e], f[e], acc[m]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int sq = s0 + m * TPJ, b = b0 + sq;
    if (sq < SB && b < a.B) a.qt[((size_t)b * a.Hq + h) * R + j] = acc[m] * a.qscale;
  }
}

template <int R>
__global__ __launch_bounds__(kThreads) void absorb_heads_kernel(AbsorbHeadsArgs a) {
  if (a.f_dtype == LRATTN_F32) absorb_body<R, LRATTN_F32>(a);
  else if (a.f_dtype == LRATTN_BF16) absorb_body<R, LRATTN_BF16>(a);
  else absorb_body<R, LRATTN_F16>(a);
}

template <int R>
hipError_t launch_r(const AbsorbHeadsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((absorb_heads_kernel<R>), dim3(a.Hq, (a.B + 7) / 8), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------- one pass over a shared stream
// AttentionPack page, section 2.A: all heads read the same compressed rows.
// Reading them once per head group multiplies the stream's traffic, and the
// value sums of many heads (heads x r accumulators) are more than the VALU
// can keep up with.  This kernel reads each tile once for up to 64 heads
// (NHB blocks of 16) and runs both products on the matrix cores:
//
//   scores  S (16 heads x 16 tokens) = q~ . L_K^T with v_mfma_f32_16x16x32_bf16,
//           q~ split exactly into three bf16 terms (the latents are bf16, so
//           every product is exact and the sums are fp32);
//   values  acc (16 heads x 16 coordinates) += P (16 heads x 32 tokens) .
//           L_V (32 tokens x 16 coordinates), the weights P split into two
//           bf16 terms (relative error below 2^-16).  The contraction runs
//           over tokens, so L_V is needed with tokens contiguous: the
//           workgroup stages each 64-token tile of L_V in LDS transposed
//           ([coordinate][token], two buffers, one barrier per tile), and P
//           goes through a small LDS tile per wave to the operand layout.
//
// Workgroup: one (sequence, stream, group of up to 16 NHB heads, partition),
// 2 NHB waves; wave w takes head block w % NHB (16 heads) and token half
// w / NHB of every 64-token step; the two halves are merged at the end
// (fixed order).  Waves 0-3 stage the tiles.  Scores and value accumulators
// share one layout (lane l, register i: head 4 (l / 16) + i), so the lazily
// moved softmax reference and its rescale stay within a lane.

namespace {

constexpr int kOnceStep = 64;            // tokens per step (32 per wave)
constexpr int kVtStride = 144;           // bytes per transposed V row: 64 tokens + pad
constexpr int kPStride = 36;             // floats per P row: 32 tokens + pad

// Transposed L_V row `row` keeps its tokens XOR 8 ((row / 8) % 8) (whole
// 8-token chunks move): a staging write (at r = 128, 16 rows 8 apart with 4
// consecutive tokens each) then spreads over the banks instead of hitting
// one group, and an operand read (8 consecutive tokens of one row) stays
// one contiguous 16-byte piece.
__device__ __forceinline__ int vt_swizzle(int row) { return 8 * ((row >> 3) & 7); }

template <int R, int NHB>
struct OnceLds {
  static constexpr int kKStride = 2 * R + 16;  // bytes per K row: r bf16 + pad
  alignas(16) unsigned char kt[2][kOnceStep * kKStride];  // L_K tiles [token][coordinate]
  alignas(16) unsigned char vt[2][R * kVtStride];         // L_V tiles [coordinate][token]
  alignas(16) float pw[2 * NHB][16 * kPStride];           // per wave: P [head][token]
  // the final merge reuses both K buffers: [head block][16 heads][R], m, l
  static_assert(NHB * 16 * (R + 2) * 4 <= 2 * kOnceStep * kKStride, "merge area");
};

// Two waves per SIMD: at R = 128 the registers fit 256 without spills, and
// with NHB = 2 two workgroups' LDS (2 x 79 KB) fit a CU, so a CU can run a
// second workgroup while the first waits on memory.
template <int R, int NHB>
__global__ __launch_bounds__(128 * NHB) __attribute__((amdgpu_waves_per_eu(2)))
void shared_once_kernel(SharedOnceArgs a) {
  constexpr int KC = R / 32;          // 32-wide steps of r (scores)
  constexpr int NBV = R / 16;         // 16-wide blocks of r (values)
  constexpr int RowB = 2 * R;         // bytes per latent row
  constexpr int KS = OnceLds<R, NHB>::kKStride;
  constexpr int KV = kOnceStep * RowB / 16 / 256;  // 16-byte pieces per thread, tile and K|V
  const int p = blockIdx.x, b = blockIdx.z;
  constexpr int GH = 16 * NHB;        // heads per group
  const int nh = a.Hq / a.S, hgs = (nh + GH - 1) / GH;  // the last group may be partial
  const int s = blockIdx.y / hgs, hg = blockIdx.y % hgs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = wave % NHB, th = wave / NHB;
  const bool stager = NHB == 2 || wave < 4;  // waves 0-3 stage the tiles
  const int len = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.T));
  const int t0 = p * a.Stok;
  const int t1 = min(t0 + a.Stok, len);
  if (t0 >= t1) return;  // partition past the sequence: nothing to write
  const int ntok = t1 - t0;
  const int head0 = s * nh + hg * GH + 16 * hb;  // first head of this wave's block
  // heads of the block that exist (a partial last group: q~ rows past them
  // load zeros, their records are not written)
  const int nvalid = min(max(nh - hg * GH - 16 * hb, 0), 16);

  __shared__ OnceLds<R, NHB> lds;
  const size_t row0 = ((size_t)b * a.S + s) * (size_t)a.T + (size_t)t0;
  const uint32_t nbytes = (uint32_t)ntok * RowB;
  const auto rk = make_rsrc(static_cast<const char*>(a.LK) + row0 * RowB, nbytes);
  const auto rv = make_rsrc(static_cast<const char*>(a.LV) + row0 * RowB, nbytes);
  // Staging: piece k of thread t (t < 256) is piece 256 k + t of the tile's
  // 16-byte pieces in memory order (CPR = r / 8 pieces a row), so every load
  // instruction reads 1 KB of consecutive rows (16 rows x 64 bytes per
  // instruction streamed 14% slower).  K goes to LDS as it is (rows padded
  // by 16 bytes: the score operand reads of 16 rows at one column are
  // conflict-free); V goes transposed (vt_swizzle).  Waves past the fourth
  // load nothing (an offset past the buffer: zeros, no memory access) and
  // write nothing.
  constexpr int CPR = RowB / 16;
  const uint32_t soff = stager ? (uint32_t)(tid & 255) * 16u : kOffNone;
  struct Tile {
    u32x4 k[KV], v[KV];
  };
  auto load_tile = [&](Tile& tl, int cb) {
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const uint32_t off = stager ? soff + (uint32_t)cb * RowB + 4096u * k : kOffNone;
      tl.k[k] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0, 2);
      tl.v[k] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, 2);
    }
  };
  auto stage_tile = [&](const Tile& tl, int buf) {
    if (!stager) return;
    uint16_t* vt = reinterpret_cast<uint16_t*>(lds.vt[buf]);
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int pc = 256 * k + (tid & 255), tk = pc / CPR, cg = pc % CPR, col = 8 * cg;
      *reinterpret_cast<u32x4*>(lds.kt[buf] + tk * KS + cg * 16) = tl.k[k];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = col + j;
        vt[row * (kVtStride / 2) + (tk ^ vt_swizzle(row))] = (uint16_t)(tl.v[k][j / 2] >> (16 * (j & 1)));
      }
    }
  };

  // ---- prologue: q~ of the wave's 16 heads (A operands), the first tiles
  Tile ta, tb;
  bf16x8 qa[3][KC];
  {
    const auto rq = make_rsrc(a.qt + ((size_t)b * a.Hq + head0) * R, (uint32_t)nvalid * R * 4u);
    u32x4 qw[KC][2];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        qw[c][h] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (int)(((lane & 15) * R + 32 * c + 8 * (lane >> 4) + 4 * h) * 4u), 0, 0);
    }
    load_tile(ta, 0);
    load_tile(tb, kOnceStep);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(qw[c][j / 4][j % 4]);
      bf16x8 t3[3];
      split3x8(x, t3);
#pragma unroll
      for (int term = 0; term < 3; ++term) qa[term][c] = t3[term];
    }
    stage_tile(ta, 0);
  }
  __syncthreads();

  f32x4 acc[NBV];
#pragma unroll
  for (int n = 0; n < NBV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mm[4], ll[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mm[i] = -FLT_MAX;
    ll[i] = 0.f;
  }
  float* pw = lds.pw[wave];
  // One 64-token step at cb from LDS buffer buf: the tile two steps ahead is
  // requested into tn, the next step's (requested a step earlier, in tp) is
  // staged into the other buffer at the end, so every latent load has a
  // whole step of work to arrive and no operand waits on memory.  The loop
  // runs whole pairs of steps; a step past the partition sees zeros and
  // masked scores and adds nothing.
  auto step = [&](int cb, int buf, Tile& tn, const Tile& tp) {
    load_tile(tn, cb + 2 * kOnceStep);
    // scores of the wave's two 16-token tiles (B operand: token l % 16,
    // columns 32 c + 8 (l / 16) .. + 7, from the K tile)
    const unsigned char* kt = lds.kt[buf];
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 kb = *reinterpret_cast<const u32x4*>(
            kt + (32 * th + 16 * t + (lane & 15)) * KS + 64 * c + 16 * (lane >> 4));
#pragma unroll
        for (int term = 0; term < 3; ++term)
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              qa[term][c], __builtin_bit_cast(bf16x8, kb), sc[t], 0, 0, 0);
      }
    }
    // mask, then the lazily moved reference per head (lanes with equal l / 16)
    float sv[2][4];
    bool need = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool masked = cb + 32 * th + 16 * t + (lane & 15) >= ntok;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[t][i] = masked ? -INFINITY : sc[t][i];
        need |= sv[t][i] > mm[i] + kLazyLog2;
      }
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = row_max16(fmaxf(sv[0][i], sv[1][i]));
        const float nm = x > mm[i] + kLazyLog2 ? x : mm[i];
        const float corr = fast_exp2(mm[i] - nm);
        mm[i] = nm;
        ll[i] *= corr;
#pragma unroll
        for (int n = 0; n < NBV; ++n) acc[n][i] *= corr;
      }
    }
    // weights into the wave's P tile [head][token]
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(sv[t][i] - mm[i]);
        ll[i] += e;
        pw[(4 * (lane >> 4) + i) * kPStride + 16 * t + (lane & 15)] = e;
      }
    }
    // LDS accesses of one wave complete in order; the asm keeps the compiler
    // from moving the reads below above the writes of other lanes
    __asm__ volatile("" ::: "memory");
    // A operand: head l % 16, tokens 8 (l / 16) .. + 7, as hi + lo bf16
    bf16x8 pa[2];
    {
      const float4 w0 = *reinterpret_cast<const float4*>(pw + (lane & 15) * kPStride + 8 * (lane >> 4));
      const float4 w1 = *reinterpret_cast<const float4*>(pw + (lane & 15) * kPStride + 8 * (lane >> 4) + 4);
      const float x[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      u32x4 hw, lw;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 h = cvt2(x[j], x[j + 1]);
        const bf16x2 l = cvt2(x[j] - (float)h[0], x[j + 1] - (float)h[1]);
        hw[j / 2] = __builtin_bit_cast(uint32_t, h);
        lw[j / 2] = __builtin_bit_cast(uint32_t, l);
      }
      pa[0] = __builtin_bit_cast(bf16x8, hw);
      pa[1] = __builtin_bit_cast(bf16x8, lw);
    }
    // values: acc[n] += P . L_V[:, 16 n .. 16 n + 15]
    const unsigned char* vt = lds.vt[buf];
#pragma unroll
    for (int n = 0; n < NBV; ++n) {
      const int row = 16 * n + (lane & 15);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(
          vt + row * kVtStride + ((32 * th + 8 * (lane >> 4)) ^ vt_swizzle(row)) * 2);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[0], __builtin_bit_cast(bf16x8, vb),
                                                       acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[1], __builtin_bit_cast(bf16x8, vb),
                                                       acc[n], 0, 0, 0);
    }
    stage_tile(tp, buf ^ 1);
    __syncthreads();
  };
  for (int cb = 0; cb < ntok; cb += 2 * kOnceStep) {
    step(cb, 0, ta, tb);
    step(cb + kOnceStep, 1, tb, ta);
  }

  // ---- merge the two token halves of each head block, write the records
  float l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = group_sum<16>(ll[i]);
  float* mrg = reinterpret_cast<float*>(lds.kt[0]);  // [hb][16 heads][R], then m, l
  float* mrg_m = mrg + NHB * 16 * R;
  float* mrg_l = mrg_m + NHB * 16;
  if (th == 1) {
#pragma unroll
    for (int n = 0; n < NBV; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mrg[(hb * 16 + 4 * (lane >> 4) + i) * R + 16 * n + (lane & 15)] = acc[n][i];
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mrg_m[hb * 16 + 4 * (lane >> 4) + i] = mm[i];
        mrg_l[hb * 16 + 4 * (lane >> 4) + i] = l[i];
      }
    }
  }
  __syncthreads();
  if (th == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hr = 4 * (lane >> 4) + i;  // head row in the block
      if (hr >= nvalid) continue;
      const float m1 = mrg_m[hb * 16 + hr], l1 = mrg_l[hb * 16 + hr];
      const float M = fmaxf(mm[i], m1);
      const float f0 = fast_exp2(mm[i] - M), f1 = fast_exp2(m1 - M);
      float* rec = a.ws + (((size_t)b * a.Hq + head0 + hr) * a.P + p) * (R + kRecPad);
#pragma unroll
      for (int n = 0; n < NBV; ++n) {
        const float o = mrg[(hb * 16 + hr) * R + 16 * n + (lane & 15)];
        rec[16 * n + (lane & 15)] = fmaf(acc[n][i], f0, o * f1);
      }
      if ((lane & 15) == 0) {
        rec[R] = M;
        rec[R + 1] = fmaf(l[i], f0, l1 * f1);
      }
    }
  }
}

}  // namespace

bool shared_once_supported(int latent_dtype, int rank, int heads_per_stream) {
  return latent_dtype == LRATTN_BF16 && (rank == 32 || rank == 64 || rank == 128) &&
         heads_per_stream >= 32;
}

int shared_once_blocks(int heads_per_stream) {
  const int nhb = (heads_per_stream + 15) / 16;
  return nhb < 2 ? 2 : nhb > 4 ? 4 : nhb;
}

template <int NHB>
hipError_t launch_once_nhb(int rank, const SharedOnceArgs& a, hipStream_t s) {
  const int groups = (a.Hq / a.S + 16 * NHB - 1) / (16 * NHB);
  const dim3 grid(a.P, a.S * groups, a.B), block(128 * NHB);
  switch (rank) {
    case 32: hipLaunchKernelGGL((shared_once_kernel<32, NHB>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((shared_once_kernel<64, NHB>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((shared_once_kernel<128, NHB>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_shared_once(int rank, const SharedOnceArgs& a, hipStream_t s) {
  switch (shared_once_blocks(a.Hq / a.S)) {
    case 2: return launch_once_nhb<2>(rank, a, s);
    case 3: return launch_once_nhb<3>(rank, a, s);
    case 4: return launch_once_nhb<4>(rank, a, s);
    default: return hipErrorInvalidValue;
  }
}

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
