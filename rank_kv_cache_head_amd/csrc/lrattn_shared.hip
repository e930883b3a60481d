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
// The decode step of a grouped cache takes the same kernel when its plan has
// many partitions per head: head h then uses its kv-head's factor B_K[h / G]
// (hpf = G), and q~ is formed once per head instead of once per partition.
//
// Grid (Hq, B): one workgroup per (head, sequence).  The head's factor block
// B_K[h] (r x d) is read as consecutive 16-byte pieces, piece t + 256 k by
// thread t, so every load instruction of a wave covers 1 KB of consecutive
// bytes; a factor row is d / (elements per piece) consecutive pieces, held by
// as many consecutive lanes of one wave, and each lane's columns are the same
// for all its pieces.  A lane forms the products of its piece with the query
// elements of those columns (exact in fp32, summed in increasing column
// order), and the row's lanes add their partial sums in a fixed butterfly.
#include <float.h>

#include "lrattn.h"
#include "lrattn_device.hpp"
#include "lrattn_internal.hpp"
#include "lrattn_shared.hpp"

namespace lrattn {
namespace {

constexpr int kAbsorbPieces = 8;  // 16-byte factor pieces per thread and round

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

// q~[b][h][j] = qscale * sum_i q[b][h][i] * B_K[h / hpf][j][i].  Every load is
// issued before anything waits: the first round of factor pieces, then the
// query row (one 16-byte piece for each of the first d * size / 16 threads).
// Pieces past the block read zeros (buffer bounds) and are not stored.
template <int R, int FT>
__device__ __forceinline__ void absorb_body(const AbsorbHeadsArgs& a) {
  constexpr int ES = FT == LRATTN_F32 ? 4 : 2;
  constexpr int EPP = 16 / ES;                   // factor elements per piece
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, d = a.d;
  const int ppr = d / EPP;                       // pieces per factor row: 8 .. 64
  const int npieces = R * ppr;
  const int c0 = (tid % ppr) * EPP;              // this thread's columns, every round
  const auto rb = make_rsrc(static_cast<const char*>(a.BK) + (size_t)(h / a.hpf) * R * d * ES,
                            (uint32_t)(R * d * ES));
  u32x4 w[kAbsorbPieces];
  auto load_round = [&](int r0) {
#pragma unroll
    for (int k = 0; k < kAbsorbPieces; ++k)
      w[k] = __builtin_amdgcn_raw_buffer_load_b128(
          rb, (int)((uint32_t)(r0 + k * kThreads + tid) * 16u), 0, 0);
  };
  load_round(0);

  __shared__ float qs[kMaxHeadDim];
  {
    const int qes = a.q_dtype == LRATTN_F32 ? 4 : 2;
    const int qpr = d * qes / 16;  // pieces of the query row
    const auto rq = make_rsrc(static_cast<const char*>(a.q) + ((size_t)b * a.Hq + h) * d * qes,
                              (uint32_t)(d * qes));
    const u32x4 qw = __builtin_amdgcn_raw_buffer_load_b128(
        rq, (int)(tid < qpr ? (uint32_t)tid * 16u : kOffNone), 0, 0);
    if (tid < qpr) {
      if (a.q_dtype == LRATTN_F32) stage_q_piece<LRATTN_F32>(qw, &qs[4 * tid]);
      else if (a.q_dtype == LRATTN_BF16) stage_q_piece<LRATTN_BF16>(qw, &qs[8 * tid]);
      else stage_q_piece<LRATTN_F16>(qw, &qs[8 * tid]);
    }
  }
  __syncthreads();
  float qv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) qv[e] = qs[c0 + e];

  float* qt = a.qt + ((size_t)b * a.Hq + h) * R;
  for (int r0 = 0; r0 < npieces; r0 += kAbsorbPieces * kThreads) {
    if (r0 > 0) {
      load_round(r0);
      __builtin_amdgcn_sched_barrier(0);  // the round's loads ahead of its arithmetic
    }
#pragma unroll
    for (int k = 0; k < kAbsorbPieces; ++k) {
      const int pc = r0 + k * kThreads + tid;  // the same for the lanes of a row
      if (r0 + k * kThreads < npieces) {     // the same in every thread (all lanes shuffle)
        float f[EPP];
        unpack_piece<FT>(w[k], f);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc = fmaf(qv[e], f[e], acc);
        for (int off = 1; off < ppr; off <<= 1) acc += __shfl_xor(acc, off);
        if (tid % ppr == 0 && pc < npieces) qt[pc / ppr] = acc * a.qscale;
      }
    }
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
  hipLaunchKernelGGL((absorb_heads_kernel<R>), dim3(a.Hq, a.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------- one pass over a shared stream
// AttentionPack page, section 2.A: all heads read the same compressed rows.
// Reading them once per head group multiplies the stream's traffic, and the
// value sums of many heads (heads x r accumulators) are more than the VALU
// can keep up with.  This kernel reads each tile once for up to 64 heads
// (NHB blocks of 16) and runs both products on the matrix cores, with the
// token axis of each 16-token tile along the rows of the scores:
//
//   scores  S^T (16 tokens x 16 heads) = L_K . q~^T with
//           v_mfma_f32_16x16x32_bf16: the A operand is the K tile's rows as
//           stored, the B operand q~ split exactly into three bf16 terms
//           (the latents are bf16, so every product is exact and the sums
//           are fp32).  Lane l receives tokens 4 (l / 16) + i (i < 4) of head
//           l % 16, so every lane keeps the softmax state of one head.
//   values  acc^T (16 coordinates x 16 heads) += L_V^T (16 coordinates x 32
//           tokens) . P^T (32 tokens x 16 heads), the weights P split into two
//           bf16 terms (relative error below 2^-16).  The weights are the
//           B operand in the registers the scores left them in (k slots
//           0-3: the first tile's tokens 4 (l / 16) + i, slots 4-7: the
//           second tile's), and the A operand takes the same tokens of L_V
//           from the LDS tile, stored as it arrives ([token][coordinate]),
//           with the transposing LDS read ds_read_b64_tr_b16: in each 16-lane
//           row, result slot k of lane i is element i % 4 of the 8-byte read
//           of lane 4 k + i / 4, so lane j reads row j / 4 at columns
//           4 (j % 4) .. + 3 of its 4 x 16 block and every lane receives one
//           coordinate of 4 consecutive tokens.
//
// Workgroup: one (sequence, stream, group of up to 16 NHB heads, partition),
// 2 NHB waves; wave w takes head block w % NHB (16 heads) and token half
// w / NHB of every 64-token step; the two halves are merged at the end
// (fixed order).  Waves 0-3 stage the tiles.

namespace {

constexpr int kOnceStep = 64;            // tokens per step (32 per wave)

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Four consecutive tokens of one coordinate from a [token][coordinate] LDS
// tile (see above for the lane pattern of the transposing read).
__device__ __forceinline__ s16x4 read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(p)));
}

template <int R, int NHB>
struct OnceLds {
  static constexpr int kStride = 2 * R + 16;  // bytes per latent row: r bf16 + pad
  alignas(16) unsigned char kt[2][kOnceStep * kStride];  // L_K tiles [token][coordinate]
  alignas(16) unsigned char vt[2][kOnceStep * kStride];  // L_V tiles [token][coordinate]
  // the final merge reuses both K buffers: [head block][16 heads][R], m, l
  static_assert(NHB * 16 * (R + 2) * 4 <= 2 * kOnceStep * kStride, "merge area");
};

// Two waves per SIMD: at R = 128 the registers fit 256 without spills, and
// with NHB = 2 two workgroups' LDS fit a CU, so a CU can run a second
// workgroup while the first waits on memory.
template <int R, int NHB>
__global__ __launch_bounds__(128 * NHB) __attribute__((amdgpu_waves_per_eu(2)))
void shared_once_kernel(SharedOnceArgs a) {
  constexpr int KC = R / 32;          // 32-wide steps of r (scores)
  constexpr int NBV = R / 16;         // 16-wide blocks of r (values)
  constexpr int RowB = 2 * R;         // bytes per latent row
  constexpr int KS = OnceLds<R, NHB>::kStride;
  constexpr int KV = kOnceStep * RowB / 16 / 256;  // 16-byte pieces per thread, tile and K|V
  const int p = blockIdx.x, b = blockIdx.z;
  constexpr int GH = 16 * NHB;        // heads per group
  const int nh = a.Hq / a.S, hgs = (nh + GH - 1) / GH;  // the last group may be partial
  const int s = blockIdx.y / hgs, hg = blockIdx.y % hgs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = wave % NHB, th = wave / NHB;
  const int grp = lane >> 4, col = lane & 15;  // lane row (token quad) and head / coordinate
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
  // instruction streamed 14% slower).  Both tiles go to LDS as they are,
  // rows padded by 16 bytes (the score operand reads of 16 rows at one
  // column and the transposing reads of 16 rows spread over the banks).
  // Waves past the fourth load nothing (an offset past the buffer: zeros,
  // no memory access) and write nothing.
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
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int pc = 256 * k + (tid & 255), tk = pc / CPR, cg = pc % CPR;
      *reinterpret_cast<u32x4*>(lds.kt[buf] + tk * KS + cg * 16) = tl.k[k];
      *reinterpret_cast<u32x4*>(lds.vt[buf] + tk * KS + cg * 16) = tl.v[k];
    }
  };

  // ---- prologue: q~ of the wave's 16 heads (B operands), the first tiles
  Tile ta, tb;
  bf16x8 qb[3][KC];
  {
    const auto rq = make_rsrc(a.qt + ((size_t)b * a.Hq + head0) * R, (uint32_t)nvalid * R * 4u);
    u32x4 qw[KC][2];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        qw[c][h] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (int)((col * R + 32 * c + 8 * grp + 4 * h) * 4u), 0, 0);
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
      for (int term = 0; term < 3; ++term) qb[term][c] = t3[term];
    }
    stage_tile(ta, 0);
  }
  __syncthreads();

  // acc[n][i]: coordinate 16 n + 4 grp + i of head col; mm, ll: head col's
  // reference max and (this lane's part of) its sum
  f32x4 acc[NBV];
#pragma unroll
  for (int n = 0; n < NBV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mm = -FLT_MAX, ll = 0.f;
  // this lane's transposing-read address in a V tile, for the first tile's
  // token quad: row 32 th + 4 grp + col / 4, columns 4 (col % 4) .. + 3
  const int vaddr = (32 * th + 4 * grp + (col >> 2)) * KS + 8 * (col & 3);
  // One 64-token step at cb from LDS buffer buf: the tile two steps ahead is
  // requested into tn, the next step's (requested a step earlier, in tp) is
  // staged into the other buffer at the end, so every latent load has a
  // whole step of work to arrive and no operand waits on memory.  The loop
  // runs whole pairs of steps; a step past the partition sees zeros and
  // masked scores and adds nothing.
  auto step = [&](int cb, int buf, Tile& tn, const Tile& tp) {
    load_tile(tn, cb + 2 * kOnceStep);
    // scores of the wave's two 16-token tiles (A operand: token l % 16,
    // columns 32 c + 8 (l / 16) .. + 7, from the K tile)
    const unsigned char* kt = lds.kt[buf];
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(
            kt + (32 * th + 16 * t + col) * KS + 64 * c + 16 * grp);
#pragma unroll
        for (int term = 0; term < 3; ++term)
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, ka), qb[term][c], sc[t], 0, 0, 0);
      }
    }
    // mask, then the lazily moved reference of head col (lanes col + 16 q)
    float sv[2][4];
    bool need = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool masked = cb + 32 * th + 16 * t + 4 * grp + i >= ntok;
        sv[t][i] = masked ? -INFINITY : sc[t][i];
        need |= sv[t][i] > mm + kLazyLog2;
      }
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      float x = sv[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, sv[t][i]);
      }
      x = max_quarters(x);
      const float nm = x > mm + kLazyLog2 ? x : mm;
      const float corr = fast_exp2(mm - nm);
      mm = nm;
      ll *= corr;
#pragma unroll
      for (int n = 0; n < NBV; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] *= corr;
      }
    }
    // weights as the B operand (k slot 4 t + i: token 16 t + 4 grp + i of
    // the wave's half), hi + lo bf16
    bf16x8 pb[2];
    {
      u32x4 hw, lw;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float e0 = fast_exp2(sv[t][i] - mm), e1 = fast_exp2(sv[t][i + 1] - mm);
          ll += e0;
          ll += e1;
          const bf16x2 h = cvt2(e0, e1);
          const bf16x2 l = cvt2(e0 - (float)h[0], e1 - (float)h[1]);
          hw[2 * t + i / 2] = __builtin_bit_cast(uint32_t, h);
          lw[2 * t + i / 2] = __builtin_bit_cast(uint32_t, l);
        }
      }
      pb[0] = __builtin_bit_cast(bf16x8, hw);
      pb[1] = __builtin_bit_cast(bf16x8, lw);
    }
    // values: acc[n] += L_V[tokens, 16 n .. 16 n + 15]^T . P^T
    const unsigned char* vt = lds.vt[buf] + vaddr;
#pragma unroll
    for (int n = 0; n < NBV; ++n) {
      const s16x4 v0 = read_tr(vt + 32 * n);
      const s16x4 v1 = read_tr(vt + 16 * KS + 32 * n);
      const s16x4 v8[2] = {v0, v1};
      const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0], acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1], acc[n], 0, 0, 0);
    }
    stage_tile(tp, buf ^ 1);
    __syncthreads();
  };
  for (int cb = 0; cb < ntok; cb += 2 * kOnceStep) {
    step(cb, 0, ta, tb);
    step(cb + kOnceStep, 1, tb, ta);
  }

  // ---- merge the two token halves of each head block, write the records
  const float lsum = sum_quarters(ll);
  float* mrg = reinterpret_cast<float*>(lds.kt[0]);  // [hb][16 heads][R], then m, l
  float* mrg_m = mrg + NHB * 16 * R;
  float* mrg_l = mrg_m + NHB * 16;
  if (th == 1) {
#pragma unroll
    for (int n = 0; n < NBV; ++n)
      *reinterpret_cast<f32x4*>(&mrg[(hb * 16 + col) * R + 16 * n + 4 * grp]) = acc[n];
    if (grp == 0) {
      mrg_m[hb * 16 + col] = mm;
      mrg_l[hb * 16 + col] = lsum;
    }
  }
  __syncthreads();
  if (th == 0 && col < nvalid) {
    const float m1 = mrg_m[hb * 16 + col], l1 = mrg_l[hb * 16 + col];
    const float M = fmaxf(mm, m1);
    const float f0 = fast_exp2(mm - M), f1 = fast_exp2(m1 - M);
    float* rec = a.ws + (((size_t)b * a.Hq + head0 + col) * a.P + p) * (R + kRecPad);
#pragma unroll
    for (int n = 0; n < NBV; ++n) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(&mrg[(hb * 16 + col) * R + 16 * n + 4 * grp]);
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = fmaf(acc[n][i], f0, o[i] * f1);
      *reinterpret_cast<f32x4*>(&rec[16 * n + 4 * grp]) = r;
    }
    if (grp == 0) {
      rec[R] = M;
      rec[R + 1] = fmaf(lsum, f0, l1 * f1);
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
