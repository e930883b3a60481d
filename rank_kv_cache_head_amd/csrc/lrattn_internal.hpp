// Internal interface between the C-ABI host layer (lrattn_api.hip) and the
// gfx950 kernels (lrattn_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrattn.h"

namespace lrattn {

constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kRecPad = 4;      // partial record: r accumulators, max, sum, 2 pad
constexpr int kMaxHeadDim = 256;
constexpr int kMaxRank = 128;
constexpr int kMaxGroup = 8;

// One partial record per (b, query head, partition):
//   rec[0..r)  sum_t 2^(s_t - m) * Lv[t]   (latent-space value accumulator)
//   rec[r]     m   reference max of the base-2 logits s_t
//   rec[r+1]   l   sum_t 2^(s_t - m)
// Base-2 logits: s_t = log2(e) * softmax_scale * <q, K[t]>, so 2^(s - m)
// equals e^(logit - reference logit).
inline int record_floats(int rank) { return rank + kRecPad; }

// Workspace: the partial records [B, Hq, P, r + kRecPad] fp32.
inline size_t records_bytes(int B, int Hq, int P, int rank) {
  const size_t b = (size_t)B * Hq * (size_t)P * (size_t)record_floats(rank) * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

// Where the merged rows go.
struct MergeArgs {
  const void* BV;          // [Hkv, r, d]
  void* out;               // [B, Hq, d]
  int32_t f_dtype, out_dtype;
};

struct PartitionArgs {
  const void* q;           // [B, Hq, d]
  const void* LK;          // [B, Hkv, T, r]
  const void* LV;          // [B, Hkv, T, r]
  const void* BK;          // [Hkv, r, d]
  const float* scales;     // [2, B, Hkv, T] or nullptr
  const int32_t* seq_lens; // [B]
  const float* rope;       // [T, d] cos | sin per position (rebuilt-key kernel), or nullptr
  const float* qt_pre;     // [B, Hq, r] q~ already absorbed (per-head factors), or nullptr
  float* ws;               // [B, Hq, P, r + kRecPad]
  int32_t B, Hq, Hkv, d, T;
  int32_t HG;              // head groups (grid y): query heads hg * G .. + G - 1
  int32_t hps;             // query heads per latent stream: group hg reads stream hg * G / hps
  int32_t P, S;            // partitions, tokens per partition
  int32_t xcd_group;       // 1: one-dimensional grid, head groups of a tile on one XCD
  int32_t q_dtype, f_dtype;
  float qscale;            // softmax_scale * log2(e)
  // token window and record slots of this launch: partition p covers tokens
  // [t_lo + p S, t_lo + (p + 1) S) clipped to min(seq_len, t_hi) and writes
  // record slot p_off + p of P_rec per head (defaults 0, T, 0, P)
  int32_t t_lo, t_hi, p_off, P_rec;
  // two factor sets (BK1 non-null): partitions [0, P_img) take the image
  // tokens [0, n_img) in parts of S_img with BK, the others the text from
  // n_img in parts of S with BK1 (record slots unchanged)
  const void* BK1;
  int32_t n_img, P_img, S_img;
  // attention-aware rank (adaptive kernels only): token t of (b, g) keeps
  // latent coordinates [0, low_rank) when imp[b, g, t] < imp_thr, all r
  // otherwise; base-2 logits go to logits [B, Hq, T]
  const float* imp;
  float* logits;
  float imp_thr;
  int32_t low_rank;
};

struct CombineArgs {
  const int32_t* seq_lens; // [B]
  const float* ws;         // [B, Hq, P, r + kRecPad]
  MergeArgs merge;
  int32_t B, Hq, Hkv, d, r, T;
  int32_t P, S;
  int32_t factor_per_head;  // B_V indexed by query head (shared latent streams)
  // two factor sets (image block, then text): merge.BV is the image set and
  // BV1 the text set; records [0, P_img) cover tokens [0, n_img) in parts of
  // S_img, records [P_img, P) the rest in parts of S (BV1 null: one set)
  const void* BV1;
  int32_t n_img, P_img, S_img;
  float* stats;             // [B, Hq, 2]: final (max, denominator) per row, or nullptr
};

// Attention-aware rank: the importance update after the step (one thread
// per token; grid ceil(T / 256) x Hkv x B).
struct ImportanceArgs {
  const float* logits;      // [B, Hkv, T, G] base-2 logits of the step (G = Hq / Hkv)
  const float* stats;       // [B, Hq, 2] final (max, denominator) per row
  float* imp;               // [B, Hkv, T] updated in place for t < seq_len
  const int32_t* seq_lens;  // [B]
  int32_t B, Hq, Hkv, T;
  float decay;
};
hipError_t launch_importance(const ImportanceArgs& a, hipStream_t s);

// Attention-aware rank: true when the adaptive partition kernel is compiled
// for (latent dtype, rank, group); launch_adaptive launches it (grid P, HG, B).
bool adaptive_supported(int latent_dtype, int rank, int group);
hipError_t launch_adaptive(int latent_dtype, int rank, int group, const PartitionArgs& a,
                           hipStream_t s);
// True when the combine has a two-factor-set (image, text) form for (d, r).
bool modal_supported(int head_dim, int rank);
// True when a partition kernel is compiled for (latent dtype, rank, group).
bool partition_supported(int latent_dtype, int rank, int group);
// Name of the partition kernel launch_partition uses for these arguments
// (static text; "" when unsupported).
const char* partition_kernel_name(int latent_dtype, int rank, int group);
// The adaptive-rank partition kernel's name ("" when unsupported).
const char* adaptive_kernel_name(int latent_dtype, int rank, int group);
// Launch the partition grid (P, Hkv, B) on `s`.  Returns the launch error.
hipError_t launch_partition(int latent_dtype, int rank, int group,
                            const PartitionArgs& a, hipStream_t s);
// Launch the combine grid (Hq, B) on `s`.
hipError_t launch_combine(int group, const CombineArgs& a, hipStream_t s);
// The rebuilt-key partition kernel (bf16 q, latents and factors; d in
// {64, 128}, r in {32, 64}, group in {1, 2, 4, 8}); a.rope selects the
// rotating instantiation.  Same grid and records as launch_partition.
bool rebuild_supported(int head_dim, int rank, int group);

// q~ per query head with its own factor (shared latent streams):
// qt[b][h][j] = qscale * sum_i q[b][h][i] * B_K[h][j][i], fp32.
struct AbsorbHeadsArgs {
  const void* q;    // [B, Hq, d]
  const void* BK;   // [Hq / hpf, r, d]
  float* qt;        // [B, Hq, r]
  int32_t B, Hq, d, r;
  int32_t hpf;      // query heads per factor block: head h uses B_K[h / hpf]
  int32_t q_dtype, f_dtype;
  float qscale;
};
hipError_t launch_absorb_heads(const AbsorbHeadsArgs& a, hipStream_t s);
hipError_t launch_rebuild(int head_dim, int rank, int group, const PartitionArgs& a,
                          hipStream_t s);

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
constexpr int kProbeBlocks = 8192;

}  // namespace lrattn
