// Shared latent streams read once for all heads (AttentionPack page, section
// 2.A): launch interface of the one-pass partition kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrattn {

struct SharedOnceArgs {
  const float* qt;          // [B, Hq, R] absorbed queries (base-2 logit scale)
  const void* LK;           // [B, S, T, R] bf16
  const void* LV;           // [B, S, T, R] bf16
  const int32_t* seq_lens;  // [B]
  float* ws;                // records [B, Hq, P, R + kRecPad]
  int32_t B, Hq, S, T;      // S latent streams, Hq / S heads per stream
  int32_t P, Stok;          // partitions, tokens per partition
};

// True when the one-pass kernel serves (latent dtype, rank, heads per stream).
bool shared_once_supported(int latent_dtype, int rank, int heads_per_stream);
// Head blocks of 16 per workgroup (2, 3 or 4): each workgroup serves up to
// 16 * that many heads of its stream.
int shared_once_blocks(int heads_per_stream);
// Grid (P, S * ceil(heads per stream / (16 blocks)), B), 128 * blocks threads.
hipError_t launch_shared_once(int rank, const SharedOnceArgs& a, hipStream_t s);

}  // namespace lrattn
