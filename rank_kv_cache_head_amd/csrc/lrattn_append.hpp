// Internal interface of the append-step kernel (lrattn_append.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrattn {

struct AppendArgs {
  const void* x;            // [B, D]            x_dtype
  const void* AK;           // [Hkv, r, D]       x_dtype
  const void* AV;           // [Hkv, r, D]       x_dtype
  const int32_t* positions; // [B]
  void* LK;                 // [B, Hkv, T, r]    latent_dtype
  void* LV;                 // [B, Hkv, T, r]    latent_dtype
  float* scales;            // [2, B, Hkv, T] (int8 latents) or nullptr
  float* ws;                // partial rows [Hkv, 2, KS, B, r] fp32
  int32_t B, Hkv, D, r, T;
  int32_t KS;               // chunks of D (one workgroup each)
  int32_t x_dtype, latent_dtype;
};

// Largest batch one launch takes (four 16-row blocks of the matrix cores).
constexpr int kAppendMaxBatch = 64;

bool append_supported(int rank, int batch, int model_dim);
// True when the one-launch path serves (latent dtype, Hkv, r).
bool append_direct(int latent_dtype, int hkv, int r);
// Chunks of D for (Hkv, D): enough workgroups to cover the chip, chunks of at
// least 128 elements that divide D.
int append_chunks(int num_kv_heads, int model_dim);
size_t append_workspace_bytes(int num_kv_heads, int batch, int rank, int chunks);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

}  // namespace lrattn
