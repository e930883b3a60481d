// Attention-aware rank: the importance update that follows the decode step.
//
// AttentionPack page, section 2.B: a moving average of each token's
// accumulated attention marks the tokens that are rebuilt at full rank.
// After the partitions (which wrote every valid token's base-2 logit per
// query head) and the combine (which wrote each row's final reference m and
// denominator L), this kernel forms the step's attention weight of token t
// averaged over the query heads of kv-head g,
//   a_t = (1/G) sum_{h in g} 2^(logit[b, h, t] - m[b, h]) / L[b, h],
// and updates imp[b, g, t] = decay * imp[b, g, t] + (1 - decay) * a_t for
// t < seq_len; the other entries are not touched.  One thread per token;
// the heads are added in ascending order (bitwise reproducible).
#include <hip/hip_runtime.h>

#include "lrattn_internal.hpp"

namespace lrattn {
namespace {

constexpr int kImpThreads = 256;

__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImportanceArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * kImpThreads + threadIdx.x;
  const int len = min(max(a.seq_lens[b], 0), a.T);
  if (t >= len) return;
  const int G = a.Hq / a.Hkv;
  float w = 0.f;
  for (int i = 0; i < G; ++i) {
    const size_t row = (size_t)b * a.Hq + (size_t)g * G + i;
    const float m = a.stats[row * 2], L = a.stats[row * 2 + 1];
    w += exp2f(a.logits[row * a.T + t] - m) / L;
  }
  float* imp = a.imp + ((size_t)b * a.Hkv + g) * a.T + t;
  *imp = a.decay * *imp + (1.f - a.decay) * (w / (float)G);
}

}  // namespace

hipError_t launch_importance(const ImportanceArgs& a, hipStream_t s) {
  const dim3 grid((a.T + kImpThreads - 1) / kImpThreads, a.Hkv, a.B), block(kImpThreads);
  hipLaunchKernelGGL(importance_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lrattn
