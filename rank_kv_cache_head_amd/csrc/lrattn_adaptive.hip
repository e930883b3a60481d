// Attention-aware rank: the importance update that follows the decode step.
//
// AttentionPack page, section 2.B: a moving average of each token's
// accumulated attention marks the tokens that are rebuilt at full rank.
// After the partitions (which wrote every valid token's base-2 logit per
// query head, [B, Hkv, T, G]) and the combine (which wrote each row's final reference m and
// denominator L), this kernel forms the step's attention weight of token t
// averaged over the query heads of kv-head g,
//   a_t = (1/G) sum_{h in g} 2^(logit[b, h, t] - m[b, h]) / L[b, h],
// and updates imp[b, g, t] = decay * imp[b, g, t] + (1 - decay) * a_t for
// t < seq_len; the other entries are not touched.  The heads are added in
// ascending order (bitwise reproducible).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lrattn_internal.hpp"

namespace lrattn {
namespace {

constexpr int kImpThreads = 256;

// The partitions leave the logits token-major per kv-head, [B, Hkv, T, G]
// with G = Hq / Hkv, so a token's G logits are contiguous.  TPT consecutive
// tokens per thread: 4 (16-byte loads of logits and scores) when T is a
// multiple of 4, so every row starts on a 16-byte boundary, else 1.  Every
// load is issued before the first is used.
template <int G, int TPT>
__global__ __launch_bounds__(kImpThreads) void importance_kernel(ImportanceArgs a) {
  using Vec = typename std::conditional<TPT == 4, float4, float>::type;
  constexpr int NL = TPT * G / (TPT == 4 ? 4 : 1);  // loads of logits per thread
  const int g = blockIdx.y, b = blockIdx.z;
  const int t = (blockIdx.x * kImpThreads + threadIdx.x) * TPT;
  const int len = min(max(a.seq_lens[b], 0), a.T);
  if (t >= len) return;
  const size_t grp = (size_t)b * a.Hkv + g;
  const Vec* src = reinterpret_cast<const Vec*>(a.logits + (grp * a.T + t) * G);
  Vec lg[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) lg[k] = src[k];
  float* imp = a.imp + grp * a.T + t;
  Vec cur = *reinterpret_cast<const Vec*>(imp);
  const float* x = reinterpret_cast<const float*>(lg);  // [token][head]
  float* c = reinterpret_cast<float*>(&cur);
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * G;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    float w = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float m = a.stats[(row0 + i) * 2], L = a.stats[(row0 + i) * 2 + 1];
      w += exp2f(x[k * G + i] - m) / L;
    }
    c[k] = a.decay * c[k] + (1.f - a.decay) * (w / (float)G);
  }
  if (t + TPT <= len) {
    *reinterpret_cast<Vec*>(imp) = cur;
  } else {
#pragma unroll
    for (int k = 0; k < TPT; ++k)
      if (t + k < len) imp[k] = c[k];
  }
}

template <int G>
hipError_t launch_g(const ImportanceArgs& a, hipStream_t s) {
  const dim3 block(kImpThreads);
  if (a.T % 4 == 0) {
    const dim3 grid((a.T / 4 + kImpThreads - 1) / kImpThreads, a.Hkv, a.B);
    hipLaunchKernelGGL((importance_kernel<G, 4>), grid, block, 0, s, a);
  } else {
    const dim3 grid((a.T + kImpThreads - 1) / kImpThreads, a.Hkv, a.B);
    hipLaunchKernelGGL((importance_kernel<G, 1>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_importance(const ImportanceArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 8: return launch_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrattn
