// Shader-clock probe: one lane reads the shader clock counter (s_memtime)
// and the 100 MHz real-time counter (s_memrealtime) around a short spin.
// Enqueued between other launches on a stream, it samples the clock those
// launches run at (the part lowers its clock under sustained matrix-core
// load).  It computes nothing of the attention method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrattn.h"
#include "lrattn_probe.h"

namespace {

constexpr uint64_t kSpinTicks = 500;       // 5 us of the 100 MHz real-time counter
constexpr int kSpinLimit = 1 << 20;        // iteration bound of the spin

__global__ void clock_probe_kernel(uint64_t* out) {
  if (threadIdx.x == 0) {
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r1 = r0;
    for (int it = 0; it < kSpinLimit && r1 - r0 < kSpinTicks; ++it)
      r1 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

extern "C" int lrattn_probe_clock(uint64_t* out, lrattn_stream stream) {
  if (!out) return LRATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 15u) != 0) return LRATTN_ERR_ALIGN;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), out);
  return hipGetLastError() == hipSuccess ? LRATTN_OK : LRATTN_ERR_HIP;
}
