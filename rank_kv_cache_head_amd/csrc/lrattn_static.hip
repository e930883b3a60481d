// lrattn_decode_static: the decode step with its workspace (the partial
// records, and the absorbed queries when the plan has them) in a static
// device buffer instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels are lrattn_decode's; only
// the place of the workspace differs.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "lrattn.h"

namespace {

// The workspace of every lrattn_decode_static call on a device.  Each device
// holds its own copy (at its own address) from the first call on it until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device address: the address comes from hipGetSymbolAddress, resolved
// once per device below, and only that address is passed to the kernels.
__device__ __align__(256) unsigned char scratch[LRATTN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_resolve;

// Device address of the current device's `scratch`.
int scratch_of_current_device(int dev, void** ptr) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_resolve);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return LRATTN_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return LRATTN_OK;
}

}  // namespace

extern "C" int lrattn_decode_static(const lrattn_params* p, const void* q, const void* L_K,
                                    const void* L_V, const void* B_K, const void* B_V,
                                    const float* scales, const int32_t* seq_lens, void* out,
                                    lrattn_stream stream) {
  size_t need = 0;
  int st = lrattn_workspace_size(p, &need);  // the parameter block, host only
  if (st != LRATTN_OK) return st;
  if (need > LRATTN_STATIC_SCRATCH_BYTES) return LRATTN_ERR_SCRATCH;
  // Every other argument, still on the host: lrattn_decode checks the
  // workspace last, so without one it returns LRATTN_ERR_WORKSPACE exactly
  // when everything else is valid, and launches nothing either way.
  st = lrattn_decode(p, q, L_K, L_V, B_K, B_V, scales, seq_lens, out, nullptr, 0, stream);
  if (st != LRATTN_ERR_WORKSPACE) return st;

  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices ||
      hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
    (void)hipGetLastError();
    return LRATTN_ERR_HIP;
  }
  if (sdev != dev) return LRATTN_ERR_UNSUPPORTED;  // the buffer used is the current device's
  void* ws = nullptr;
  st = scratch_of_current_device(dev, &ws);
  if (st != LRATTN_OK) return st;
  return lrattn_decode(p, q, L_K, L_V, B_K, B_V, scales, seq_lens, out, ws,
                       (size_t)LRATTN_STATIC_SCRATCH_BYTES, stream);
}
