// fb_step_noalloc: the always-recompute denoising step for callers that
// cannot allocate device memory.  Its split partials and per-head flags live
// in `scratch`, a file-scope device array of FB_NOALLOC_SCRATCH_BYTES that
// each GPU holds until the process ends; the caller passes the inputs and
// the outputs (A_out, L_out and the step's output).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device, with that device current, by
// hipGetSymbolAddress at the entry point's first call there, and only that
// address is passed on.  Every call on a GPU shares its array: calls that
// overlap on one GPU (other streams, other threads) race.  Nothing in the
// scratch has to start at zero (every value is written before it is read in
// the same call).
#include <hip/hip_runtime.h>

#include <mutex>

#include "fb.h"
#include "fb_internal.h"

namespace {

__device__ __align__(256) char scratch[FB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;   // device address of `scratch` on the device
  int n_cu = 0;
};
std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

}  // namespace

extern "C" fb_status fb_step_noalloc(const fb_config* cfg, const void* q_blk, const void* k_blk, const void* v_blk,
                                     const void* k_prefix, const void* v_prefix, int32_t prefix_len, float* a_out,
                                     float* l_out, void* out, void* stream) {
  if (!cfg) return fbk::report(FB_E_ARG, "config is null");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fbk::report(FB_E_HIP, "no usable HIP device");
  if (dev < 0 || dev >= kMaxDevices) return fbk::report(FB_E_UNSUPPORTED, "device index beyond 63");
  DeviceScratch ds;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_dev[dev].ptr == nullptr) {   // first call on this device (it is current)
      void* p = nullptr;
      hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return fbk::report(FB_E_HIP, "hipGetSymbolAddress of the scratch array failed");
      }
      int n_cu = 0;
      if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n_cu = 0;
      g_dev[dev].ptr = p;
      g_dev[dev].n_cu = n_cu;
    }
    ds = g_dev[dev];
  }
  return fbk::noalloc_step(cfg, ds.ptr, FB_NOALLOC_SCRATCH_BYTES, ds.n_cu, q_blk, k_blk, v_blk, k_prefix, v_prefix,
                           prefix_len, a_out, l_out, out, stream);
}
