// moe_layer_forward_noalloc: the layer forward with the library's own device
// scratch array in place of a caller workspace, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops).
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy (loaded with this file's code object) until the process
// ends. Host code never passes the array's name to a kernel (on the host it is
// only a stand-in symbol): the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress, with that device current, and kept.
#include <stdio.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "moe.h"
#include "api_internal.h"

// The scratch array (device side). Its name is never used as an address in
// host code; see scratch_for_current_device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up on first use).
moe_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::api_error(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return moe::api_error(MOE_ERR_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return moe::api_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* d, const moe_layer_weights_t* w,
                                                  const void* x, void* y, hipStream_t stream) {
  size_t need = 0;
  MOE_RETURN_IF_ERROR(moe_workspace_size(d, &need));
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof(msg), "layer needs %zu bytes of scratch, the no-allocation entry point has %zu", need,
             kScratchBytes);
    return moe::api_error(MOE_ERR_WORKSPACE_TOO_SMALL, msg);
  }
  if (d->num_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  MOE_RETURN_IF_ERROR(scratch_for_current_device(&ws));
  // Every kernel of the forward writes what it later reads in the workspace, so
  // nothing in the scratch array has to start at zero.
  return moe_layer_forward_ex(d, w, x, y, ws, kScratchBytes, stream, nullptr);
}
