// moe_forward for callers that cannot allocate device memory: its workspace is a
// fixed device array of the library, one per GPU, instead of a caller buffer.
#include <cstdio>
#include <mutex>

#include "kernels.h"
#include "moe.h"

namespace moe {
// sets the message moe_last_error() returns on this thread (moe_api.hip)
moe_status report_error(moe_status s, const char* msg);
}  // namespace moe

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

// The device array. In host code this name is a host-side stand-in, not a
// device address: only the address hipGetSymbolAddress returns for the current
// device is passed to kernels.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];   // scratch's address on each device, once looked up

// scratch's device address on the current device (looked up on the first call
// there, with that device current); nullptr with *err set on failure.
void* device_scratch(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_config* cfg, const void* x,
                                          const void* w_router, const float* sel_bias,
                                          const void* w1, const void* w3, const void* w2,
                                          const void* ws1, const void* ws3, const void* ws2,
                                          float* y, int32_t* idx_out, float* gates_out,
                                          const moe_stats* stats, void* stream) {
  size_t need = 0;
  moe_status st = moe_workspace_size(cfg, MOE_STAGE_FORWARD, &need);
  if (st != MOE_OK) return st;
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof(msg),
             "moe_forward_noalloc: the layer needs %zu bytes of scratch, above the fixed %zu",
             need, kScratchBytes);
    return moe::report_error(MOE_ERR_WORKSPACE, msg);
  }
  hipError_t e = hipSuccess;
  void* ws = device_scratch(&e);
  if (ws == nullptr) {
    char msg[160];
    snprintf(msg, sizeof(msg), "moe_forward_noalloc: scratch address: %s", hipGetErrorString(e));
    return moe::report_error(MOE_ERR_HIP, msg);
  }
  return moe_forward(cfg, x, w_router, sel_bias, w1, w3, w2, ws1, ws3, ws2, y, idx_out,
                     gates_out, stats, ws, kScratchBytes, stream);
}
