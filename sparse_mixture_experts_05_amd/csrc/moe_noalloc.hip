// moe_forward_noalloc: the whole layer without a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The workspace moe_forward needs lives in a file-scope device array of a
// fixed size. Each GPU holds its own copy from the time the library's code is
// loaded on it until the process ends. On a device's first call, the array's
// device address is looked up once (the array's name in host code is only a
// host-side stand-in) and kept per device; every later call passes that
// address on as moe_forward's workspace. Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.h"
#include "moe.h"

namespace {

constexpr size_t kScratchBytes = size_t(320) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up on the
// device's first call), or a failure status.
moe_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::set_error(MOE_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return moe::set_error(MOE_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return moe::set_error(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_forward_noalloc(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                               const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* topk_idx_opt,
                               float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt, float* importance_opt,
                               float* P_opt, float* balance_opt, float* smooth_load_opt, hipStream_t stream) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  const size_t need = moe_workspace_bytes(c);
  if (need > kScratchBytes)
    return moe::set_error(MOE_ERR_WORKSPACE,
                          "this layer needs %zu bytes of workspace; the allocation-free entry point holds at most "
                          "%zu (use moe_forward with a caller workspace)",
                          need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(c, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, topk_idx_opt, topk_w_opt, kept_opt, load_opt,
                     importance_opt, P_opt, balance_opt, smooth_load_opt, ws, kScratchBytes, stream);
}

}  // extern "C"
