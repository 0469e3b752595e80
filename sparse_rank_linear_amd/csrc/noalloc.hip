// salr_linear_forward_noalloc (include/salr.h): the forward with its
// workspace in a fixed library-owned device array instead of a caller
// buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file's code object: each GPU the library runs on
// holds its own copy (SALR_NOALLOC_SCRATCH_BYTES) until the process ends.
// In host code its name stands for a host-side shadow, not a device
// address, so the device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever handed to a kernel or a
// memory call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "salr.h"
#include "salr_api_internal.hpp"

namespace {

constexpr size_t kScratchBytes = SALR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
constexpr size_t kErrWordOffset = 8;  // the workspace's wait-error word

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_setup_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's array (set up on its first call: address looked up,
// whole array zero-filled on `s` and waited for, so the counters start at
// zero and no tagged word carries a launch tag).  Set-up must not be
// captured into a graph; later calls may be.
int device_scratch(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SALR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SALR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_setup_mu);
  if (g_scratch[dev]) {
    *out = g_scratch[dev];
    return SALR_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return SALR_ERR_HIP;
  if (cap != hipStreamCaptureStatusNone) return SALR_ERR_UNSUPPORTED;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SALR_ERR_HIP;
  if (hipMemsetAsync(p, 0, kScratchBytes, s) != hipSuccess) return SALR_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SALR_ERR_HIP;
  g_scratch[dev] = p;
  *out = p;
  return SALR_OK;
}

}  // namespace

extern "C" int salr_linear_forward_noalloc(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y,
                                           uint32_t* wait_err, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Arguments first, with no workspace: every argument error is reported
  // before the device is touched (SALR_ERR_WORKSPACE here means "valid").
  const int pre = salr::forward_impl(L, X, M, Y, nullptr, 0, nullptr, s);
  if (pre != SALR_ERR_WORKSPACE) return pre;
  if (wait_err && (reinterpret_cast<uintptr_t>(wait_err) & 3u)) return SALR_ERR_INVALID_ARG;
  void* ws = nullptr;
  const int st = device_scratch(s, &ws);
  if (st != SALR_OK) return st;
  uint32_t* err = wait_err ? wait_err : reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kErrWordOffset);
  // (a layer and M whose workspace exceeds the array: SALR_ERR_WORKSPACE)
  return salr::forward_impl(L, X, M, Y, ws, kScratchBytes, err, s);
}
