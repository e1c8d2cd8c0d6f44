// gdla_decode_noalloc: the decode step of gdla_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// Its workspace is `scratch`, a static device array of this translation unit: each GPU holds its
// own copy, from the first call on that GPU (when its code object is loaded) until the process
// ends.  Host code never uses the array's name as an address: its per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// handed to the kernels.  Every call on one GPU shares that GPU's array and leaves its contents
// behind; the decode kernels write every workspace byte they read, so nothing needs clearing.
#include "gdla_internal.h"

#include <mutex>
#include <stdio.h>

#define GDLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = (size_t)GDLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (its address taken once per device), or null with
// *err set.
void *scratch_ptr(hipError_t *err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

GDLA_EXPORT gdla_status gdla_decode_noalloc(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                            int32_t B, const int32_t *pos_host, void *cache, int32_t max_len,
                                            void *out, const gdla_debug *dbg, hipStream_t stream) {
  // Invalid arguments, and a size the scratch cannot hold, are refused before any HIP call.
  const gdla_status st = gdla::check_decode_args(dims, w, x, B, pos_host, cache, max_len, out);
  if (st != GDLA_OK || B == 0) return st;
  const size_t need = gdla_workspace_bytes(dims, GDLA_OP_DECODE, B, 1, pos_host, max_len);
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "gdla_decode_noalloc: this call needs %zu bytes of workspace, above the library's static "
             "scratch of %zu bytes (GDLA_NOALLOC_SCRATCH_BYTES)", need, kScratchBytes);
    return gdla::report_error(GDLA_ERR_WORKSPACE, msg);
  }
  hipError_t e = hipSuccess;
  void *ws = scratch_ptr(&e);
  if (!ws) {
    char msg[200];
    snprintf(msg, sizeof(msg), "gdla_decode_noalloc: no address for the static scratch on this device: %s",
             hipGetErrorString(e));
    return gdla::report_error(GDLA_ERR_HIP, msg);
  }
  return gdla_decode(dims, w, x, B, pos_host, cache, max_len, out, ws, kScratchBytes, dbg, stream);
}
