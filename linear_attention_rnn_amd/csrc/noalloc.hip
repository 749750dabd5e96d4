// Scratch memory of the allocation-free forward (wkv7_forward_noalloc): a
// file-scope device array that every GPU the library runs on holds for the
// life of the process, so the call needs no allocation of its own.
//
// In host code the array's name is only a host-side stand-in; its device
// address on each GPU comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is handed to
// kernels or copies.

#include "host.h"

#include <hip/hip_runtime.h>

#include <mutex>

static __device__ __align__(256) unsigned char scratch[wkv7::kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace wkv7 {

wkv7_status static_scratch_setup(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return host_fail(WKV7_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return host_fail(WKV7_ERR_UNSUPPORTED, "device %d beyond %d", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return host_fail(WKV7_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                       hipGetErrorString(e));
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return WKV7_OK;
}

}  // namespace wkv7
