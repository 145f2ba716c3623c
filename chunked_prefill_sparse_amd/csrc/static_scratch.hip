// The static device array behind ca_chunk_attention_split_noalloc, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  One copy per device,
// held from the library's load on that device until the process ends.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address: passing it to a kernel would fault.  The device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.

#include <mutex>

#include "kernels.hpp"

namespace {

__device__ __align__(256) unsigned char scratch[CA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

}  // namespace

namespace ca {

void* static_scratch_address(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  *err = hipSuccess;
  return addr[dev];
}

}  // namespace ca
