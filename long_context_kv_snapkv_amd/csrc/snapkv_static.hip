// Fixed scratch area for snapkv_compress_static: the compression's
// workspace for callers that cannot allocate device memory. The array lives
// in the library's code object, one copy per device the library runs on,
// for the life of the process. Host code never uses the array's name as a
// device address (in host code it names a host-side stand-in): the device
// address is looked up once per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "snapkv_kernels.h"

namespace snapkv {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace snapkv
