// escha_static.hip -- the library's one device-resident scratch array, for
// the entry point that allocates nothing (escha_moe_layer_decode_static).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the name is only a host-side stand-in, so its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; kernels and host calls only ever see that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "escha_launch.hpp"

namespace escha {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace escha
