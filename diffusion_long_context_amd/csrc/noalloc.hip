// Library-held scratch memory of the decode entry point that allocates
// nothing (pdllm_split_attn_decode_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, zero-filled when the code object is loaded, until the
// process ends.  In host code its name is only a host-side stand-in, so host
// code never passes it: the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pdllm_internal.h"

namespace pdllm {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return (int)hipSuccess;
}

}  // namespace pdllm
