// Static device scratch for the allocation-free decode entry point
// (diffattn_decode_noalloc): the split partials of the decode step live in a file-scope
// device array instead of a caller workspace. Every device the library runs on holds its
// own copy, DIFFATTN_DECODE_SCRATCH_BYTES long, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to a kernel.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "diffattn.h"
#include "launch.h"

static __device__ __align__(256) float scratch[DIFFATTN_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace diffattn {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<float*> g_ptr[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_lookup;

}  // namespace

hipError_t decode_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<float*>(addr);
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace diffattn
