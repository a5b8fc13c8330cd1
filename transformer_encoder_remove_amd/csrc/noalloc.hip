// Library-owned scratch memory for the entry point that allocates nothing
// (tel_encoder_layer_forward_noalloc): a file-scope device array, one copy per GPU, held
// until the process ends.
//
// In host code `scratch` names a host-side stand-in of the array, not its device address,
// so it is never passed to a kernel or a copy. The device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept; every later use
// goes through the kept pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "tel.h"

namespace tel {

static_assert(TEL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) char scratch[TEL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = TEL_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace tel
