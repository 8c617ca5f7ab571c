// Scratch of the no-allocation decode pair (orthros_decode_pair_noalloc):
// a static device array, one copy per device the library runs on, alive
// until the process ends. Its first ORTHROS_NOALLOC_COUNTER_BYTES hold the
// split-KV arrival counters (zero at load; every call leaves them zero), the
// rest the partial results.
//
// Host code never uses the array's name as an address (in host code it is a
// stand-in, not a device pointer): the device address is looked up once per
// device, with that device current, by hipGetSymbolAddress, and kept.
#include <mutex>

#include "../../include/orthros.h"
#include "common.h"

namespace {

__device__ __align__(256) unsigned char scratch[ORTHROS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {nullptr};

}  // namespace

namespace orthros {

hipError_t noalloc_scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace orthros
