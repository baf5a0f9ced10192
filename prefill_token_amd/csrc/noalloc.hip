// Static device scratch of the allocation-free entry point (sparse_mla_fwd_noalloc).
//
// The step's kernels take their scratch -- the work-item scheduler's counters, the item
// order of an unsplit call, the split partials -- from one buffer.  sparse_mla_fwd takes it
// from the caller's workspace; the allocation-free variant takes it from `scratch` below,
// a file-scope device array that every GPU the library runs on holds (zero-filled when the
// code object loads) until the process ends.  In host code the array's name is only a
// stand-in: its device address, which differs per GPU, is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; only that address is ever
// passed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "smla.h"
#include "smla_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

}  // namespace

namespace smla {

hipError_t noalloc_scratch(void** ptr) {
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

}  // namespace smla
