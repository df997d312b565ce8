// Device scratch for the no-allocation entry point (agmm_run_noalloc).
//
// A file-scope device array holds the split-K partial sums of callers that
// cannot allocate device memory.  Every GPU the library runs on holds its own
// copy from the moment the library's code is loaded on it until the process
// ends.  In host code the array's name is only a host-side stand-in for it:
// its device address, which differs from GPU to GPU, is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept, and
// only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "agmm_kernels.h"

namespace agmm {

namespace {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace agmm
