// The library's one allocation-free scratch buffer: a static device array that holds the factor's
// workspace (status words, sort keys and the three staging panels) for gptq_factor_noalloc, for
// callers that cannot allocate device memory.
//
// Every device the library runs on holds its own copy of the array, at its own address, until the
// process ends. The array's name is only a host-side stand-in for the symbol: host code takes each
// device's address once with hipGetSymbolAddress (with that device current) and passes that pointer
// to the kernels, never the name. Calls on one device share its copy, so calls that overlap on one
// device race.
#include "common.hpp"

#include <mutex>

namespace gptq {
namespace {

__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace gptq
