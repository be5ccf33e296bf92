// Per-device helper streams and events: parts of one call that do not depend on each other run on
// a helper stream and join the caller's stream through events.
#include "common.hpp"

#include <mutex>

namespace gptq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_create;
Helpers* g_helpers[kMaxDevices] = {};

}  // namespace

hipError_t helpers(Helpers** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_create);
  if (!g_helpers[dev]) {
    // built completely before it is published; on a failed create, what was created is destroyed
    // and nothing is cached, so a later call tries again
    Helpers h{};
    int ns = 0, ne = 0;   // streams and events created so far
    while (e == hipSuccess && ns < 2) {
      e = hipStreamCreateWithFlags(&h.stream[ns], hipStreamNonBlocking);
      if (e == hipSuccess) ++ns;
    }
    while (e == hipSuccess && ne < 8) {
      e = hipEventCreateWithFlags(&h.event[ne], hipEventDisableTiming);
      if (e == hipSuccess) ++ne;
    }
    if (e != hipSuccess) {
      for (int i = 0; i < ne; ++i) (void)hipEventDestroy(h.event[i]);
      for (int i = 0; i < ns; ++i) (void)hipStreamDestroy(h.stream[i]);
      return e;
    }
    h.mu = new std::mutex;
    g_helpers[dev] = new Helpers(h);
  }
  *out = g_helpers[dev];
  return hipSuccess;
}

void helpers_lock(Helpers* h) { static_cast<std::mutex*>(h->mu)->lock(); }
void helpers_unlock(Helpers* h) { static_cast<std::mutex*>(h->mu)->unlock(); }

}  // namespace gptq
