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
    Helpers* h = new Helpers{};
    for (auto& st : h->stream)
      if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
    for (auto& ev : h->event)
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
    h->mu = new std::mutex;
    g_helpers[dev] = h;
  }
  *out = g_helpers[dev];
  return hipSuccess;
}

void helpers_lock(Helpers* h) { static_cast<std::mutex*>(h->mu)->lock(); }
void helpers_unlock(Helpers* h) { static_cast<std::mutex*>(h->mu)->unlock(); }

}  // namespace gptq
