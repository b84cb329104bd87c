// launch_attr.hpp -- kernel attributes that must be set on each device before
// a kernel's first launch there, set once per device and thread-safe.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

namespace moe {

// Devices on which an attribute has been set (bit d = device d).  A launcher
// keeps one as a function-local static per kernel configuration.
struct DeviceOnce {
  std::atomic<unsigned long long> done{0};
  std::mutex mu;
};

// Raise the dynamic LDS limit of the kernels `fs` to `bytes` on the current
// device, the first time this is asked for that device.  Devices past the 64
// the mask holds get the call every time (it is idempotent).
inline hipError_t lds_limit_once(DeviceOnce& once, std::initializer_list<const void*> fs, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (once.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  std::lock_guard<std::mutex> g(once.mu);
  if (bit && (once.done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  for (const void* f : fs) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  once.done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

}  // namespace moe
