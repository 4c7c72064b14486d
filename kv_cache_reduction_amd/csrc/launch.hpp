// Host helpers for kernel launches.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace slim {

constexpr int kMaxDevices = 64;

// Raises a kernel's dynamic LDS limit to `lds` bytes on the current device
// (hipFuncSetAttribute), remembering per device the largest size already
// granted, so that the attribute call is made once per device and size.
// Sizes up to 64 KB need no attribute.  Safe to call from several threads.
inline hipError_t allow_lds(const void* kern, size_t lds, std::atomic<int> (&granted)[kMaxDevices]) {
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  std::atomic<int>* g = (dev >= 0 && dev < kMaxDevices) ? &granted[dev] : nullptr;
  if (g && g->load(std::memory_order_relaxed) >= (int)lds) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (g) {
    int cur = g->load(std::memory_order_relaxed);
    while (cur < (int)lds && !g->compare_exchange_weak(cur, (int)lds, std::memory_order_relaxed)) {
    }
  }
  return hipSuccess;
}

}  // namespace slim
