// Host-side launch helpers shared by the launchers: compute units of the
// current device and how many workgroups of a kernel one compute unit holds.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace sdpa14 {

// Compute units of the current device, looked up once per device (0 on error).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of kernel K resident per compute unit (queried once per kernel; 0 on error).
template <auto K>
int resident_per_cu(int threads) {
  static std::atomic<int> cache{-1};
  int n = cache.load(std::memory_order_relaxed);
  if (n < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, threads, 0) != hipSuccess) n = 0;
    cache.store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace sdpa14
