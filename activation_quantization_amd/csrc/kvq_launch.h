// Host-side launch helpers shared by the kernels' launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

namespace kvq {

// Workgroups of `kernel` (with `threads` threads) that fit on the device at once, rounded down to
// a multiple of the 8 XCDs, capped at `units`; cached per (kernel, device).
template <typename K>
static int64_t persistent_grid(K kernel, int threads, int64_t units) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int64_t> cache;     // (device, kernel) -> resident workgroups
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t key = ((uint64_t)(uintptr_t)(const void*)kernel << 8) ^ (uint64_t)dev;
  int64_t g;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it == cache.end()) {
      int cus = 0, per_cu = 0;
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
      if (cus < 8) cus = 8;
      g = (int64_t)per_cu * cus;
      g -= g % 8;
      cache.emplace(key, g);
    } else {
      g = it->second;
    }
  }
  return units < g ? units : g;
}

}  // namespace kvq
