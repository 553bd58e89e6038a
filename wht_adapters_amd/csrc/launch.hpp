// Host-side launch helpers: persistent grids sized from the device's CU
// count and each kernel instance's occupancy (queried once, then cached).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

namespace whtq {

int device_cu_count(int dev);  // defined in abi.hip (per-device cache)

template <typename K>
int blocks_per_cu(K kernel, int block, size_t dyn_lds) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, block, dyn_lds) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

// Grid of min(groups, CUs * resident blocks) for a grid-stride kernel.
// `nb` is the kernel's resident blocks per CU (callers cache it per instance).
inline unsigned persistent_grid(int64_t groups, int nb) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int64_t cap = (int64_t)device_cu_count(dev) * nb;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(groups, cap));
}

}  // namespace whtq
