// Launch geometry of the weight-streaming small-M kernels (host side).
//
// Those kernels give each wave 8 weight rows ("a row group") and stage the
// M activation rows in LDS once per workgroup. One wide workgroup per
// compute unit, rather than several narrow ones, keeps the same number of
// waves streaming per CU while staging (and, for W8A8, quantising) the
// activations once per CU instead of once per narrow workgroup, and lets an
// LDS footprint of up to the whole CU hold all groups of a launch at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace w8a8 {

constexpr int kMinWaves = 4;    // waves per workgroup, lower bound
constexpr int kMaxWaves = 12;   // 3 waves per SIMD: the kernels' register budget

// Compute units of the current device, cached per device id (a device
// property: threads that race on the first query store the same value).
inline int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

struct RowGroupGrid {
  int waves;         // waves per workgroup (kMinWaves..kMaxWaves)
  unsigned blocks;   // workgroups
};

// Enough waves per workgroup that one workgroup per CU covers every group
// (from min_waves to kMaxWaves); workgroup b owns groups b*waves ..
// b*waves+waves-1.
inline RowGroupGrid row_group_grid(int64_t N, int min_waves = kMinWaves) {
  const int64_t groups = (N + 7) / 8;
  const int64_t cus = device_cus();
  int64_t w = (groups + cus - 1) / cus;
  w = w < min_waves ? min_waves : (w > kMaxWaves ? kMaxWaves : w);
  return RowGroupGrid{(int)w, (unsigned)((groups + w - 1) / w)};
}

}  // namespace w8a8
