// Host-side facts about the current device used by the kernels that keep every
// workgroup resident (compute units, wall-clock rate), cached per device.
#include <atomic>

#include "internal.h"

namespace dspark {

DeviceInfo device_info() {
  static thread_local DeviceInfo cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return DeviceInfo{};
  DeviceInfo& d = cache[dev];
  if (d.cus == 0) {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&d.clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      d = DeviceInfo{};
  }
  return d;
}

// number of a call of a kernel that marks its own state with it (never 0, the
// value of a zero-filled workspace)
unsigned next_epoch() {
  static std::atomic<unsigned> counter{0};
  unsigned e = counter.fetch_add(1u) + 1u;
  if (e == 0u) e = counter.fetch_add(1u) + 1u;
  return e;
}

}  // namespace dspark
