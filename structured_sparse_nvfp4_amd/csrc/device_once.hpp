// Per-device, thread-safe one-time set-up for the host launchers: the first call on each device
// runs `f` with that device current and keeps its status; later calls on that device return the
// kept status without running it again. std::call_once makes concurrent first calls from
// several host threads safe.
#pragma once
#include <hip/hip_runtime.h>

#include <mutex>

namespace ssn {

constexpr int kMaxDevices = 64;

struct PerDeviceOnce {
  std::once_flag flag[kMaxDevices];
  hipError_t status[kMaxDevices] = {};
};

template <typename F>
hipError_t once_per_device(PerDeviceOnce& o, F&& f) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return f();   // beyond the table: set up on every call
  std::call_once(o.flag[dev], [&] { o.status[dev] = f(); });
  return o.status[dev];
}

// Compute units of the current device (cached per device; 256 if the query fails).
inline int cu_count() {
  static PerDeviceOnce once;
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  (void)once_per_device(once, [&]() -> hipError_t {   // always succeeds: 256 CUs if the query fails
    int n = 0;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    cus[dev] = (e == hipSuccess && n > 0) ? n : 256;
    return hipSuccess;
  });
  return cus[dev];
}

}  // namespace ssn
