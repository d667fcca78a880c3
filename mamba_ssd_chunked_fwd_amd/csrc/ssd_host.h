// ssd_host.h -- host-side helpers shared by the kernel launchers (internal
// to libssd): per-device caches of launch properties, and clearing the HIP
// error state before a launch.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace ssd {

constexpr int kMaxDevices = 64;

// One positive int per device (a CU count, a resident-workgroup count):
// properties of the device model and of a kernel, computed on first use on
// each device and never changed afterwards.  Devices past kMaxDevices are
// computed on every call.  Objects of this type live in static storage,
// which zero-initialises the slots.
struct PerDeviceInt {
  std::atomic<int> slot[kMaxDevices];

  template <class F>
  int get(F compute) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < 0 || dev >= kMaxDevices) return compute(dev);
    int v = slot[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    v = compute(dev);
    if (v > 0) slot[dev].store(v, std::memory_order_relaxed);
    return v;
  }
};

// Compute units of device `dev` (0 if the query fails).
inline int query_cus(int dev) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// Workgroups of `kernel` (`threads` threads, no dynamic LDS) resident on all
// compute units of the current device `dev` at once, rounded down to a
// multiple of 8 so the XCD-aware placement of the persistent kernels
// applies; 0 if a query fails.
inline int resident_slots(const void* kernel, int threads, int dev) {
  const int cus = query_cus(dev);
  int per = 0;
  if (cus <= 0) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess)
    return 0;
  const int slots = (per < 1 ? 1 : per) * cus;
  return slots < 8 ? slots : slots / 8 * 8;
}

// Reset the calling thread's last HIP error, so that the error read after a
// launch belongs to that launch and not to an unrelated earlier call.
inline void clear_launch_error() { (void)hipGetLastError(); }

}  // namespace ssd
