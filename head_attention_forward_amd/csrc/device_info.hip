// Launch-shape facts of the current device, read from the runtime once per
// device: compute units (how many workgroups fill the chip) and XCDs (how
// many L2 domains workgroups are dealt to, round-robin by workgroup index).
#include <mutex>

#include "kernels.h"

namespace mha {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  int cus = 0;
  int xcds = 0;
};
std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

const DeviceInfo& info() {
  static const DeviceInfo fallback{256, 8};  // MI355X, if the runtime cannot say
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
  std::call_once(g_once[dev], [dev] {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0)
      xcds = 8;
    g_info[dev] = DeviceInfo{cus, xcds};
  });
  return g_info[dev];
}

}  // namespace

int device_compute_units() { return info().cus; }
int device_xcds() { return info().xcds; }

}  // namespace mha
