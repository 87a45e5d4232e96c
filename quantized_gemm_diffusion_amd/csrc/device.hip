// device.hip -- per-device properties the launchers size their grids by,
// looked up once per device and cached (thread-safe).
#include <mutex>

#include "dq_internal.h"

namespace dq {

namespace {
constexpr int kMaxDevices = 64;
// gfx950 parts are built of accelerator complex dies (XCDs) of 32 compute
// units, each with its own L2; a device exposes 1 (CPX partition) to 8 (SPX,
// the whole MI355X) of them.
constexpr int kCusPerXcd = 32;
}  // namespace

DeviceProps device_props() {
  static std::mutex mu;
  static DeviceProps cache[kMaxDevices];
  static bool have[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceProps{};
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    DeviceProps p;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0) {
      p.cus = cus;
      p.xcds = cus >= kCusPerXcd ? cus / kCusPerXcd : 1;
    }
    cache[dev] = p;
    have[dev] = true;
  }
  return cache[dev];
}

}  // namespace dq
