// device.cpp -- the shape of the device a call runs on: its compute-unit
// count and, from it, the number of XCDs (gfx950 dies hold 32 active CUs
// each: the full MI355X has 256 CUs in 8 XCDs, a CPX partition 32 in one).
// Queried once per device and cached for the process.
#include <atomic>

#include "sdc_internal.h"

namespace sdc {
namespace {
constexpr int kMaxDevices = 64;
// 0 = not queried yet; else the CU count.  Racing first queries store the same value.
std::atomic<uint32_t> g_cus[kMaxDevices];
}  // namespace

uint32_t xcds_of(uint32_t cus) { return cus >= kCusPerXcd ? cus / kCusPerXcd : 1u; }

int32_t current_device_shape(DeviceShape* out) {
  int dev = 0;
  int32_t st = hip_status(hipGetDevice(&dev));
  if (st) return st;
  uint32_t cus = (dev >= 0 && dev < kMaxDevices) ? g_cus[dev].load(std::memory_order_relaxed) : 0u;
  if (cus == 0) {
    int v = 0;
    st = hip_status(hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev));
    if (st) return st;
    if (v <= 0) return SDC_ERR_RANGE;
    cus = (uint32_t)v;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  out->cus = cus;
  out->xcds = xcds_of(cus);
  return SDC_OK;
}

}  // namespace sdc
