// Compute-unit and XCD counts of the current device, for the decode plan.
#include <hip/hip_runtime.h>

#include <atomic>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_xcds[kMaxDevices];

}  // namespace

void device_topology(int* cus, int* xcds) {
  *cus = kDefaultCUs;
  *xcds = kDefaultXcds;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // no device: plan for the default topology
    return;
  }
  int c = g_cus[dev].load(std::memory_order_relaxed);
  int x = g_xcds[dev].load(std::memory_order_relaxed);
  if (c <= 0 || x <= 0) {
    int v = 0;
    c = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v
                                                                                                     : kDefaultCUs;
    v = 0;
    x = hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0 ? v : kDefaultXcds;
    (void)hipGetLastError();
    g_xcds[dev].store(x, std::memory_order_relaxed);
    g_cus[dev].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  *xcds = x;
}

}  // namespace mla
