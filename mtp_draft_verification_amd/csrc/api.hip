// api.hip -- status strings, version and the device check of libspecverify.
#include <atomic>
#include <cstring>

#include "sv_host.h"

namespace sv {

static constexpr int kMaxDevices = 64;
// per device: 0 = not queried yet, 1 = gfx950, -1 = something else.  Written once
// per device (racing writers store the same value), read lock-free afterwards.
static std::atomic<int> g_arch[kMaxDevices];
static std::atomic<int> g_cus[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SV_ERR_DEVICE;
  }
  int s = g_arch[dev].load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return SV_ERR_DEVICE;
    }
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch[dev].store(s, std::memory_order_release);
  }
  (void)hipGetLastError();  // start the call's launches from a clean error state
  return s == 1 ? SV_OK : SV_ERR_DEVICE;
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int c = g_cus[dev].load(std::memory_order_relaxed);
  return c > 0 ? c : 256;
}

}  // namespace sv

extern "C" const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_ARG: return "SV_ERR_ARG: invalid argument";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: shape or dtype not implemented";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing or too small";
    case SV_ERR_LAUNCH: return "SV_ERR_LAUNCH: kernel launch failed";
    case SV_ERR_DEVICE: return "SV_ERR_DEVICE: no gfx950 device is current";
    case SV_ERR_SCRATCH: return "SV_ERR_SCRATCH: the call needs more than the library's static scratch";
    default: return "unknown sv_status";
  }
}

extern "C" const char* sv_version(void) { return "libspecverify 0.1.0 gfx950"; }
