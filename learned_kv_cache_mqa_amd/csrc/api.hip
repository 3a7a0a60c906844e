// Host-side plumbing shared by every entry point: status strings, the thread-local
// error message and the gfx950 device check.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "common.hpp"

namespace kvm {

static thread_local char g_err[512] = "";

kvm_status set_error(kvm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvm_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVM_OK;
  return set_error(KVM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// 0 = unknown, 1 = gfx950, 2 = other architecture
static std::atomic<int> g_arch[64];

kvm_status require_gfx950() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return set_error(KVM_ERR_ARCH, "device index %d out of range", dev);
  int v = g_arch[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return check_hip(e, "hipGetDeviceProperties");
    v = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(v, std::memory_order_relaxed);
    if (v != 1) return set_error(KVM_ERR_ARCH, "device %d is %s, not gfx950", dev, p.gcnArchName);
  }
  return v == 1 ? KVM_OK : set_error(KVM_ERR_ARCH, "device %d is not gfx950", dev);
}

}  // namespace kvm

extern "C" int kvm_abi_version(void) { return KVM_ABI_VERSION; }

extern "C" const char* kvm_status_string(kvm_status s) {
  switch (s) {
    case KVM_OK: return "ok";
    case KVM_ERR_NULL: return "null pointer";
    case KVM_ERR_SHAPE: return "bad shape";
    case KVM_ERR_DTYPE: return "bad dtype";
    case KVM_ERR_ALIGN: return "misaligned pointer";
    case KVM_ERR_RANGE: return "value out of range";
    case KVM_ERR_WORKSPACE: return "workspace too small";
    case KVM_ERR_ARCH: return "device is not gfx950";
    case KVM_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" const char* kvm_last_error(void) { return kvm::g_err; }

extern "C" kvm_status kvm_check_device(void) { return kvm::require_gfx950(); }
