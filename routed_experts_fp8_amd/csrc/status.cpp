// Status strings, thread-local error detail and the post-launch check of the
// libmoefp8 C ABI.
#include <stdlib.h>
#include <atomic>
#include <string.h>

#include "host_common.h"

namespace moefp8 {

static thread_local char g_detail[512];

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}

void clear_detail() { g_detail[0] = '\0'; }

static bool sync_check_enabled() {
  static const bool on = [] {
    const char* v = getenv("MOEFP8_SYNC_CHECK");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

moe_status after_launch(const char* what, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (sync_check_enabled()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: device error: %s", what, hipGetErrorString(e));
  }
  return MOE_OK;
}

// Compute units of the current device (looked up once per device; the
// stored value is the same whichever thread stores it).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace moefp8

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: invalid or inconsistent sizes";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: request outside the implemented range";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer not aligned as required";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}

extern "C" const char* moe_last_error_detail(void) { return moefp8::g_detail; }
