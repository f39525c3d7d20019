// Library-wide host entry points: ABI version, error text, sizes, device cache.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "q4dec_internal.h"

namespace q4dec {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

}  // namespace q4dec

extern "C" {

int32_t q4dec_abi_version(void) { return Q4DEC_ABI_VERSION; }

const char* q4dec_last_error(void) { return q4dec::g_err; }

size_t q4_packed_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || (k % 32) != 0) return 0;
  return q4dec::nib_plane_bytes(n, k) + q4dec::scale_plane_bytes(n, k);
}

}  // extern "C"
