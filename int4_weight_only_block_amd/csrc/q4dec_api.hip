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

Q4DEC_DEBUG_READER(api)

// fails its one check on purpose, so a debug build's reporting can be tested
__global__ void debug_selftest_kernel() { Q4_DCHECK(false, kDbgSelfTest); }

}  // namespace q4dec

extern "C" {

int q4dec_debug_status(uint32_t* word) {
  using namespace q4dec;
  if (!word) return fail(Q4DEC_ERR_NULL, "q4dec_debug_status: word is NULL");
  *word = 0;
  if (!Q4DEC_DEBUG)
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4dec_debug_status: library built without Q4DEC_DEBUG");
  const hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(Q4DEC_ERR_HIP, "q4dec_debug_status: %s", hipGetErrorString(e));
  *word = debug_take_q4_gemv() | debug_take_q4_multi() | debug_take_q4_chain() | debug_take_q4_gemm() |
          debug_take_rowq_gemv() | debug_take_ple_gather() | debug_take_q4_pack() | debug_take_q4_quantize() |
          debug_take_api();
  return Q4DEC_OK;
}

int q4dec_debug_selftest(void* stream) {
  using namespace q4dec;
  if (!Q4DEC_DEBUG)
    return fail(Q4DEC_ERR_UNSUPPORTED, "q4dec_debug_selftest: library built without Q4DEC_DEBUG");
  hipLaunchKernelGGL(debug_selftest_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return launch_status("q4dec_debug_selftest");
}

int32_t q4dec_abi_version(void) { return Q4DEC_ABI_VERSION; }

const char* q4dec_last_error(void) { return q4dec::g_err; }

size_t q4_packed_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || (k % 32) != 0) return 0;
  return q4dec::nib_plane_bytes(n, k) + q4dec::scale_plane_bytes(n, k);
}

}  // extern "C"
