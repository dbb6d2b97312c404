// Host-side status handling of libmoesq: thread-local error detail, status
// names, launch checks and the per-device compute-unit count.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "common.hpp"

namespace moesq {

static thread_local std::string g_last_error;

void clear_error() { g_last_error.clear(); }

moesq_status_t fail(moesq_status_t st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

moesq_status_t launch_status(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MOESQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MOESQ_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moesq

extern "C" {

const char *moesq_status_string(moesq_status_t st) {
  switch (st) {
    case MOESQ_OK: return "MOESQ_OK";
    case MOESQ_ERR_NULL: return "MOESQ_ERR_NULL: a required pointer is NULL";
    case MOESQ_ERR_SHAPE: return "MOESQ_ERR_SHAPE: size outside the supported range";
    case MOESQ_ERR_WORKSPACE: return "MOESQ_ERR_WORKSPACE: workspace missing or too small";
    case MOESQ_ERR_LAYOUT: return "MOESQ_ERR_LAYOUT: unknown weight layout";
    case MOESQ_ERR_HIP: return "MOESQ_ERR_HIP: HIP call or kernel launch failed";
    case MOESQ_ERR_ARG: return "MOESQ_ERR_ARG: invalid argument";
  }
  return "unknown moesq status";
}

const char *moesq_last_error(void) { return moesq::g_last_error.c_str(); }

int32_t moesq_version(void) { return 100; /* 0.1.0 */ }

}  // extern "C"
