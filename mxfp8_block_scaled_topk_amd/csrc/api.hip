// Host-side plumbing of the C ABI: thread-local error text, launch checks,
// device properties.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "common.h"

namespace mxmoe {

namespace {
thread_local std::string g_last_error = "no error";
std::mutex g_cu_mutex;
int g_cus[64] = {0};
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MX_OK;
}

int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

}  // namespace mxmoe

extern "C" const char* mx_last_error(void) { return mxmoe::g_last_error.c_str(); }
