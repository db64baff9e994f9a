// Status reporting shared by every entry point of libstp.
#include <stdarg.h>
#include <stdio.h>

#include "stp_internal.h"

namespace {
thread_local char g_last_error[512] = "no error";
}

namespace stp {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(STP_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return STP_OK;
}

int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace stp

extern "C" const char* stp_last_error(void) { return g_last_error; }

extern "C" const char* stp_version(void) { return "stp 0.1 gfx950"; }

extern "C" int stp_host_device_pointer(const void* host, void** dev) {
  if (!host || !dev) return stp::fail(STP_ERR_INVALID_ARG, "host_device_pointer: null pointer");
  if (hipHostGetDevicePointer(dev, const_cast<void*>(host), 0) != hipSuccess)
    return stp::fail(STP_ERR_HIP, "host_device_pointer: not pinned host memory");
  return STP_OK;
}
