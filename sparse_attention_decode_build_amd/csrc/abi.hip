// Error state shared by every libsad.so entry point.
#include <stdarg.h>
#include <stdio.h>

#include "sad_internal.h"

namespace sad {

static thread_local char g_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_error[0] = '\0'; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return SAD_ELAUNCH;
  }
  return SAD_OK;
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();  // a failed query must not read as a later launch failure
    return 256;
  }
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  return n;
}

}  // namespace sad

extern "C" const char* sad_last_error(void) { return sad::g_error; }
