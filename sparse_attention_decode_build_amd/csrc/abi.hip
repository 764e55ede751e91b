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

}  // namespace sad

extern "C" const char* sad_last_error(void) { return sad::g_error; }
