// Thread-local error reporting behind pa_last_error().
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "pa_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pa {

pa_status fail(pa_status code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_msg[0] = '\0'; }

pa_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

extern "C" const char *pa_last_error(void) { return g_msg; }
extern "C" const char *pa_version(void) { return "0.1.0"; }
