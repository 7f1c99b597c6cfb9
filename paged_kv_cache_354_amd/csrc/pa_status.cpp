#include "pa_status.h"

namespace {
thread_local char g_last_error[512] = "no error";
}

namespace pa {

pa_status_t fail(pa_status_t code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pa

extern "C" const char *pa_last_error(void) { return g_last_error; }

extern "C" const char *pa_version(void) { return "pagedkv 0.1 gfx950"; }
