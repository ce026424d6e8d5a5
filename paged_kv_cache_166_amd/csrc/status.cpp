#include "status.h"

#include <cstdarg>
#include <cstdio>

namespace {
thread_local char g_last_error[512] = "";
}

namespace pa {

pa_status fail(pa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_last_error; }
