// Thread-local error message behind pa_last_error().
#include "pa_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }
extern "C" const char* pa_version(void) { return "paged_kv_cache_212_amd 0.1.0 (gfx950)"; }
