// Status messages of the C ABI (host only): the thread-local text behind
// tcs_last_error, and the library version string.
#include <cstdarg>
#include <cstdio>

#include "tcs_internal.h"

namespace tcs {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

}  // namespace tcs

extern "C" const char* tcs_last_error(void) { return tcs::g_err; }
extern "C" const char* tcs_version(void) { return "libtcs 0.2 (gfx950)"; }
