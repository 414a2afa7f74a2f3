// Library-wide entry points: version and error text.
#include <string>

#include "sa2_common.h"

namespace sa2 {

static thread_local std::string g_last_error;

sa2_status fail(sa2_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

sa2_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SA2_EDEVICE, std::string(what) + ": launch failed: " + hipGetErrorString(e));
  return SA2_OK;
}

}  // namespace sa2

extern "C" const char* sa2_version(void) { return "sa2 0.1.0 gfx950"; }

extern "C" const char* sa2_last_error(void) { return sa2::g_last_error.c_str(); }
