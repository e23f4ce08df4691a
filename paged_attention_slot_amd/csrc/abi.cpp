// Error reporting and version of libpkv's C ABI.
#include <cstdio>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

pkv_status fail(pkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pkv

extern "C" {

int32_t pkv_version(void) { return 100; }  // 0.1.0

const char* pkv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
