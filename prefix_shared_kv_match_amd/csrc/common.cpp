#include "common.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }
extern "C" int pkv_version(void) { return 1; }

#ifndef PKV_SOURCE_HASH
#define PKV_SOURCE_HASH "unknown"
#endif
extern "C" const char* pkv_source_hash(void) { return PKV_SOURCE_HASH; }
