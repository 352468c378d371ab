// Status reporting shared by every entry point of libcsahca.so.
#include "common.hpp"

namespace csahca {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

}  // namespace csahca

extern "C" const char* csahca_last_error(void) { return csahca::g_last_error.c_str(); }

extern "C" int csahca_version(void) { return 10000; }
