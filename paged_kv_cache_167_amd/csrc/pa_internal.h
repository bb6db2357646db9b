// Internal to libpa.so: the per-thread error text that every C entry point sets, shared
// by the library's source files.
#ifndef PA_INTERNAL_H
#define PA_INTERNAL_H

#include <cstdarg>
#include <cstdio>
#include <string>

namespace pa_detail {

inline thread_local std::string g_error;

// Record a formatted error and return its code.
inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

}  // namespace pa_detail

#endif  // PA_INTERNAL_H
