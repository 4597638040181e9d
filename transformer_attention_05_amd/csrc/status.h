// Thread-local error text behind attn_last_error().
#pragma once

#include <cstdarg>
#include <cstdio>

#include "mi_attn.h"

namespace mi_attn {

char* error_buffer();

inline int ok() {
  error_buffer()[0] = '\0';
  return ATTN_OK;
}

#if defined(__GNUC__)
__attribute__((format(printf, 2, 3)))
#endif
inline int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(error_buffer(), 512, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace mi_attn
