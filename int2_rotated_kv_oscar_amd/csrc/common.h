// Internal helpers shared by the liboscar translation units (not part of the ABI).
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/oscar.h"

namespace oscar {

// Thread-local detail for the last non-OK status (oscar_last_error()).
void set_error(const char* fmt, ...);
void clear_error();

inline oscar_status fail(oscar_status s, const char* what) {
  set_error("%s: %s", oscar_status_string(s), what);
  return s;
}

}  // namespace oscar
