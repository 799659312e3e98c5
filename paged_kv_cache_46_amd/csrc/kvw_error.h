// The message behind the last non-OK status, shared by every source file of
// the library (kvw_last_error() returns it).  One buffer per calling thread.
#pragma once

#include "kvw.h"

namespace kvw_detail {

__attribute__((visibility("hidden"), format(printf, 2, 3)))
kvw_status fail(kvw_status st, const char *fmt, ...);

__attribute__((visibility("hidden"))) const char *last_error();

}  // namespace kvw_detail
