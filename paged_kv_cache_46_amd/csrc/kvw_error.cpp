// The message behind the last non-OK status of any entry point, one buffer per
// calling thread (kvw_last_error() in include/kvw.h returns it).

#include <cstdarg>
#include <cstdio>

#include "kvw.h"
#include "kvw_error.h"

namespace kvw_detail {

namespace {
thread_local char g_last_error[512] = "";
}

kvw_status fail(kvw_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

const char *last_error() { return g_last_error; }

}  // namespace kvw_detail

extern "C" const char *kvw_last_error(void) { return kvw_detail::last_error(); }
