// The message behind the last non-OK status, shared by every source file of
// the library (kvw_last_error() returns it).  One buffer per calling thread.
#pragma once

#include "kvw.h"

namespace kvw_detail {

__attribute__((visibility("hidden"), format(printf, 2, 3)))
kvw_status fail(kvw_status st, const char *fmt, ...);

__attribute__((visibility("hidden"))) const char *last_error();

// Context-parallel arguments shared by the write and the read entry points:
// world 0 or 1 is no context parallelism; otherwise 0 <= rank < world, the
// interleave divides block_size and block_size * world fits an int32.
__attribute__((visibility("hidden")))
kvw_status check_cp(const char *fn, int32_t block_size, int32_t world, int32_t rank,
                    int32_t interleave);

}  // namespace kvw_detail
