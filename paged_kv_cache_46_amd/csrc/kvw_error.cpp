// The message behind the last non-OK status of any entry point, one buffer per
// calling thread (kvw_last_error() in include/kvw.h returns it), and the
// argument checks that more than one source file of the library applies.

#include <cstdarg>
#include <cstdint>
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

kvw_status check_cp(const char *fn, int32_t block_size, int32_t world, int32_t rank,
                    int32_t interleave)
{
    if (world < 0) return fail(KVW_ERR_INVALID_ARG, "%s: cp_world_size %d is negative", fn, world);
    if (world == 0) return KVW_OK;
    if (rank < 0 || rank >= world)
        return fail(KVW_ERR_INVALID_ARG, "%s: cp_rank %d outside [0, %d)", fn, rank, world);
    if (interleave < 1 || block_size % interleave != 0)
        return fail(KVW_ERR_INVALID_ARG, "%s: cp_interleave_size %d does not divide block_size %d",
                    fn, interleave, block_size);
    if (static_cast<int64_t>(block_size) * world > INT32_MAX)
        return fail(KVW_ERR_INVALID_ARG, "%s: block_size * cp_world_size overflows int32", fn);
    return KVW_OK;
}

}  // namespace kvw_detail

extern "C" const char *kvw_last_error(void) { return kvw_detail::last_error(); }
