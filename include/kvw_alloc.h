/*
 * kvw_alloc.h -- contiguous-range block allocator (host side) and the checked
 * coordinate offset of the write path.
 *
 * The allocator hands each request its cache blocks as contiguous ranges, so
 * that the slot of a position is a closed form of its logical block; it is
 * the producer of the range descriptors that kvw_slot_mapping_ranges and
 * kvw_kv_write consume.  Source: "Range-addressed KV cache blocks for the
 * vLLM serving engine", section "The allocator: contiguous ranges as the
 * closed form" (aligned range allocation, an always-coalesced free list,
 * in-place growth for decode, merging of adjacent ranges on append, prefix
 * sharing by reference, least-recently-used eviction of cache-only ranges,
 * request and cache references kept apart) and "Measured Results" (the host
 * scenarios).  The pages list these properties but not the placement policy;
 * the policy below is the plainest one that has them.
 *
 * Model
 * -----
 *  - The pool has num_blocks blocks.  They are handed out in chunks of
 *    `alignment` blocks at chunk-aligned starts (block index a multiple of
 *    alignment), and every count passed in must be a multiple of alignment.
 *    Chunks holding a block below first_block are reserved (block 0 is the
 *    null block of the block table), as is a trailing partial chunk.
 *  - A request occupies a row in [0, max_rows) (its row of the block table
 *    and of the range descriptors).  A row holds an ordered list of extents;
 *    its logical blocks are the blocks of those extents laid end to end.
 *  - An extent [start, start+len) is held by the rows that list it (request
 *    references) and optionally by one prefix-cache key (a cache reference).
 *    It is free again when it has neither.  An extent held only by the cache
 *    is "cache-only" and sits in a least-recently-used list, in the order in
 *    which it became cache-only.
 *  - Placement (first fit): n blocks go at the lowest chunk-aligned start
 *    whose next n blocks are all free.  If no free run is that long, the
 *    lowest free runs are taken in address order, whole, the last one only
 *    as far as needed, each becoming one extent.
 *  - Growth in place: a row whose last extent it holds alone, uncached, and
 *    whose next n blocks are free grows that extent instead.
 *  - Eviction: when fewer than n blocks are free, cache-only extents are
 *    evicted oldest first until n blocks are free; if even evicting all of
 *    them would not free enough, the call fails and changes nothing.
 *  - Export: a row's ranges are its extents with physically adjacent
 *    neighbours merged, so a row that only ever grows keeps one range.
 *
 * Conventions: host memory only; not thread-safe (one allocator per
 * scheduler thread); every call returns a kvw_status and on failure changes
 * nothing; kvw_last_error() describes the failure.
 */
#ifndef KVW_ALLOC_H
#define KVW_ALLOC_H

#include <stdint.h>

#include "kvw.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvw_alloc kvw_alloc;

/* Statistics of an allocator (all counts in blocks unless named otherwise). */
typedef struct kvw_alloc_stats {
    int64_t usable_blocks;     /* blocks that can ever be handed out */
    int64_t free_blocks;       /* neither request- nor cache-held */
    int64_t cache_only_blocks; /* held by the prefix cache alone (evictable) */
    int64_t free_runs;         /* maximal runs of free blocks (coalesced free list length) */
    int64_t extents;           /* live extents */
    int64_t cache_entries;     /* keys in the prefix cache */
} kvw_alloc_stats;

/* Create an allocator over num_blocks blocks with the given alignment
 * (>= 1), rows [0, max_rows), blocks below first_block reserved.
 * KVW_ERR_INVALID_ARG for non-positive sizes or num_blocks > 2^31 - 1. */
kvw_status kvw_alloc_create(int64_t num_blocks, int32_t alignment, int64_t first_block,
                            int32_t max_rows, kvw_alloc **out);
void kvw_alloc_destroy(kvw_alloc *a);

/* Append num_blocks blocks to row `row` (empty or not): in place, else
 * first fit, else the lowest free runs; evicting cache-only extents first
 * when too few blocks are free.  KVW_ERR_NO_SPACE when even full eviction
 * would not make room; KVW_ERR_INVALID_ARG for a bad row or a count that is
 * negative or not a multiple of the alignment. */
kvw_status kvw_alloc_extend(kvw_alloc *a, int32_t row, int64_t num_blocks);

/* Drop row `row`'s references; its extents that nobody holds are freed (and
 * coalesced), those the cache holds become cache-only (newest in the LRU
 * list, in the row's order).  The row becomes empty. */
kvw_status kvw_alloc_release(kvw_alloc *a, int32_t row);

/* Register logical blocks [first, first+count) of row `row` under `key`.
 * They must lie inside one extent of the row that is not cached yet (such an
 * extent has this row as its only holder: extents are shared only through
 * the cache); if they are a strict part of it, the extent is split into up
 * to three.  first and count: multiples of the alignment, count > 0.
 * KVW_ERR_INVALID_ARG otherwise, or if the key exists. */
kvw_status kvw_alloc_cache_insert(kvw_alloc *a, uint64_t key, int32_t row, int64_t first,
                                  int64_t count);

/* Append the extent cached under `key` to row `row`, by reference (a prefix
 * hit); a cache-only extent leaves the LRU list.  KVW_ERR_NOT_FOUND if the
 * key is absent. */
kvw_status kvw_alloc_cache_acquire(kvw_alloc *a, uint64_t key, int32_t row);

/* Evict up to max_extents cache-only extents, oldest first; *evicted (may be
 * NULL) receives how many were evicted. */
kvw_status kvw_alloc_cache_evict(kvw_alloc *a, int64_t max_extents, int64_t *evicted);

/* Range descriptors of rows rows[0..n) (host arrays, as the GPU calls take
 * them): start, len, cum int32[n][range_stride], num_ranges int32[n].
 * Entries past a row's count are 0.  KVW_ERR_RANGE_CAP (nothing written)
 * when a row has more than range_stride ranges. */
kvw_status kvw_alloc_ranges(const kvw_alloc *a, const int32_t *rows, int32_t n,
                            int32_t range_stride, int32_t *start, int32_t *len, int32_t *cum,
                            int32_t *num_ranges);

/* Block table rows of rows[0..n): table int32[n][stride] (blocks in logical
 * order, 0 past the count), counts int32[n] (may be NULL).
 * KVW_ERR_RANGE_CAP (nothing written) when a row holds more than stride
 * blocks. */
kvw_status kvw_alloc_block_table(const kvw_alloc *a, const int32_t *rows, int32_t n,
                                 int32_t stride, int32_t *table, int32_t *counts);

/* Extents of row `row` in order: up to max entries of (start, len) into
 * starts/lens; *count (may be NULL) receives the row's extent count. */
kvw_status kvw_alloc_row_extents(const kvw_alloc *a, int32_t row, int32_t max, int64_t *starts,
                                 int64_t *lens, int32_t *count);

/* Free runs in address order: up to max (start, len) pairs; *count receives
 * the number of runs. */
kvw_status kvw_alloc_free_runs(const kvw_alloc *a, int64_t max, int64_t *starts, int64_t *lens,
                               int64_t *count);

/* Cache-only extents, oldest first: up to max (start, len) pairs; *count
 * receives how many there are. */
kvw_status kvw_alloc_lru(const kvw_alloc *a, int64_t max, int64_t *starts, int64_t *lens,
                         int64_t *count);

kvw_status kvw_alloc_get_stats(const kvw_alloc *a, kvw_alloc_stats *out);

/* Checked coordinate offset ("The Coordinate Approach"): for layer < L,
 * block < B, token < T, *offset = ((layer*B + block)*T + token) *
 * bytes_per_token.  KVW_ERR_INVALID_ARG for a coordinate out of range or a
 * negative size, KVW_ERR_UNSUPPORTED if the offset overflows int64. */
kvw_status kvw_coord_offset(int64_t layer, int64_t block, int64_t token, int64_t num_layers,
                            int64_t num_blocks, int64_t block_size, int64_t bytes_per_token,
                            int64_t *offset);

/* The same computation inline, for per-token host loops that should not pay a
 * call into the shared library: the same result and status as
 * kvw_coord_offset for every input, but no error message is recorded
 * (kvw_last_error is left as it was).  kvw_coord_offset is this function plus
 * the message.  Needs GCC or Clang (checked-arithmetic builtins). */
static inline kvw_status kvw_coord_offset_inline(int64_t layer, int64_t block, int64_t token,
                                                 int64_t num_layers, int64_t num_blocks,
                                                 int64_t block_size, int64_t bytes_per_token,
                                                 int64_t *offset)
{
    uint64_t n = 0;
    /* unsigned compares reject negative coordinates too */
    if (!offset || bytes_per_token < 0 || (uint64_t)layer >= (uint64_t)num_layers ||
        (uint64_t)block >= (uint64_t)num_blocks || (uint64_t)token >= (uint64_t)block_size)
        return KVW_ERR_INVALID_ARG;
    /* Checked 64-bit steps.  The sizes are at least 1 here (each exceeds its
     * coordinate), so with bytes_per_token >= 1 every partial value is at most
     * the result, and a step wraps only when the result exceeds 2^64 - 1. */
    if (bytes_per_token > 0 &&
        (__builtin_mul_overflow((uint64_t)layer, (uint64_t)num_blocks, &n) ||
         __builtin_add_overflow(n, (uint64_t)block, &n) ||
         __builtin_mul_overflow(n, (uint64_t)block_size, &n) ||
         __builtin_add_overflow(n, (uint64_t)token, &n) ||
         __builtin_mul_overflow(n, (uint64_t)bytes_per_token, &n) || n > (uint64_t)INT64_MAX))
        return KVW_ERR_UNSUPPORTED;
    *offset = (int64_t)n;
    return KVW_OK;
}

#ifdef __cplusplus
}
#endif

#endif /* KVW_ALLOC_H */
