/*
 * CPU oracle of the paged KV-cache write path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the write path computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant generator with the GPU library; the few
 * numeric conventions both must agree on (the pad id, the flag bits) are
 * restated here from the interface documentation.
 *
 * Sources (pages as published; sections named, not quoted):
 *  [P1] "Range-addressed KV cache blocks for the vLLM serving engine",
 *       sections "The block-table access pattern", "The Innovation: Range
 *       Arithmetic Replaces the Per-Position Gather", "The Coordinate
 *       Approach", "The Direction", "Measured Results" and "Status".
 *  [P2] "Blocktabelle: Abbildung von logischen Token auf physische KV-Blocks",
 *       sections "Verantwortung", "Entwurfsmotivation", "Datenfluss" and
 *       "Grenzen und Fehler".
 *  [P3] "vLLM Block Table Management: From PagedAttention to the V1 KV Cache
 *       Stack", "Symbol Map" (the block_size row) and Deep Dive sections 7
 *       ("Worker-side block table materialization") and 8 ("slot_mapping:
 *       token -> physical slot").
 *
 * Every loop below walks the definition in the order it is stated; nothing
 * is blocked, fused or reordered.  Integer arithmetic is done in int64.
 *
 * Readings where the pages leave a step open:
 *  - a token whose position is negative, or whose logical block lies past
 *    the blocks its request owns, or past every range, gets the pad id;
 *  - range descriptors are (start, len, cum) with cum the exclusive prefix
 *    sum of len; the first range containing the logical block is used;
 *  - a manager block b expands to kernel blocks b*k .. b*k+k-1, k the ratio
 *    of the block sizes; table entries past a row's count become block 0;
 *  - a padded token writes nothing; a slot outside the cache is skipped and
 *    reported through a flag bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PAD_ID (-1)

/* Return codes of the oracle: 0 = computed; >0 = the input violates a
 * precondition the oracle checks (the output is then not meaningful). */
#define ORC_OK 0
#define ORC_E_ARG 1
#define ORC_E_QSL 2
#define ORC_E_RANGES 3
#define ORC_E_DUPLICATE 4

/* Flag bits reported for recoverable, data-dependent conditions. */
#define ORC_FLAG_NUM_TOKENS 1u /* query_start_loc[num_reqs] outside [0, max_num_tokens] */
#define ORC_FLAG_COUNT 2u      /* per-request block or range count outside [0, stride] */
#define ORC_FLAG_BAD_BLOCK 4u  /* resolved physical block id negative or not representable */
#define ORC_FLAG_SLOT_OOB 8u   /* slot past the cache: the write is skipped */

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi, uint32_t *flags, uint32_t bit)
{
    if (v < lo) { *flags |= bit; return lo; }
    if (v > hi) { *flags |= bit; return hi; }
    return v;
}

/* Number of tokens scheduled this step: the last entry of query_start_loc
 * ([P2] "Datenfluss": the kernel's token ranges per request). */
static int64_t num_tokens_of(const int32_t *qsl, int32_t num_reqs, int64_t max_num_tokens,
                             uint32_t *flags)
{
    return clamp64((int64_t)qsl[num_reqs], 0, max_num_tokens, flags, ORC_FLAG_NUM_TOKENS);
}

static int qsl_ok(const int32_t *qsl, int32_t num_reqs)
{
    if (qsl[0] < 0) return 0;
    for (int32_t r = 0; r < num_reqs; ++r)
        if (qsl[r + 1] < qsl[r]) return 0;
    return 1;
}

/*
 * Paged slot mapping ([P2] "Entwurfsmotivation", slot_mapping as a kernel;
 * [P3] section 8): for token t of request r at position p,
 *   logical block  = p / block_size,  offset = p % block_size,
 *   physical block = block_table[r][logical block],
 *   slot           = physical block * block_size + offset,
 * and every entry from num_tokens up to max_num_tokens is the pad id
 * ([P2] "Datenfluss": the last program pads the tail for graph replay).
 * num_blocks_per_req (may be NULL) bounds the valid logical blocks of a row;
 * NULL means the full row width.  A request's count is read (clamped to
 * [0, table_stride], flagged if outside) for each of its tokens with a
 * non-negative position.  With max_num_tokens == 0 nothing is read.
 */
int orc_slot_mapping_paged(const int32_t *qsl, int32_t num_reqs, const int64_t *positions,
                           int64_t max_num_tokens, const int32_t *block_table,
                           int32_t table_stride, const int32_t *num_blocks_per_req,
                           int32_t block_size, int64_t *slot_mapping, uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (!qsl || num_reqs < 0 || max_num_tokens < 0 || block_size <= 0 || table_stride < 0 ||
        (max_num_tokens > 0 && !slot_mapping))
        return ORC_E_ARG;
    if (!qsl_ok(qsl, num_reqs)) return ORC_E_QSL;

    if (max_num_tokens == 0) return ORC_OK;            /* no token rows: nothing is read */
    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = ORC_PAD_ID;
    int64_t num_tokens = num_tokens_of(qsl, num_reqs, max_num_tokens, &flags);

    for (int32_t r = 0; r < num_reqs; ++r) {
        for (int64_t t = qsl[r]; t < qsl[r + 1] && t < num_tokens; ++t) {
            int64_t p = positions[t];
            if (p < 0) continue;                       /* pad id */
            int64_t bound = table_stride;
            if (num_blocks_per_req)
                bound = clamp64(num_blocks_per_req[r], 0, table_stride, &flags, ORC_FLAG_COUNT);
            int64_t logical = p / block_size;
            int64_t offset = p % block_size;
            if (logical >= bound) continue;            /* no block owned there: pad id */
            int64_t physical = block_table[(int64_t)r * table_stride + logical];
            if (physical < 0) { flags |= ORC_FLAG_BAD_BLOCK; continue; }
            slot_mapping[t] = physical * block_size + offset;
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/*
 * Range-arithmetic slot mapping ([P1] "The Innovation"): a request's blocks
 * are contiguous runs; run i covers logical blocks [cum[i], cum[i]+len[i])
 * and starts at physical block start[i], so
 *   physical block = start[i] + (logical block - cum[i]).
 * A position inside no run gets the pad id.  The oracle scans the runs in
 * order and takes the first that contains the logical block.
 * Precondition (checked): len[i] >= 1 and cum is the exclusive prefix sum
 * of len, for the first num_ranges[r] (clamped) entries of every request.
 */
int orc_slot_mapping_ranges(const int32_t *qsl, int32_t num_reqs, const int64_t *positions,
                            int64_t max_num_tokens, const int32_t *range_start,
                            const int32_t *range_len, const int32_t *range_cum,
                            const int32_t *num_ranges, int32_t range_stride, int32_t block_size,
                            int64_t *slot_mapping, uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (!qsl || num_reqs < 0 || max_num_tokens < 0 || block_size <= 0 || range_stride < 0 ||
        (max_num_tokens > 0 && !slot_mapping))
        return ORC_E_ARG;
    if (num_reqs > 0 && (!range_start || !range_len || !range_cum || !num_ranges))
        return ORC_E_ARG;
    if (!qsl_ok(qsl, num_reqs)) return ORC_E_QSL;

    /* descriptor precondition */
    for (int32_t r = 0; r < num_reqs; ++r) {
        uint32_t dummy = 0;
        int64_t n = clamp64(num_ranges[r], 0, range_stride, &dummy, ORC_FLAG_COUNT);
        int64_t expect_cum = 0;
        for (int64_t i = 0; i < n; ++i) {
            int64_t k = (int64_t)r * range_stride + i;
            if (range_len[k] < 1 || range_cum[k] != expect_cum) return ORC_E_RANGES;
            expect_cum += range_len[k];
        }
    }

    if (max_num_tokens == 0) return ORC_OK;
    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = ORC_PAD_ID;
    int64_t num_tokens = num_tokens_of(qsl, num_reqs, max_num_tokens, &flags);

    for (int32_t r = 0; r < num_reqs; ++r) {
        for (int64_t t = qsl[r]; t < qsl[r + 1] && t < num_tokens; ++t) {
            int64_t p = positions[t];
            if (p < 0) continue;
            int64_t n = clamp64(num_ranges[r], 0, range_stride, &flags, ORC_FLAG_COUNT);
            int64_t logical = p / block_size;
            int64_t offset = p % block_size;
            for (int64_t i = 0; i < n; ++i) {
                int64_t k = (int64_t)r * range_stride + i;
                int64_t cum = range_cum[k], len = range_len[k];
                if (cum <= logical && logical < cum + len) {
                    int64_t physical = (int64_t)range_start[k] + (logical - cum);
                    if (physical < 0) flags |= ORC_FLAG_BAD_BLOCK;
                    else slot_mapping[t] = physical * block_size + offset;
                    break;
                }
            }
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/*
 * Context-parallel slot mapping ([P2] "Entwurfsmotivation", DCP/PCP
 * interleaving: with context parallelism the kernel writes real slots only
 * for the positions of its own rank and the pad id for every other token;
 * [P3] "Symbol Map", the block_size row: context parallelism multiplies the
 * block size the attention groups see).  The pages name the three
 * parameters -- world size W, rank, interleave size I -- but not the
 * placement.  The reading taken is the plainest that fits both statements:
 *  - the W ranks deal a request's positions among themselves in chunks of I
 *    consecutive positions, round robin: position p is held by rank
 *    (p / I) % W;
 *  - a table entry names a virtual block of block_size*W positions, kept as
 *    one block of block_size slots on every rank under the same id, and each
 *    rank fills its block with its own positions in order.
 * For position p of this rank, with span = block_size*W and o = p % span:
 *   logical block = p / span,
 *   offset        = (o / (I*W)) * I + o % I   (this rank's positions before
 *                                              p in the virtual block),
 *   slot          = block_table[r][logical block] * block_size + offset.
 * A token of another rank is the pad id and reads nothing.  I must divide
 * block_size (so a rank's share of a virtual block is whole chunks and fits
 * its block); W = 1 is orc_slot_mapping_paged.  Other rules as there.
 * Parity unpinned as to the reading: the pages print no values for this
 * placement, so its pins check this code against a dealing simulation of the
 * same reading, not against the pages.
 */
static int cp_args_ok(int32_t block_size, int32_t world, int32_t rank, int32_t interleave)
{
    return world >= 1 && rank >= 0 && rank < world && interleave >= 1 &&
           block_size % interleave == 0;
}

int orc_slot_mapping_paged_cp(const int32_t *qsl, int32_t num_reqs, const int64_t *positions,
                              int64_t max_num_tokens, const int32_t *block_table,
                              int32_t table_stride, const int32_t *num_blocks_per_req,
                              int32_t block_size, int32_t cp_world_size, int32_t cp_rank,
                              int32_t cp_interleave_size, int64_t *slot_mapping,
                              uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (!qsl || num_reqs < 0 || max_num_tokens < 0 || block_size <= 0 || table_stride < 0 ||
        (max_num_tokens > 0 && !slot_mapping))
        return ORC_E_ARG;
    if (!cp_args_ok(block_size, cp_world_size, cp_rank, cp_interleave_size)) return ORC_E_ARG;
    if (!qsl_ok(qsl, num_reqs)) return ORC_E_QSL;

    if (max_num_tokens == 0) return ORC_OK;
    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = ORC_PAD_ID;
    int64_t num_tokens = num_tokens_of(qsl, num_reqs, max_num_tokens, &flags);
    int64_t W = cp_world_size, I = cp_interleave_size, span = (int64_t)block_size * W;

    for (int32_t r = 0; r < num_reqs; ++r) {
        for (int64_t t = qsl[r]; t < qsl[r + 1] && t < num_tokens; ++t) {
            int64_t p = positions[t];
            if (p < 0) continue;
            if ((p / I) % W != cp_rank) continue;      /* another rank's position */
            int64_t bound = table_stride;
            if (num_blocks_per_req)
                bound = clamp64(num_blocks_per_req[r], 0, table_stride, &flags, ORC_FLAG_COUNT);
            int64_t logical = p / span;
            int64_t o = p % span;
            int64_t offset = (o / (I * W)) * I + o % I;
            if (logical >= bound) continue;
            int64_t physical = block_table[(int64_t)r * table_stride + logical];
            if (physical < 0) { flags |= ORC_FLAG_BAD_BLOCK; continue; }
            slot_mapping[t] = physical * block_size + offset;
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/* The same placement through range descriptors (runs of virtual blocks);
 * W = 1 is orc_slot_mapping_ranges, whose precondition applies. */
int orc_slot_mapping_ranges_cp(const int32_t *qsl, int32_t num_reqs, const int64_t *positions,
                               int64_t max_num_tokens, const int32_t *range_start,
                               const int32_t *range_len, const int32_t *range_cum,
                               const int32_t *num_ranges, int32_t range_stride,
                               int32_t block_size, int32_t cp_world_size, int32_t cp_rank,
                               int32_t cp_interleave_size, int64_t *slot_mapping,
                               uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (!qsl || num_reqs < 0 || max_num_tokens < 0 || block_size <= 0 || range_stride < 0 ||
        (max_num_tokens > 0 && !slot_mapping))
        return ORC_E_ARG;
    if (num_reqs > 0 && (!range_start || !range_len || !range_cum || !num_ranges))
        return ORC_E_ARG;
    if (!cp_args_ok(block_size, cp_world_size, cp_rank, cp_interleave_size)) return ORC_E_ARG;
    if (!qsl_ok(qsl, num_reqs)) return ORC_E_QSL;
    for (int32_t r = 0; r < num_reqs; ++r) {
        uint32_t dummy = 0;
        int64_t n = clamp64(num_ranges[r], 0, range_stride, &dummy, ORC_FLAG_COUNT);
        int64_t expect_cum = 0;
        for (int64_t i = 0; i < n; ++i) {
            int64_t k = (int64_t)r * range_stride + i;
            if (range_len[k] < 1 || range_cum[k] != expect_cum) return ORC_E_RANGES;
            expect_cum += range_len[k];
        }
    }

    if (max_num_tokens == 0) return ORC_OK;
    for (int64_t t = 0; t < max_num_tokens; ++t) slot_mapping[t] = ORC_PAD_ID;
    int64_t num_tokens = num_tokens_of(qsl, num_reqs, max_num_tokens, &flags);
    int64_t W = cp_world_size, I = cp_interleave_size, span = (int64_t)block_size * W;

    for (int32_t r = 0; r < num_reqs; ++r) {
        for (int64_t t = qsl[r]; t < qsl[r + 1] && t < num_tokens; ++t) {
            int64_t p = positions[t];
            if (p < 0) continue;
            if ((p / I) % W != cp_rank) continue;      /* another rank's position */
            int64_t n = clamp64(num_ranges[r], 0, range_stride, &flags, ORC_FLAG_COUNT);
            int64_t logical = p / span;
            int64_t o = p % span;
            int64_t offset = (o / (I * W)) * I + o % I;
            for (int64_t i = 0; i < n; ++i) {
                int64_t k = (int64_t)r * range_stride + i;
                int64_t cum = range_cum[k], len = range_len[k];
                if (cum <= logical && logical < cum + len) {
                    int64_t physical = (int64_t)range_start[k] + (logical - cum);
                    if (physical < 0) flags |= ORC_FLAG_BAD_BLOCK;
                    else slot_mapping[t] = physical * block_size + offset;
                    break;
                }
            }
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/* Expansion factor of manager blocks into kernel blocks, or 0 when the
 * kernel block size does not divide the manager block size ([P2]
 * "Grenzen und Fehler": such a pair is rejected). */
static int64_t blocks_per_kv_block(int32_t block_size, int32_t kernel_block_size)
{
    if (block_size <= 0 || kernel_block_size <= 0) return 0;
    if (block_size % kernel_block_size != 0) return 0;
    return block_size / kernel_block_size;
}

/* A kernel block id b*k+j must stay a non-negative int32. */
static int expandable(int64_t id, int64_t k)
{
    return id >= 0 && id * k + (k - 1) <= INT32_MAX;
}

/*
 * Manager-to-kernel block expansion ([P2] "Entwurfsmotivation" and
 * "Schluesseldateien"; [P3] section 7): each manager block of a row becomes
 * k consecutive kernel blocks, k = block_size / kernel_block_size, in order:
 *   out[r][i*k + j] = in[r][i]*k + j,   0 <= j < k, i < count[r].
 * Entries of the output row past count[r]*k are block 0 (the null block).
 * counts may be NULL (every row full).  counts_out (may be NULL) receives
 * each row's kernel-block count, count[r]*k.
 */
int orc_map_to_kernel_blocks(const int32_t *ids, const int32_t *counts, int32_t rows,
                             int32_t in_stride, int32_t block_size, int32_t kernel_block_size,
                             int32_t *out, int32_t out_stride, int32_t *counts_out,
                             uint32_t *flags_out)
{
    uint32_t flags = 0;
    int64_t k = blocks_per_kv_block(block_size, kernel_block_size);
    if (k == 0) return ORC_E_ARG;
    if (rows < 0 || in_stride < 0 || out_stride < (int64_t)in_stride * k) return ORC_E_ARG;
    if (out_stride == 0) return ORC_OK;                /* empty rows: nothing is read */
    for (int32_t r = 0; r < rows; ++r) {
        int64_t count = in_stride;
        if (counts) count = clamp64(counts[r], 0, in_stride, &flags, ORC_FLAG_COUNT);
        for (int64_t c = 0; c < out_stride; ++c) out[(int64_t)r * out_stride + c] = 0;
        if (counts_out) counts_out[r] = (int32_t)(count * k);
        for (int64_t i = 0; i < count; ++i) {
            int64_t id = ids[(int64_t)r * in_stride + i];
            for (int64_t j = 0; j < k; ++j) {
                int64_t v = 0;
                if (expandable(id, k)) v = id * k + j;
                else flags |= ORC_FLAG_BAD_BLOCK;
                out[(int64_t)r * out_stride + i * k + j] = (int32_t)v;
            }
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/*
 * The same expansion applied to range descriptors: manager run
 * (start, len, cum) covers kernel blocks [start*k, (start+len)*k) and
 * logical kernel blocks [cum*k, (cum+len)*k), so all three fields scale by
 * k.  num_ranges is copied (clamped to the stride); entries past it are 0.
 */
int orc_map_ranges_to_kernel_blocks(const int32_t *start, const int32_t *len, const int32_t *cum,
                                    const int32_t *num_ranges, int32_t rows, int32_t range_stride,
                                    int32_t block_size, int32_t kernel_block_size,
                                    int32_t *out_start, int32_t *out_len, int32_t *out_cum,
                                    int32_t *out_num_ranges, uint32_t *flags_out)
{
    uint32_t flags = 0;
    int64_t k = blocks_per_kv_block(block_size, kernel_block_size);
    if (k == 0 || rows < 0 || range_stride < 0) return ORC_E_ARG;
    for (int32_t r = 0; r < rows; ++r) {
        int64_t n = clamp64(num_ranges[r], 0, range_stride, &flags, ORC_FLAG_COUNT);
        out_num_ranges[r] = (int32_t)n;
        for (int64_t i = 0; i < range_stride; ++i) {
            int64_t q = (int64_t)r * range_stride + i;
            int64_t s = 0, l = 0, c = 0;
            if (i < n) {
                if (expandable(start[q], k) && expandable(len[q], k) && expandable(cum[q], k)) {
                    s = (int64_t)start[q] * k;
                    l = (int64_t)len[q] * k;
                    c = (int64_t)cum[q] * k;
                } else {
                    flags |= ORC_FLAG_BAD_BLOCK;
                }
            }
            out_start[q] = (int32_t)s;
            out_len[q] = (int32_t)l;
            out_cum[q] = (int32_t)c;
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/*
 * Block table filled from range descriptors ([P1] "Status", GPU level: a
 * range-expansion kernel that writes the attention side's block table
 * straight from the range tables, in place of the per-step copy of a staged
 * table).  The row of a request is its runs laid end to end -- the same
 * relation that makes the range arithmetic and the gather give one slot
 * ([P1] "Measured Results", slot-mapping structural model) -- with the manager-to-kernel
 * expansion of [P3] section 7 applied on the way:
 *   run i (start, len) contributes blocks start, start+1, ..., start+len-1;
 *   block b contributes kernel blocks b*k, b*k+1, ..., b*k+k-1;
 *   out[r][q] = the q-th id of that list for q < min(length, out_stride),
 *   out[r][q] = 0 (the null block) for the rest of the row.
 * counts_out[r] (may be NULL) = min(length, out_stride); a list longer than
 * the row sets COUNT.  A stored entry whose block is negative or whose
 * kernel id does not fit an int32 is 0 and sets BAD_BLOCK (entries past
 * out_stride are not examined).
 * Precondition (checked): as for orc_slot_mapping_ranges.
 */
int orc_ranges_to_block_table(const int32_t *start, const int32_t *len, const int32_t *cum,
                              const int32_t *num_ranges, int32_t rows, int32_t range_stride,
                              int32_t block_size, int32_t kernel_block_size, int32_t *out,
                              int32_t out_stride, int32_t *counts_out, uint32_t *flags_out)
{
    uint32_t flags = 0;
    int64_t k = blocks_per_kv_block(block_size, kernel_block_size);
    if (k == 0 || rows < 0 || range_stride < 0 || out_stride < 0) return ORC_E_ARG;
    if (rows > 0 && (!num_ranges || (range_stride > 0 && (!start || !len || !cum)) ||
                     (out_stride > 0 && !out)))
        return ORC_E_ARG;

    for (int32_t r = 0; r < rows; ++r) {
        uint32_t dummy = 0;
        int64_t n = clamp64(num_ranges[r], 0, range_stride, &dummy, ORC_FLAG_COUNT);
        int64_t expect_cum = 0;
        for (int64_t i = 0; i < n; ++i) {
            int64_t q = (int64_t)r * range_stride + i;
            if (len[q] < 1 || cum[q] != expect_cum) return ORC_E_RANGES;
            expect_cum += len[q];
        }
    }

    for (int32_t r = 0; r < rows; ++r) {
        int32_t *row = out + (int64_t)r * out_stride;
        int64_t n = clamp64(num_ranges[r], 0, range_stride, &flags, ORC_FLAG_COUNT);
        for (int64_t q = 0; q < out_stride; ++q) row[q] = 0;
        int64_t length = 0; /* ids in the list so far */
        for (int64_t i = 0; i < n; ++i) {
            int64_t d = (int64_t)r * range_stride + i;
            for (int64_t b = start[d]; b < (int64_t)start[d] + len[d]; ++b) {
                for (int64_t j = 0; j < k; ++j) {
                    if (length >= out_stride) break; /* stored entries only */
                    if (expandable(b, k)) row[length] = (int32_t)(b * k + j);
                    else flags |= ORC_FLAG_BAD_BLOCK;
                    ++length;
                }
                if (length >= out_stride) break;
            }
        }
        int64_t full = 0; /* the whole list's length */
        for (int64_t i = 0; i < n; ++i) full += (int64_t)len[(int64_t)r * range_stride + i] * k;
        if (full > out_stride) flags |= ORC_FLAG_COUNT;
        if (counts_out) counts_out[r] = (int32_t)(full < out_stride ? full : out_stride);
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}

/* bf16 bit pattern -> double: the 16 bits are the high half of a float32, so
 * the widening is exact. */
static double bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* scale * (q . k) over one head's head_dim entries */
static double attention_score(const uint16_t *qh, const uint16_t *kr, int32_t head_dim,
                              double scale)
{
    double sc = 0.0;
    for (int32_t d = 0; d < head_dim; ++d) sc += bf16_value(qh[d]) * bf16_value(kr[d]);
    return sc * scale;
}

/*
 * Decode attention over the paged cache: the read path, where the attention
 * kernels resolve each position's block again ([P1] "The block-table access
 * pattern", block-table lookup per position; "The Direction", M7: range
 * arithmetic in the attention kernels).  The attention itself is the standard
 * scaled dot product, which the pages do not restate: for selected request
 * i (request id reqs[i]), its context slots slots[begin[i] .. begin[i+1]) (one
 * per position 0, 1, ..., in order; a slot < 0 holds no token and is skipped),
 * query head h and key/value head g = h / (num_q_heads / num_kv_heads):
 *   s_j = scale * sum_d q[reqs[i]][h][d] * K[slot_j][g][d]
 *   w_j = exp(s_j - max s) / sum_j' exp(s_j' - max s)
 *   out[i][h][d] = sum_j w_j * V[slot_j][g][d]
 * in double precision (bf16 inputs widened exactly); no token gives 0.
 * lse_out (may be NULL) receives, per selected request and query head, the
 * natural log of the softmax normalizer, log sum_j exp(s_j) = max s +
 * log sum_j exp(s_j - max s), or -inf with no token.  That is what merges
 * attention computed over disjoint sets of positions (for instance the
 * positions each context-parallel rank holds, [P2] "Entwurfsmotivation"):
 * with L = log sum_r exp(lse_r), out = sum_r exp(lse_r - L) out_r.
 * Cache rows: [cache_rows][num_kv_heads][head_dim] bf16.
 */
int orc_decode_attention(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         int64_t cache_rows, const int64_t *slots, const int64_t *begin,
                         const int32_t *reqs, int32_t num_sel, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, double scale, double *out,
                         double *lse_out)
{
    if (num_sel < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_heads % num_kv_heads != 0 || cache_rows < 0)
        return ORC_E_ARG;
    int64_t group = num_q_heads / num_kv_heads;
    for (int32_t i = 0; i < num_sel; ++i) {
        for (int64_t j = begin[i]; j < begin[i + 1]; ++j)
            if (slots[j] >= cache_rows) return ORC_E_ARG;
        for (int32_t h = 0; h < num_q_heads; ++h) {
            int64_t g = h / group;
            const uint16_t *qh = q + ((int64_t)reqs[i] * num_q_heads + h) * head_dim;
            double *o = out + ((int64_t)i * num_q_heads + h) * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
            if (lse_out) lse_out[(int64_t)i * num_q_heads + h] = -1.0 / 0.0;
            /* scores and their maximum */
            double smax = -1.0 / 0.0;
            int64_t n = 0;
            for (int64_t j = begin[i]; j < begin[i + 1]; ++j) {
                if (slots[j] < 0) continue;
                const uint16_t *kr = k_cache + (slots[j] * num_kv_heads + g) * head_dim;
                double sc = attention_score(qh, kr, head_dim, scale);
                if (sc > smax) smax = sc;
                ++n;
            }
            if (n == 0) continue;
            /* normalizer, then the weighted sum of value rows */
            double denom = 0.0;
            for (int64_t j = begin[i]; j < begin[i + 1]; ++j) {
                if (slots[j] < 0) continue;
                const uint16_t *kr = k_cache + (slots[j] * num_kv_heads + g) * head_dim;
                denom += exp(attention_score(qh, kr, head_dim, scale) - smax);
            }
            if (lse_out) lse_out[(int64_t)i * num_q_heads + h] = smax + log(denom);
            for (int64_t j = begin[i]; j < begin[i + 1]; ++j) {
                if (slots[j] < 0) continue;
                const uint16_t *kr = k_cache + (slots[j] * num_kv_heads + g) * head_dim;
                const uint16_t *vr = v_cache + (slots[j] * num_kv_heads + g) * head_dim;
                double w = exp(attention_score(qh, kr, head_dim, scale) - smax) / denom;
                for (int32_t d = 0; d < head_dim; ++d) o[d] += w * bf16_value(vr[d]);
            }
        }
    }
    return ORC_OK;
}

/*
 * Coordinate form ([P1] "The Coordinate Approach"):
 *   n(layer, block, token) = (layer * B + block) * T + token,
 *   offset = n * bytes_per_token,
 * B blocks per layer, T tokens per block.
 */
int64_t orc_coord_n(int64_t layer, int64_t block, int64_t token, int64_t num_blocks,
                    int64_t block_size)
{
    return (layer * num_blocks + block) * block_size + token;
}

int64_t orc_coord_offset(int64_t layer, int64_t block, int64_t token, int64_t num_blocks,
                         int64_t block_size, int64_t bytes_per_token)
{
    return orc_coord_n(layer, block, token, num_blocks, block_size) * bytes_per_token;
}

/*
 * K/V scatter through slot_mapping ([P2] "Verantwortung": the attention
 * side reads and writes the cache at each token's slot; [P3] section 8):
 * for every layer and every token t whose slot s is not the pad id,
 *   block = s / T, token-in-block = s % T,
 *   copy the token's K row to the K cache at the coordinate offset of
 *   (layer, block, token-in-block), and its V row likewise.
 * A slot at or past B*T is skipped and flagged.  Nothing else is written.
 *
 * The caller holds a window of the caches: rows [row_begin, row_begin +
 * row_count) of the [layers][B][T] row space (k_window/v_window point at
 * the window's first row), so caches larger than host memory can be
 * checked piecewise.  Rows outside the window are not touched.
 * Precondition (checked): no two tokens share a valid slot.
 */
static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* 1 when two tokens carry the same in-cache slot, -1 on allocation failure. */
static int has_duplicate_slot(const int64_t *slot_mapping, int64_t n, int64_t rows_per_layer)
{
    int64_t *v = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    int64_t m = 0;
    int dup = 0;
    if (!v) return -1;
    for (int64_t t = 0; t < n; ++t)
        if (slot_mapping[t] >= 0 && slot_mapping[t] < rows_per_layer) v[m++] = slot_mapping[t];
    qsort(v, (size_t)m, sizeof(int64_t), cmp_i64);
    for (int64_t i = 1; i < m; ++i)
        if (v[i] == v[i - 1]) { dup = 1; break; }
    free(v);
    return dup;
}

int orc_kv_write(const int64_t *slot_mapping, int64_t max_num_tokens, int32_t num_layers,
                 const uint8_t *key, const uint8_t *value, int64_t kv_layer_stride,
                 int64_t kv_token_stride, int64_t num_blocks, int32_t block_size,
                 int64_t bytes_per_token, uint8_t *k_window, uint8_t *v_window,
                 int64_t row_begin, int64_t row_count, uint32_t *flags_out)
{
    uint32_t flags = 0;
    if (max_num_tokens < 0 || num_layers < 0 || num_blocks < 0 || block_size <= 0 ||
        bytes_per_token <= 0 || row_begin < 0 || row_count < 0)
        return ORC_E_ARG;
    int64_t rows_per_layer = num_blocks * block_size;
    if (has_duplicate_slot(slot_mapping, max_num_tokens, rows_per_layer)) return ORC_E_DUPLICATE;
    for (int64_t layer = 0; layer < num_layers; ++layer) {
        for (int64_t t = 0; t < max_num_tokens; ++t) {
            int64_t s = slot_mapping[t];
            if (s < 0) continue;                         /* padded token: no write */
            if (s >= rows_per_layer) { flags |= ORC_FLAG_SLOT_OOB; continue; }
            int64_t block = s / block_size;
            int64_t token = s % block_size;
            int64_t n = orc_coord_n(layer, block, token, num_blocks, block_size);
            if (n < row_begin || n >= row_begin + row_count) continue;
            int64_t dst = (n - row_begin) * bytes_per_token;
            int64_t src = layer * kv_layer_stride + t * kv_token_stride;
            memcpy(k_window + dst, key + src, (size_t)bytes_per_token);
            memcpy(v_window + dst, value + src, (size_t)bytes_per_token);
        }
    }
    if (flags_out) *flags_out |= flags;
    return ORC_OK;
}
