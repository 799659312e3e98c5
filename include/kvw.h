/*
 * kvw.h -- paged KV-cache write path for AMD Instinct MI355X (gfx950).
 *
 * The write path turns every scheduled token's position into a physical
 * cache slot ("slot mapping") and copies the token's K and V rows into the
 * paged cache at that slot.  Sources (cited by page title and section):
 *
 *  [P1] "Range-addressed KV cache blocks for the vLLM serving engine":
 *       "The Innovation: Range Arithmetic Replaces the Per-Position Gather"
 *       (the two slot-mapping strategies, pad id for positions outside every
 *       range), "The Coordinate Approach" (cache coordinates) and "Status"
 *       (the block table filled from the range tables).
 *  [P2] "Blocktabelle: Abbildung von logischen Token auf physische
 *       KV-Blocks": "Verantwortung" (block table shape, slot_mapping),
 *       "Entwurfsmotivation" (manager/kernel block sizes, the slot-mapping
 *       kernel), "Datenfluss" (kernel arguments, tail padding for graph
 *       replay) and "Grenzen und Fehler" (rejected block-size pairs).
 *  [P3] "vLLM Block Table Management: From PagedAttention to the V1 KV Cache
 *       Stack": Deep Dive sections 7 (worker-side block table) and 8
 *       (slot_mapping: token -> physical slot).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller; the
 *    library allocates no memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Every call is asynchronous: it validates host-side scalars, enqueues
 *    its kernels on `stream` and returns.  No call synchronizes.
 *  - Launch shapes depend only on host scalars (max_num_tokens, row counts,
 *    strides, layer count), never on device data, so a call can be captured
 *    into a HIP graph once and replayed with new device contents.
 *  - Errors: a non-KVW_OK status means nothing was enqueued, except
 *    KVW_ERR_HIP after a failed launch; kvw_last_error() then describes it.
 *    Conditions that depend on device data are never synchronized on: the
 *    kernels clamp or skip as documented and OR a KVW_FLAG_* bit into
 *    `*err_flag` (a device int32, may be NULL; never cleared by the library).
 *  - Token ranges: request r owns tokens [query_start_loc[r],
 *    query_start_loc[r+1]); num_tokens = query_start_loc[num_reqs] is read on
 *    the device.  query_start_loc must be non-decreasing (not checked).
 *  - Pad id: KVW_PAD_ID (-1) marks a token without a slot: tokens at or past
 *    num_tokens, tokens of no request, negative positions, positions past
 *    the blocks a request owns ([P3] section 8; [P2] "Datenfluss"), and
 *    with context parallelism the positions another rank holds.
 *  - Context parallelism ([P2] "Entwurfsmotivation": the slot-mapping kernel
 *    of a context-parallel rank gives real slots only to that rank's
 *    positions; [P3] "Symbol Map": context parallelism multiplies the block
 *    size the attention groups see).  The slot-mapping calls and the fused
 *    write take cp_world_size W, cp_rank and cp_interleave_size I.  The ranks
 *    deal a request's positions in chunks of I consecutive positions, round
 *    robin (position p is held by rank (p / I) % W); a block-table entry, or
 *    a run's block, names a virtual block of block_size*W positions, stored as
 *    one block of block_size slots on every rank under the same id, each rank
 *    filling it with its own positions in order.  For p held by this rank,
 *    with o = p % (block_size*W):
 *      lb   = p / (block_size*W),
 *      slot = block(lb) * block_size + (o / (I*W)) * I + o % I;
 *    every other token gets KVW_PAD_ID and reads no table entry or run.
 *    W = 0 or 1 is the plain mapping.  For W >= 1: 0 <= cp_rank < W,
 *    I >= 1 divides block_size, block_size*W <= INT32_MAX, else
 *    KVW_ERR_INVALID_ARG.  The pages give the three parameters but not the
 *    placement: this is the plainest placement with both properties.
 */
#ifndef KVW_H
#define KVW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVW_ABI_VERSION 7
#define KVW_PAD_ID (-1)
/* Largest accepted range_stride (range descriptors per request). */
#define KVW_MAX_RANGE_STRIDE 65536

typedef enum kvw_status {
    KVW_OK = 0,
    KVW_ERR_INVALID_ARG = 1, /* a host-side argument is out of its domain */
    KVW_ERR_UNSUPPORTED = 2, /* a well-formed request the library does not support */
    KVW_ERR_RANGE_CAP = 3,   /* range_stride above KVW_MAX_RANGE_STRIDE */
    KVW_ERR_HIP = 4,         /* the HIP runtime reported an error */
    KVW_ERR_NO_SPACE = 5,    /* allocator: not enough blocks even after eviction */
    KVW_ERR_NOT_FOUND = 6    /* allocator: no prefix-cache entry under the key */
} kvw_status;

/* Sticky bits OR-ed into *err_flag by the kernels. */
#define KVW_FLAG_NUM_TOKENS 1 /* query_start_loc[num_reqs] outside [0, max_num_tokens]; clamped */
#define KVW_FLAG_COUNT 2      /* a per-request block or range count outside [0, stride]; clamped */
#define KVW_FLAG_BAD_BLOCK 4  /* a resolved physical block id is negative (token gets the pad id),
                                 or an id cannot be expanded within int32 (written as block 0) */
#define KVW_FLAG_SLOT_OOB 8   /* a slot at or past num_blocks*block_size: its write is skipped */

/* Slot sources of kvw_kv_write. */
#define KVW_SLOTS_PRECOMPUTED 0 /* read slot_mapping_in */
#define KVW_SLOTS_PAGED 1       /* resolve through the block table (fused) */
#define KVW_SLOTS_RANGES 2      /* resolve through range descriptors (fused) */

/* Kernel schedules of kvw_kv_write in the paged and range modes. */
#define KVW_SCHEDULE_AUTO 0        /* two kernels for large writes when slot_mapping_out is set */
#define KVW_SCHEDULE_TWO_KERNELS 1 /* slot mapping kernel, then the scatter (needs slot_mapping_out) */
#define KVW_SCHEDULE_ONE_KERNEL 2  /* one kernel resolves each token's slot and copies its rows */
/* AUTO picks two kernels from this many token rows (max_num_tokens * num_layers) up. */
#define KVW_TWO_KERNEL_MIN_ROWS 65536

/* KVW_ABI_VERSION of the loaded library. */
int32_t kvw_abi_version(void);

/* Message for the last non-KVW_OK status returned on the calling thread. */
const char *kvw_last_error(void);

/*
 * Paged slot mapping ([P2] "Entwurfsmotivation" and "Datenfluss"; [P3]
 * section 8).  For token t < num_tokens of request r at position p >= 0:
 *   lb = p / block_size, off = p % block_size,
 *   slot_mapping[t] = block_table[r][lb] * block_size + off
 * when lb < num_blocks_per_req[r] (or lb < block_table_stride when
 * num_blocks_per_req is NULL), else KVW_PAD_ID.  Every t in
 * [num_tokens, max_num_tokens) is KVW_PAD_ID.
 *
 *   query_start_loc    int32[num_reqs + 1]
 *   positions          int64[max_num_tokens], all of it readable; entries
 *                      past num_tokens are ignored
 *   block_table        int32[max_num_reqs][block_table_stride], row-major;
 *                      row r holds request r's physical block ids in
 *                      logical order
 *   num_blocks_per_req int32[max_num_reqs] or NULL
 *   slot_mapping       int64[max_num_tokens] (output)
 * Flags: KVW_FLAG_NUM_TOKENS, KVW_FLAG_COUNT, KVW_FLAG_BAD_BLOCK.
 * Errors: KVW_ERR_INVALID_ARG for NULL required pointers, misaligned
 * pointers, negative sizes, block_size <= 0 or max_num_tokens >= 2^31.
 */
kvw_status kvw_slot_mapping_paged(const int32_t *query_start_loc, int32_t num_reqs,
                                  const int64_t *positions, int64_t max_num_tokens,
                                  const int32_t *block_table, int32_t block_table_stride,
                                  const int32_t *num_blocks_per_req, int32_t block_size,
                                  int32_t cp_world_size, int32_t cp_rank,
                                  int32_t cp_interleave_size, int64_t *slot_mapping,
                                  int32_t *err_flag, void *stream);

/*
 * Range-arithmetic slot mapping ([P1] "The Innovation").  Request r owns
 * num_ranges[r] contiguous runs; run i starts at physical block
 * range_start[r][i], spans range_len[r][i] blocks and covers the logical
 * blocks [range_cum[r][i], range_cum[r][i] + range_len[r][i]).  For token t
 * of request r at position p >= 0 with lb = p / block_size:
 *   slot_mapping[t] = (range_start[r][i] + lb - range_cum[r][i]) * block_size
 *                     + p % block_size
 * for the run i containing lb, else KVW_PAD_ID; the tail is padded as in
 * kvw_slot_mapping_paged.  Precondition (not checked on the device):
 * range_len >= 1 and range_cum is the exclusive prefix sum of range_len
 * within each request.  Given the same physical layout, the result equals
 * kvw_slot_mapping_paged through the materialized table.
 *
 *   range_start, range_len, range_cum  int32[max_num_reqs][range_stride]
 *   num_ranges                         int32[max_num_reqs]
 * Flags: KVW_FLAG_NUM_TOKENS, KVW_FLAG_COUNT (num_ranges clamped to
 * [0, range_stride]), KVW_FLAG_BAD_BLOCK.
 * Errors: as kvw_slot_mapping_paged, plus KVW_ERR_RANGE_CAP when
 * range_stride > KVW_MAX_RANGE_STRIDE.
 */
kvw_status kvw_slot_mapping_ranges(const int32_t *query_start_loc, int32_t num_reqs,
                                   const int64_t *positions, int64_t max_num_tokens,
                                   const int32_t *range_start, const int32_t *range_len,
                                   const int32_t *range_cum, const int32_t *num_ranges,
                                   int32_t range_stride, int32_t block_size,
                                   int32_t cp_world_size, int32_t cp_rank,
                                   int32_t cp_interleave_size, int64_t *slot_mapping,
                                   int32_t *err_flag, void *stream);

/*
 * Manager-to-kernel block expansion ([P2] "Entwurfsmotivation" and
 * "Grenzen und Fehler"; [P3] section 7).  With k = block_size /
 * kernel_block_size, each manager block b becomes kernel blocks
 * b*k .. b*k+k-1 (the same memory at the finer block size):
 *   out[r][i*k + j] = ids[r][i] * k + j   for i < counts[r], j < k,
 *   out[r][c] = 0 (the null block)         for c >= counts[r] * k.
 *   ids    int32[rows][in_stride]; counts int32[rows] or NULL (full rows)
 *   out    int32[rows][out_stride] (output), out_stride >= in_stride * k
 * Flags: KVW_FLAG_COUNT, KVW_FLAG_BAD_BLOCK (id < 0 or id*k+k-1 > INT32_MAX:
 * written as 0).
 * Errors: KVW_ERR_INVALID_ARG when kernel_block_size does not divide
 * block_size (or either is <= 0), or out_stride < in_stride * k.
 */
kvw_status kvw_map_to_kernel_blocks(const int32_t *ids, const int32_t *counts, int32_t rows,
                                    int32_t in_stride, int32_t block_size,
                                    int32_t kernel_block_size, int32_t *out, int32_t out_stride,
                                    int32_t *err_flag, void *stream);

/*
 * The same expansion for range descriptors: a manager run (start, len,
 * cum) is the kernel run (start*k, len*k, cum*k).  out_num_ranges[r] =
 * num_ranges[r] clamped to [0, range_stride]; descriptor entries past it
 * are written 0.  All arrays are [rows][range_stride] (num_ranges: [rows]).
 * Flags and errors as kvw_map_to_kernel_blocks (plus KVW_ERR_RANGE_CAP).
 */
kvw_status kvw_map_ranges_to_kernel_blocks(const int32_t *range_start, const int32_t *range_len,
                                           const int32_t *range_cum, const int32_t *num_ranges,
                                           int32_t rows, int32_t range_stride, int32_t block_size,
                                           int32_t kernel_block_size, int32_t *out_start,
                                           int32_t *out_len, int32_t *out_cum,
                                           int32_t *out_num_ranges, int32_t *err_flag,
                                           void *stream);

/*
 * The attention side's block table filled straight from the range
 * descriptors, with no staged table to copy ([P1] "Status": the
 * range-expansion kernel in place of the per-step materialization copy).
 * A row is its request's runs laid end to end, each manager block b
 * expanded to kernel blocks b*k .. b*k+k-1 (k = block_size /
 * kernel_block_size; k = 1 gives the table at the manager block size):
 *   block_table[r][q] = (start[i] + q/k - cum[i]) * k + q%k
 *                       for the run i with cum[i] <= q/k < cum[i] + len[i],
 *   block_table[r][q] = 0 (the null block) past the last run.
 *   num_blocks_per_req[r] = min((cum[n-1] + len[n-1]) * k, block_table_stride),
 *                       n = num_ranges[r] clamped (0 when n = 0).
 * With the same descriptors, kvw_slot_mapping_paged on this table (and
 * count) gives the slots kvw_slot_mapping_ranges gives at the manager block
 * size, and kvw_slot_mapping_paged at kernel_block_size does too.
 *   range_start, range_len, range_cum  int32[rows][range_stride] (input, as
 *                                      kvw_slot_mapping_ranges, manager units)
 *   num_ranges                         int32[rows] (input)
 *   block_table                        int32[rows][block_table_stride] (output,
 *                                      every entry written)
 *   num_blocks_per_req                 int32[rows] (output) or NULL
 * Flags: KVW_FLAG_COUNT (num_ranges outside [0, range_stride], or more
 * kernel blocks than block_table_stride: the row keeps the first ones),
 * KVW_FLAG_BAD_BLOCK (a stored entry whose block is negative or whose
 * kernel id exceeds INT32_MAX: written as 0).
 * Errors: KVW_ERR_INVALID_ARG when kernel_block_size does not divide
 * block_size (or either is <= 0), for negative sizes, NULL or misaligned
 * required arrays; KVW_ERR_RANGE_CAP when range_stride >
 * KVW_MAX_RANGE_STRIDE.  Under the descriptor precondition of
 * kvw_slot_mapping_ranges; inputs that break it give in-bounds but
 * unspecified table contents.
 */
kvw_status kvw_ranges_to_block_table(const int32_t *range_start, const int32_t *range_len,
                                     const int32_t *range_cum, const int32_t *num_ranges,
                                     int32_t rows, int32_t range_stride, int32_t block_size,
                                     int32_t kernel_block_size, int32_t *block_table,
                                     int32_t block_table_stride, int32_t *num_blocks_per_req,
                                     int32_t *err_flag, void *stream);

/*
 * Arguments of kvw_kv_write.  Byte strides; every pointer of key, value,
 * k_cache, v_cache and every stride must be a multiple of 16.
 */
typedef struct kvw_kv_write_args {
    int32_t mode;                      /* KVW_SLOTS_* */
    int32_t num_reqs;                  /* PAGED/RANGES */
    const int32_t *query_start_loc;    /* PAGED/RANGES: int32[num_reqs + 1] */
    const int64_t *positions;          /* PAGED/RANGES: int64[max_num_tokens] */
    int64_t max_num_tokens;            /* token rows of key/value and slot mappings */
    const int64_t *slot_mapping_in;    /* PRECOMPUTED: int64[max_num_tokens] */
    int64_t *slot_mapping_out;         /* PAGED/RANGES: int64[max_num_tokens] or NULL */
    const int32_t *block_table;        /* PAGED: as kvw_slot_mapping_paged */
    const int32_t *num_blocks_per_req; /* PAGED: or NULL */
    int32_t block_table_stride;        /* PAGED */
    int32_t range_stride;              /* RANGES */
    const int32_t *range_start;        /* RANGES: as kvw_slot_mapping_ranges */
    const int32_t *range_len;
    const int32_t *range_cum;
    const int32_t *num_ranges;
    int32_t block_size;                /* T: token slots per cache block */
    int32_t num_layers;                /* L */
    int64_t num_blocks;                /* B: cache blocks per layer */
    const void *key;                   /* row of token t, layer l at key + l*kv_layer_stride
                                          + t*kv_token_stride, bytes_per_token bytes */
    const void *value;                 /* same layout as key */
    int64_t kv_layer_stride;
    int64_t kv_token_stride;
    void *k_cache;                     /* [L][B][T] rows of bytes_per_token bytes */
    void *v_cache;                     /* same layout as k_cache */
    int64_t bytes_per_token;           /* multiple of 16, below 2^31 */
    int32_t *err_flag;                 /* device int32 or NULL */
    int32_t schedule;                  /* KVW_SCHEDULE_*; ignored in the precomputed mode */
    int32_t cp_world_size;             /* PAGED/RANGES: context parallelism (0 = none); the */
    int32_t cp_rank;                   /* cache holds this rank's blocks of block_size slots */
    int32_t cp_interleave_size;
    /* PAGED/RANGES, optional: the attention side's block table for the same
     * step, at table_block_size (which divides block_size; k = block_size /
     * table_block_size).  PAGED: block_table expanded as kvw_map_to_kernel_blocks
     * does; RANGES: filled from the runs as kvw_ranges_to_block_table does.
     * Rows: num_reqs.  table_counts_out (or NULL) receives each row's kernel-block
     * count.  With the two-kernel schedule the table is written by the same
     * launch as the slot mapping (one launch fewer than a separate call); with
     * one kernel, by a launch before it; with max_num_tokens == 0, alone. */
    int32_t *table_out;                /* int32[num_reqs][table_out_stride] or NULL */
    int32_t *table_counts_out;         /* int32[num_reqs] or NULL */
    int32_t table_out_stride;          /* > 0; PAGED: >= block_table_stride * k */
    int32_t table_block_size;
} kvw_kv_write_args;

/* sizeof(kvw_kv_write_args) as compiled into the library. */
size_t kvw_kv_write_args_size(void);

/*
 * K/V scatter through the slot mapping, optionally fused with it ([P2]
 * "Verantwortung": attention writes each token's KV at its slot; [P1] "The
 * Coordinate Approach": coordinates n(layer, block, token) =
 * (layer*B + block)*T + token, byte offset n*bytes_per_token).
 * For every layer l < L and token t < max_num_tokens whose slot s (read
 * from slot_mapping_in, or resolved as in kvw_slot_mapping_paged /
 * kvw_slot_mapping_ranges) satisfies 0 <= s < B*T:
 *   k_cache + n*bytes_per_token <- key row (l, t),  v_cache likewise,
 *   with n = (l*B + s/T)*T + s%T.
 * A slot >= B*T is skipped (KVW_FLAG_SLOT_OOB); the pad id writes nothing.
 * No other cache byte is touched.  In the fused modes the slots are also
 * stored to slot_mapping_out when it is non-NULL (tail padded).
 * Precondition: no two tokens share a slot (else the surviving row is
 * unspecified).
 * Execution: the precomputed mode enqueues one scatter kernel.  In the
 * paged and range modes the call enqueues either two kernels on `stream`
 * (the slot mapping, written to slot_mapping_out, then the scatter that
 * reads it) or one kernel that resolves each token's slot and copies its
 * rows (and stores slot_mapping_out if set).  KVW_SCHEDULE_AUTO takes two
 * kernels when slot_mapping_out is set and max_num_tokens * num_layers >=
 * KVW_TWO_KERNEL_MIN_ROWS (measured crossover on MI355X), one otherwise.
 * Results are identical either way.  Cost: without slot_mapping_out a large
 * write always takes one kernel, which is slower than two on fragmented caches
 * and long multi-layer writes (and 1-2% faster on contiguous ones).  Measured
 * on MI355X: 131,072 tokens of 2 KiB rows, every 32-slot block its own run,
 * one kernel at 73-74% of 8 TB/s (paged and ranges) against 77-78% for two
 * kernels; 16,384 tokens x 32 layers, 77-79% against 81-82%.  Callers that
 * write large fragmented batches should keep the slot mapping (the attention
 * side needs it anyway).
 * Errors: KVW_ERR_INVALID_ARG for an unknown mode or schedule,
 * KVW_SCHEDULE_TWO_KERNELS without slot_mapping_out, NULL required
 * pointers, misalignment, negative sizes, bytes_per_token % 16 != 0 or
 * >= 2^31, or a cache size beyond int64; KVW_ERR_RANGE_CAP as
 * kvw_slot_mapping_ranges.
 */
kvw_status kvw_kv_write(const kvw_kv_write_args *args, void *stream);

/*
 * Decode attention over the paged cache: the read path, where each position's
 * block is resolved again ([P1] "The block-table access pattern"; "The
 * Direction", M7: range arithmetic in the attention kernels).  One query token
 * per request; request r attends its positions 0 .. context_lens[r]-1, whose
 * slots follow the slot-mapping definitions above (PAGED: block table; RANGES:
 * range descriptors); a position without a block (pad id) is skipped.  For
 * query head h and key/value head g = h / (num_q_heads / num_kv_heads):
 *   out[r][h] = sum_j softmax_j(scale * q[r][h] . K[slot_j][g]) * V[slot_j][g]
 * computed in fp32 from bf16 inputs; no position gives 0.  Each workgroup
 * takes a chunk of chunk_positions positions of one request, resolves their
 * slots once into LDS for all heads and folds them into a running softmax;
 * the chunks are combined in a second launch through `workspace`.  For 32
 * requests or more, a first launch lists the chunks that hold positions in
 * `workspace` (full chunks first, then the partial ones longest first); the
 * order affects only the schedule, not the result.
 *   q                  bf16 [num_reqs][num_q_heads][head_dim], 16-byte aligned
 *   context_lens       int32 [num_reqs] (device); clamped to [0, max_context]
 *                      with KVW_FLAG_COUNT
 *   max_context        host bound on the context lengths; sets the grid, so a
 *                      graph captured once serves any lengths up to it
 *   k_cache, v_cache   bf16 [num_blocks * block_size][num_kv_heads][head_dim]
 *                      (one layer, the K/V write's layout), 16-byte aligned
 *   out                fp32 [num_reqs][num_q_heads][head_dim]
 *   workspace          device memory of kvw_decode_workspace_size(...) bytes, owned by
 *                      the caller; its contents need no initialisation and are
 *                      overwritten; calls that overlap on one workspace race
 *   chunk_positions    positions per workgroup: 256, 512, 1024 or 2048; 0 picks the
 *                      longest that gives num_reqs * ceil(max_context / chunk) >= 256
 *                      workgroups (at most 1024 for 32 requests or more); results
 *                      differ only in rounding
 *   cp_world_size, cp_rank, cp_interleave_size
 *                      decode context parallelism ([P2] "Entwurfsmotivation"; the
 *                      placement of kvw_slot_mapping_paged): this rank attends only
 *                      the positions it holds, from its own cache of block_size slots
 *                      per block; the others are skipped without a flag.  0 or 1 = none.
 *                      KVW_ERR_INVALID_ARG as kvw_slot_mapping_paged
 *   lse_out            NULL, or fp32 [num_reqs][num_q_heads]: log sum_j exp(s_j) over
 *                      the positions attended (natural log; -inf with none), what
 *                      kvw_decode_merge needs to combine the ranks' results
 * Supported: head_dim 128; num_q_heads / num_kv_heads G in {1, 2, 4, 8};
 * num_kv_heads 1..16, or 1..8 when G = 8 (so up to 64 query heads); else
 * KVW_ERR_UNSUPPORTED.  Flags: KVW_FLAG_COUNT,
 * KVW_FLAG_BAD_BLOCK, KVW_FLAG_SLOT_OOB (slot past the cache: skipped).
 */
typedef struct kvw_decode_args {
    int32_t mode;                      /* KVW_SLOTS_PAGED or KVW_SLOTS_RANGES */
    int32_t num_reqs;
    const void *q;
    const int32_t *context_lens;
    int32_t max_context;
    int32_t block_size;
    const int32_t *block_table;        /* PAGED: as kvw_slot_mapping_paged */
    const int32_t *num_blocks_per_req; /* PAGED: or NULL */
    int32_t block_table_stride;
    int32_t range_stride;              /* RANGES: as kvw_slot_mapping_ranges */
    const int32_t *range_start;
    const int32_t *range_len;
    const int32_t *range_cum;
    const int32_t *num_ranges;
    const void *k_cache;
    const void *v_cache;
    int64_t num_blocks;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    float scale;                       /* e.g. 1 / sqrt(head_dim) */
    float *out;
    void *workspace;
    int64_t workspace_bytes;
    int32_t *err_flag;
    int32_t chunk_positions;           /* 256, 512, 1024, 2048, or 0 (chosen by the library) */
    int32_t cp_world_size;             /* context parallelism: 0 or 1 = none */
    int32_t cp_rank;
    int32_t cp_interleave_size;
    float *lse_out;                    /* NULL or fp32 [num_reqs][num_q_heads] */
} kvw_decode_args;

/* Bytes of workspace kvw_decode_attention needs for these sizes. */
int64_t kvw_decode_workspace_size(int32_t num_reqs, int32_t max_context, int32_t num_q_heads,
                                  int32_t head_dim);

/* Size of kvw_decode_args as compiled into the library (binding check). */
size_t kvw_decode_args_size(void);

kvw_status kvw_decode_attention(const kvw_decode_args *args, void *stream);

/* Bytes of the static workspace of kvw_decode_attention_noalloc, on each GPU. */
#define KVW_DECODE_STATIC_WORKSPACE_BYTES (64LL << 20)

/*
 * kvw_decode_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same operation, kernels and results; the chunk workspace is
 * a static device array of KVW_DECODE_STATIC_WORKSPACE_BYTES that the library
 * holds on each GPU it runs on until the process ends, and args->workspace and
 * args->workspace_bytes are ignored.  The call allocates nothing: its first
 * call on a GPU looks that GPU's array up (hipGetSymbolAddress, the GPU made
 * current for the lookup).  The workspace this call needs, with chunk the
 * chunk length used (chunk_positions, or the library's choice) and
 * U = num_reqs * ceil(max_context / chunk), is
 *   U * num_q_heads * (head_dim + 2) * 4 bytes, plus U * 8 + 4 for 32 or more requests;
 * above KVW_DECODE_STATIC_WORKSPACE_BYTES the call fails with
 * KVW_ERR_UNSUPPORTED before anything is enqueued (e.g. 256 requests of up to
 * 8192 positions with 32 query heads need 34 MB at the library's chunk of
 * 1024; 16 requests of 131,072 positions, 17 MB).  Every call on a GPU uses
 * that GPU's one array and leaves its contents behind (no call needs them
 * cleared): calls in stream order are safe, calls that overlap on one GPU
 * (other streams, other threads) race.
 * Errors: as kvw_decode_attention; KVW_ERR_HIP if the lookup fails.
 */
kvw_status kvw_decode_attention_noalloc(const kvw_decode_args *args, void *stream);

/*
 * Merges decode attention computed over disjoint sets of each request's
 * positions, for instance by the ranks of decode context parallelism: with
 * L = log sum_p exp(lse_p),
 *   out[r][h][d] = sum_p exp(lse_p[r][h] - L) * outs_p[r][h][d],  lse_out = L.
 * A part with lse -inf (no position) adds nothing; none with a position gives
 * out 0 and lse -inf.
 *   outs      fp32 [num_parts][num_reqs][num_q_heads][head_dim] (device), the
 *             parts' kvw_decode_attention outputs stacked
 *   lses      fp32 [num_parts][num_reqs][num_q_heads] (device), their lse_out
 *   out       fp32 [num_reqs][num_q_heads][head_dim]; lse_out NULL or fp32
 *             [num_reqs][num_q_heads]
 * Errors: KVW_ERR_INVALID_ARG for num_parts < 1, head_dim outside 1..1024,
 * num_reqs or num_q_heads outside their ranges, NULL or misaligned pointers.
 */
kvw_status kvw_decode_merge(int32_t num_parts, int32_t num_reqs, int32_t num_q_heads,
                            int32_t head_dim, const float *outs, const float *lses, float *out,
                            float *lse_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVW_H */
