// Paged KV-cache write path for MI355X (gfx950, CDNA4, wave64).
//
// Kernels:
//   slot_mapping_kernel<MODE>    one token per lane: paged gather or range
//                                arithmetic, tail padded with the pad id;
//   kv_scatter_kernel<TPW>       one 1 KiB slice of one K or V row per wave
//                                (of TPW consecutive tokens under context
//                                parallelism), slot read from a slot mapping;
//   kv_scatter_small_kernel      rows under 1 KiB: one plane of several
//                                consecutive tokens per wave;
//   kv_write_fused_kernel<MODE>  one wave per token and plane: slot resolution
//                                and the copy of the token's row in one pass;
//   expand_blocks_kernel,
//   expand_ranges_kernel         manager-to-kernel block expansion;
//   fill_table_kernel            the attention side's block table filled
//                                straight from the range descriptors.
// kvw_kv_write in a fused mode runs slot_mapping_kernel then
// kv_scatter_kernel for large writes whose slot mapping the caller keeps
// (the usual case: attention consumes it), and kv_write_fused_kernel
// otherwise (small writes pay less for one launch than for two).  The host
// functions at the bottom validate host-side scalars and launch on the
// caller's stream; include/kvw.h holds the contract.
//
// Sources: "Range-addressed KV cache blocks for the vLLM serving engine"
// ("The Innovation", "The Coordinate Approach", and "Status" on filling the
// block table from the range tables); "Blocktabelle: Abbildung von logischen
// Token auf physische KV-Blocks" ("Entwurfsmotivation", "Datenfluss",
// "Grenzen und Fehler"); "vLLM Block Table Management"
// (Deep Dive sections 7 and 8).
//
// The path is a memory-bound gather/scatter: no matrix cores are involved.
// Measured on MI355X, HBM throughput of a copy is highest when every wave
// moves a single 1 KiB span (one 16-byte load and one 16-byte store per
// lane) and retires: larger per-wave batches, loops and persistent grids
// all lose 5-30%.  A copy wave therefore cannot afford a dependent chain of
// metadata loads, which is why the scatter reads ready-made slots and the
// slot resolution runs one token per lane in its own kernel.  All cache
// addressing is 64-bit: a 32-layer cache plane reaches 32 GiB.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "kvw.h"
#include "kvw_device.h"
#include "kvw_error.h"

#ifndef KVW_SCATTER_WAVES
#define KVW_SCATTER_WAVES 1
#endif
#ifndef KVW_FUSED_WAVES
#define KVW_FUSED_WAVES 1
#endif
#ifndef KVW_NT_LOADS
#define KVW_NT_LOADS 1
#endif

#ifndef KVW_NT_STORES
#define KVW_NT_STORES 1
#endif
#ifndef KVW_TOKEN_WAVE_MAX_ROWS
#define KVW_TOKEN_WAVE_MAX_ROWS 8192
#endif

namespace {

constexpr int kBlockThreads = 256;           // expansion and table-fill kernels
constexpr int kSlotThreads = kWave;          // slot-mapping launch (both roles): one wave per workgroup
constexpr int kSliceBytes = kWave * 16;      // one wave-wide 16-byte access
constexpr int kScatterWaves = KVW_SCATTER_WAVES;
constexpr int kScatterThreads = kScatterWaves * kWave;
constexpr int kFusedWaves = KVW_FUSED_WAVES;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kMaxSlicesPerLane = 4;         // rows up to 4 KiB are held in registers whole
constexpr unsigned kMaxGridX = 0x7fffffffu;
constexpr unsigned kMaxGridY = 65535u;

enum : int { kPrecomputed = KVW_SLOTS_PRECOMPUTED, kPaged = KVW_SLOTS_PAGED, kRanges = KVW_SLOTS_RANGES };


// Everything the slot resolution reads.
struct MapArgs {
    const int32_t *qsl;
    const int64_t *positions;
    const int32_t *block_table;
    const int32_t *num_blocks_per_req;
    const int32_t *range_start;
    const int32_t *range_len;
    const int32_t *range_cum;
    const int32_t *num_ranges;
    int64_t *slots_out;
    int32_t *err_flag;
    int64_t max_num_tokens;
    int32_t num_reqs;
    int32_t table_stride;
    int32_t range_stride;
    int32_t block_size;
    int32_t cp_world;       // context-parallel ranks (<= 1: none)
    int32_t cp_rank;
    int32_t cp_interleave;  // positions per dealt chunk; divides block_size
    // Optional attention-side block table, written by extra workgroups of the
    // slot-mapping launch (blockIdx.x >= slot_blocks): the block table expanded
    // (paged) or filled from the runs (ranges) at table_k kernel blocks per block.
    int32_t *table_out;
    int32_t *table_counts_out;
    int32_t table_out_stride;
    int32_t table_k;
    uint32_t slot_blocks;           // workgroups of the slot-mapping role
    uint32_t table_blocks_per_row;  // ranges: workgroups per table row
};

// Everything the K/V copy touches.
struct CopyArgs {
    const uint8_t *key;
    const uint8_t *value;
    uint8_t *k_cache;
    uint8_t *v_cache;
    int64_t kv_layer_stride;
    int64_t kv_token_stride;
    int64_t rows_per_layer;   // B * T
    int64_t bytes_per_token;
    int64_t max_num_tokens;
    int32_t num_layers;
    int32_t layers_per_wave;  // fused kernel: layers handled by one wave
    uint32_t slices_per_row;  // ceil(bytes_per_token / 1 KiB)
    uint32_t items_per_token; // 2 planes x slices_per_row
    int32_t items_log2;       // log2(items_per_token), or -1 if not a power of two
    uint32_t lanes_per_row;   // rows under 1 KiB: bytes_per_token / 16 lanes per row
    uint32_t rows_per_wave;   // rows under 1 KiB: 64 / lanes_per_row tokens per wave
};


// num_tokens = query_start_loc[num_reqs], clamped to [0, max_num_tokens]; a
// clamp sets KVW_FLAG_NUM_TOKENS in `flags`.  Flags are collected in
// registers and raised after the metadata loads, so that no store precedes
// those loads (they may then be scalar loads for a wave-uniform token).
__device__ __forceinline__ int64_t device_num_tokens(const MapArgs &a, uint32_t &flags)
{
    // one uniform word: read through the constant address space, so it is a scalar
    // load that does not queue behind the wave's vector loads
    int64_t n = reinterpret_cast<const __attribute__((address_space(4))) int32_t *>(
        reinterpret_cast<uintptr_t>(a.qsl))[a.num_reqs];
    if (n < 0) { n = 0; flags |= KVW_FLAG_NUM_TOKENS; }
    if (n > a.max_num_tokens) { n = a.max_num_tokens; flags |= KVW_FLAG_NUM_TOKENS; }
    return n;
}

// Logical block and in-block offset of position p on this rank (cp_locate).
__device__ __forceinline__ bool locate(const MapArgs &a, int64_t p, int64_t &lb, int32_t &off)
{
    return cp_locate(p, a.block_size, a.cp_world, a.cp_rank, a.cp_interleave, lb, off);
}

// Paged gather: one table load per position (wave-uniform: scalar loads).  The
// entry and the row's count go out together, both unconditional at valid
// addresses (the entry at a clamped index; without counts the "count" re-reads
// the entry and is ignored), so the two cost one memory latency: a load under
// the branch on the count pointer would go out only after the entry arrived.
__device__ __forceinline__ int64_t paged_block(const MapArgs &a, int32_t r, int64_t lb,
                                               uint32_t &flags)
{
    const int32_t stride = a.table_stride;
    const int32_t *counts = a.num_blocks_per_req;
    if (stride <= 0 && !counts) return -1;  // uniform: no row, nothing to load
    const int32_t *entry = stride > 0
        ? a.block_table + static_cast<int64_t>(r) * stride + min(lb, static_cast<int64_t>(stride) - 1)
        : counts + r;
    const int32_t *count = counts ? counts + r : entry;
    int32_t b = *entry, n = *count;
    asm volatile("" : "+s"(b), "+s"(n));  // both issued before either is waited on
    int64_t bound = stride;
    if (counts) bound = clamp_count(n, stride, flags);
    if (lb >= bound) return -1;  // with stride 0 every lb is out of the row
    if (b < 0) { flags |= KVW_FLAG_BAD_BLOCK; return -1; }
    return b;
}

// Block of lb in the run (cum c, length l, start st), or -1.  Branch-free: a
// field used only under a branch would be loaded there, after the others.
__device__ __forceinline__ int64_t run_block(int64_t c, int64_t l, int64_t st, int64_t lb,
                                             uint32_t &flags)
{
    const bool in = lb >= c && lb < c + l;
    const int64_t b = st + (lb - c);
    flags |= in && b < 0 ? static_cast<uint32_t>(KVW_FLAG_BAD_BLOCK) : 0u;
    return in && b >= 0 ? b : -1;
}

// Run of lb among runs [0, m) of a row (fields cum, len, start) whose next
// run starts at c_end > lb (cum[m] = c_end): the largest i < m with
// cum[i] <= lb, or -1.  Interpolation first: with runs of equal length the run
// is i = lb * m / c_end, and with unequal ones it lies near there, so one
// 64-entry window around that guess, its three fields loaded together (one
// memory latency) and a ballot, usually settles it; otherwise the full
// wave-uniform search.  The run's fields go to c_i, l_i and s_i.
__device__ __forceinline__ int32_t run_below(const int32_t *cum, const int32_t *len,
                                             const int32_t *start, int32_t m, int64_t lb,
                                             int64_t c_end, int64_t &c_i, int64_t &l_i,
                                             int64_t &s_i)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (m <= 0) return -1;
    const int32_t g = static_cast<int32_t>(lb * m / c_end);  // 0 <= g < m: 0 <= lb < c_end
    const int32_t a = max(0, min(g - kWave / 2, m - kWave));
    const int32_t wlen = min(kWave, m - a);
    const int32_t w = a + min(lane, wlen - 1);  // unconditional loads at a clamped index
    int32_t cw = cum[w], lw = len[w], sw = start[w];
    asm volatile("" : "+v"(cw), "+v"(lw), "+v"(sw));  // all three out before any is waited on
    const int32_t cv = lane < wlen ? cw : INT32_MAX;
    const int32_t cnt = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(__popcll(__ballot(cv <= lb))));
    if (cnt > 0 && (cnt < wlen || a + wlen == m)) {
        c_i = __builtin_amdgcn_readlane(cv, cnt - 1);
        l_i = __builtin_amdgcn_readlane(lw, cnt - 1);
        s_i = __builtin_amdgcn_readlane(sw, cnt - 1);
        return a + cnt - 1;
    }
    if (cnt == 0 && a == 0) return -1;
    const int32_t i = wave_uniform_upper_index(cum, m, lb);
    if (i >= 0) {
        c_i = cum[i];
        l_i = len[i];
        s_i = start[i];
    }
    return i;
}

// Slot of token t < num_tokens of request r (-1: none) at position p
// (one-kernel path: t is the same on every lane of the wave), or the pad id.
// All loads are wave-uniform.  Ranges: count_raw is num_ranges[r], found
// together with r.
template <int MODE>
__device__ __forceinline__ int64_t resolve_slot(const MapArgs &a, int32_t r, int64_t p,
                                                int32_t count_raw, uint32_t &flags)
{
    if (r < 0 || p < 0) return KVW_PAD_ID;
    int64_t lb;
    int32_t off;
    if (!locate(a, p, lb, off)) return KVW_PAD_ID;  // another context-parallel rank's token
    int64_t b;
    if (MODE == kPaged) {
        b = paged_block(a, r, lb, flags);
    } else {
        const int32_t n = static_cast<int32_t>(clamp_count(count_raw, a.range_stride, flags));
        if (n == 0) return KVW_PAD_ID;
        const int64_t row = static_cast<int64_t>(r) * a.range_stride;
        // the last run first, its three fields loaded together and waited on once (a
        // widening fused with each load would wait for it before the next goes out);
        // then the runs below it
        int32_t c32 = a.range_cum[row + n - 1], l32 = a.range_len[row + n - 1],
                s32 = a.range_start[row + n - 1];
        asm volatile("" : "+s"(c32), "+s"(l32), "+s"(s32));  // every use comes after all three
        const int64_t c_last = c32, l_last = l32, s_last = s32;
        if (lb >= c_last) {
            b = run_block(c_last, l_last, s_last, lb, flags);
        } else {
            int64_t c_i = 0, l_i = 0, s_i = 0;
            const int32_t i = run_below(a.range_cum + row, a.range_len + row, a.range_start + row,
                                        n - 1, lb, c_last, c_i, l_i, s_i);
            if (i < 0) return KVW_PAD_ID;
            b = run_block(c_i, l_i, s_i, lb, flags);
        }
    }
    if (b < 0) return KVW_PAD_ID;
    return b * a.block_size + off;
}

// The first level of the search of one request's runs by the lanes of a wave
// (the rows of range descriptors are loaded once for the wave's positions):
// for rows of at most 128 descriptors (width = range_stride), every cum, len
// and start entry, two per lane; above that, 64 evenly spaced cum entries.
// None of it depends on the positions or on the row's count, so these loads
// go out together with the position and count loads; entries past the count
// are masked afterwards.
struct RunWindow {
    int32_t c0, c1, l0, l1, s0, s1;  // window: entries lane and lane + 64
    int32_t step;                    // 0: window of the whole row; else the cum samples are
                                     // c0 = cum[lane * step]
};

__device__ __forceinline__ RunWindow run_window(const MapArgs &a, int64_t row, int32_t width)
{
    const int lane = threadIdx.x & (kWave - 1);
    RunWindow w{0, 0, 0, 0, 0, 0, 0};
    if (width <= 0) return w;  // uniform; loads below are unconditional at clamped indices
    if (width <= 2 * kWave) {
        const int64_t i0 = row + min(lane, width - 1), i1 = row + min(lane + kWave, width - 1);
        w.c0 = a.range_cum[i0];
        w.l0 = a.range_len[i0];
        w.s0 = a.range_start[i0];
        w.c1 = a.range_cum[i1];
        w.l1 = a.range_len[i1];
        w.s1 = a.range_start[i1];
    } else {
        w.step = (width + kWave - 1) / kWave;
        w.c0 = a.range_cum[row + min(lane * w.step, width - 1)];
    }
    return w;
}

// The search of row `row` (n descriptors, n <= width) for the lanes with part
// (every lane calls), in two phases so that the loads of several searches go
// out before any of them is waited on.  run_probe: in window mode the window
// is already in registers; otherwise the samples give each lane a bucket, and
// the loads of one window (cum, len and start) covering all of the wave's
// buckets are issued, or, when the buckets lie too far apart, each lane
// binary-searches its own bucket.  run_pick: the last i with cum[i] <= lb and
// that run's descriptor.  Ranks are counted with ballots when the lanes' keys
// span few values (consecutive positions span few logical blocks: 64 tokens
// at block size 16 at most 5): one compare and one ballot per distinct key,
// and the descriptor taken with readlane from the uniform index; otherwise
// with a shuffle search per lane and shuffles from the lane holding the run.
constexpr int32_t kNarrowKeys = 16;
constexpr int32_t kFewStarts = 4;  // run starts inside a narrow key span taken without a loop

struct RunProbe {
    int32_t lo, len;                 // the window [lo, lo + len) of the row
    int32_t c0, c1, l0, l1, s0, s1;  // its entries lane and lane + 64
    int32_t hit;                     // len == 0: this lane's own result, or -1
    int64_t hc, hl, hs;
    int32_t kmin, kmax;              // the taking-part lanes' keys (clamped to int32)
};

// Key of a lane for comparisons with int32 entries: lb clamped (entries are int32).
__device__ __forceinline__ int32_t key32(int64_t lb) { return lb > INT32_MAX ? INT32_MAX : static_cast<int32_t>(lb); }

// Number of the window's entries <= k (k wave-uniform), the window in (w0, w1) for
// lanes below len.
__device__ __forceinline__ int32_t ballot_rank(int32_t w0, int32_t w1, int32_t len, int32_t k)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t c0 = __popcll(__ballot(lane < len && w0 <= k));
    const int32_t c1 = __popcll(__ballot(lane + kWave < len && w1 <= k));
    return c0 == kWave ? kWave + c1 : c0;
}

__device__ RunProbe run_probe(const MapArgs &a, int64_t row, const RunWindow &w, int32_t n,
                              int64_t lb, bool part)
{
    const int lane = threadIdx.x & (kWave - 1);
    RunProbe p{0, n, w.c0, w.c1, w.l0, w.l1, w.s0, w.s1, -1, 0, 0, 0, 0, 0};
    const int32_t key = key32(lb);
    p.kmin = wave_min(part ? key : INT32_MAX);
    p.kmax = wave_max(part ? key : INT32_MIN);
    if (n <= 0 || p.kmin == INT32_MAX) {
        p.len = 0;
        return p;
    }
    if (w.step == 0) return p;
    const bool sampled = lane * w.step < n;
    int32_t cnt = 0, u_lo, u_hi;
    if (p.kmax - p.kmin < kNarrowKeys) {
        // buckets of the smallest and largest key bound every lane's
        const int32_t cmin = __popcll(__ballot(sampled && w.c0 <= p.kmin));
        const int32_t cmax = __popcll(__ballot(sampled && w.c0 <= p.kmax));
        u_lo = cmax == 0 ? INT32_MAX : max(cmin - 1, 0) * w.step;
        u_hi = min(cmax * w.step, n);
        if (u_lo != INT32_MAX && u_hi - u_lo > 2 * kWave)
            for (int32_t k = p.kmin; k <= p.kmax; ++k) {  // each lane's own count
                const int32_t ck = __popcll(__ballot(sampled && w.c0 <= k));
                if (key == k) cnt = ck;
            }
    } else {
        cnt = wave_rank(sampled ? static_cast<int64_t>(w.c0) : INT64_MAX, lb);
        int32_t b_lo = INT32_MAX, b_hi = INT32_MIN;  // this lane's bucket [b_lo, b_hi)
        if (part && cnt > 0) {
            b_lo = (cnt - 1) * w.step;
            b_hi = min(cnt * w.step, n);
        }
        u_lo = wave_min(b_lo);
        u_hi = wave_max(b_hi);
    }
    if (u_lo == INT32_MAX || u_hi - u_lo > 2 * kWave) {
        p.len = 0;
        if (u_lo != INT32_MAX && part && cnt > 0) {
            int32_t x = (cnt - 1) * w.step, h = min(cnt * w.step, n);  // cum[x] <= lb
            while (h - x > 1) {
                const int32_t mid = (x + h) >> 1;
                if (a.range_cum[row + mid] <= lb) x = mid; else h = mid;
            }
            p.hit = x;
            p.hc = a.range_cum[row + x];
            p.hl = a.range_len[row + x];
            p.hs = a.range_start[row + x];
        }
        return p;
    }
    p.lo = u_lo;
    p.len = u_hi - u_lo;  // >= 1; the loads are unconditional at clamped indices
    const int64_t i0 = row + p.lo + min(lane, p.len - 1), i1 = row + p.lo + min(lane + kWave, p.len - 1);
    p.c0 = a.range_cum[i0];
    p.l0 = a.range_len[i0];
    p.s0 = a.range_start[i0];
    p.c1 = a.range_cum[i1];
    p.l1 = a.range_len[i1];
    p.s1 = a.range_start[i1];
    return p;
}

__device__ int32_t run_pick(const RunProbe &p, int64_t lb, bool part, int64_t &c, int64_t &l,
                            int64_t &st)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (p.len == 0) {  // uniform
        if (!part || p.hit < 0) return -1;
        c = p.hc;
        l = p.hl;
        st = p.hs;
        return p.hit;
    }
    if (p.kmax - p.kmin < kNarrowKeys) {  // uniform
        const int32_t key = key32(lb);
        // Runs c_lo - 1 .. c_hi - 1 of the window hold every lane's key; with few
        // run starts between the smallest and the largest key, each lane counts
        // the starts at or below its key (read once, uniform) and takes its run's
        // descriptor from the lane that holds it.  Every read happens while all
        // lanes are active: the lane read from need not take part.
        const int32_t c_lo = ballot_rank(p.c0, p.c1, p.len, p.kmin);
        const int32_t c_hi = ballot_rank(p.c0, p.c1, p.len, p.kmax);
        if (c_hi == c_lo) {  // uniform: one run
            if (c_lo == 0) return -1;  // every key before the first run
            const int32_t idx = c_lo - 1, src = idx & (kWave - 1);
            const bool hi = idx >= kWave;
            const int32_t ck = __builtin_amdgcn_readlane(hi ? p.c1 : p.c0, src);
            const int32_t lk = __builtin_amdgcn_readlane(hi ? p.l1 : p.l0, src);
            const int32_t sk = __builtin_amdgcn_readlane(hi ? p.s1 : p.s0, src);
            if (!part) return -1;
            c = ck;
            l = lk;
            st = sk;
            return p.lo + idx;
        }
        if (c_hi - c_lo <= kFewStarts) {  // uniform
            int32_t idx = c_lo - 1;
#pragma unroll
            for (int32_t j = 0; j < kFewStarts; ++j) {
                const int32_t e = min(c_lo + j, c_hi - 1);  // a run start inside the keys' span
                const int32_t ce = __builtin_amdgcn_readlane(e >= kWave ? p.c1 : p.c0, e & (kWave - 1));
                idx += c_lo + j < c_hi && ce <= key ? 1 : 0;
            }
            const int32_t src = max(idx, 0) & (kWave - 1);
            const int32_t cl = __shfl(p.c0, src), ch = __shfl(p.c1, src);
            const int32_t ll = __shfl(p.l0, src), lh = __shfl(p.l1, src);
            const int32_t sl = __shfl(p.s0, src), sh = __shfl(p.s1, src);
            if (!part || idx < 0) return -1;
            c = idx < kWave ? cl : ch;
            l = idx < kWave ? ll : lh;
            st = idx < kWave ? sl : sh;
            return p.lo + idx;
        }
        int32_t found = -1;
        for (int32_t k = p.kmin; k <= p.kmax; ++k) {
            const int32_t cnt = ballot_rank(p.c0, p.c1, p.len, k);
            if (cnt == 0) continue;  // uniform: every key k's lane is before the first run
            const int32_t idx = cnt - 1, src = idx & (kWave - 1);
            const bool hi = idx >= kWave;
            const int32_t ck = __builtin_amdgcn_readlane(hi ? p.c1 : p.c0, src);
            const int32_t lk = __builtin_amdgcn_readlane(hi ? p.l1 : p.l0, src);
            const int32_t sk = __builtin_amdgcn_readlane(hi ? p.s1 : p.s0, src);
            if (part && key == k) {
                c = ck;
                l = lk;
                st = sk;
                found = p.lo + idx;
            }
        }
        return found;
    }
    int cnt = wave_rank(lane < p.len ? static_cast<int64_t>(p.c0) : INT64_MAX, lb);
    const int cnt1 = wave_rank(lane + kWave < p.len ? static_cast<int64_t>(p.c1) : INT64_MAX, lb);
    if (cnt == kWave) cnt += cnt1;
    const int32_t k = part && cnt > 0 ? cnt - 1 : -1;  // index inside the window
    const int src = k >= 0 ? (k & (kWave - 1)) : 0;
    const int32_t cl = __shfl(p.c0, src), ch = __shfl(p.c1, src);
    const int32_t ll = __shfl(p.l0, src), lh = __shfl(p.l1, src);
    const int32_t sl = __shfl(p.s0, src), sh = __shfl(p.s1, src);
    if (k < 0) return -1;
    c = k < kWave ? cl : ch;
    l = k < kWave ? ll : lh;
    st = k < kWave ? sl : sh;
    return p.lo + k;
}

// Entry q of row r of a kernel-unit table expanded from a manager table
// ([P2] "Entwurfsmotivation"; [P3] section 7): ids[r][i]*k + j for q = i*k + j
// while i < count[r], else 0 (the null block).  With counts_out, entry 0 of a
// row also writes the row's kernel-block count, count[r] * k.
__device__ __forceinline__ void expand_entry(const int32_t *ids, const int32_t *counts,
                                             int32_t in_stride, int32_t k, int32_t *out,
                                             int32_t out_stride, int32_t *counts_out, int32_t r,
                                             int32_t q, uint32_t &flags)
{
    const int32_t i = q / k, j = q - (q / k) * k;
    const int64_t count = counts ? clamp_count(counts[r], in_stride, flags) : in_stride;
    int32_t v = 0;
    if (i < count) {
        const int64_t id = ids[static_cast<int64_t>(r) * in_stride + i];
        if (expandable(id, k)) v = static_cast<int32_t>(id * k + j);
        else flags |= KVW_FLAG_BAD_BLOCK;
    }
    out[static_cast<int64_t>(r) * out_stride + q] = v;
    if (counts_out && q == 0) counts_out[r] = static_cast<int32_t>(count * k);
}

// Entry q (one per lane; r uniform over the wave, every lane calls) of row r
// of a block table filled from range descriptors ([P1] "Status"): kernel
// block j = q % k of the manager block at logical index q / k, i.e. of
// start[i] + (q / k - cum[i]) for the run i holding it; 0 past the runs.  The
// consecutive logical blocks of a wave (at most 64, each run at least one
// block long) fall in at most 64 consecutive runs, found with one wavefront
// search of the row's cum column.  Entry 0 writes the count,
// (cum[n-1] + len[n-1]) * k clamped to the row width, which under the
// descriptor precondition is the total length of the runs.
__device__ __forceinline__ void fill_table_row(const int32_t *start, const int32_t *len,
                                               const int32_t *cum, const int32_t *num_ranges,
                                               int32_t range_stride, int32_t k, int32_t *out,
                                               int32_t out_stride, int32_t *counts_out, int32_t r,
                                               int64_t q, uint32_t &flags)
{
    const bool in = q < out_stride;
    const uint32_t uq = static_cast<uint32_t>(in ? q : 0);
    const uint32_t lb32 = uq / static_cast<uint32_t>(k);
    const int64_t lb = lb32;
    const int32_t j = static_cast<int32_t>(uq - lb32 * static_cast<uint32_t>(k));
    uint32_t count_flags = 0;
    const int64_t row = static_cast<int64_t>(r) * range_stride;
    const int32_t n = static_cast<int32_t>(clamp_count(num_ranges[r], range_stride, count_flags));
    const int32_t i = wave_upper_index(cum + row, n, lb, in);
    int32_t v = 0;
    if (in && i >= 0) {
        const int64_t c = cum[row + i];
        if (lb >= c && lb < c + len[row + i]) {
            const int64_t b = static_cast<int64_t>(start[row + i]) + (lb - c);
            if (expandable(b, k)) v = static_cast<int32_t>(b * k + j);
            else flags |= KVW_FLAG_BAD_BLOCK;
        }
    }
    if (in) out[static_cast<int64_t>(r) * out_stride + q] = v;
    if (q == 0) {
        int64_t total = 0;
        if (n > 0) total = (static_cast<int64_t>(cum[row + n - 1]) + len[row + n - 1]) * k;
        if (total < 0) total = 0;
        if (total > out_stride) count_flags |= KVW_FLAG_COUNT;
        if (counts_out) counts_out[r] = static_cast<int32_t>(total < out_stride ? total : out_stride);
        flags |= count_flags;
    }
}

// The table role of a slot-mapping launch: workgroup tb of the workgroups
// past the slot-mapping ones.
template <int MODE>
__device__ __forceinline__ void table_role(const MapArgs &a, uint32_t tb)
{
    uint32_t flags = 0;
    if (MODE == kPaged) {
        const int64_t idx = static_cast<int64_t>(tb) * kSlotThreads + threadIdx.x;
        if (idx < static_cast<int64_t>(a.num_reqs) * a.table_out_stride) {
            const int32_t r = static_cast<int32_t>(idx / a.table_out_stride);
            const int32_t q = static_cast<int32_t>(idx - static_cast<int64_t>(r) * a.table_out_stride);
            expand_entry(a.block_table, a.num_blocks_per_req, a.table_stride, a.table_k, a.table_out,
                         a.table_out_stride, a.table_counts_out, r, q, flags);
        }
    } else {
        const int32_t r = static_cast<int32_t>(tb / a.table_blocks_per_row);
        const int64_t q = static_cast<int64_t>(tb - static_cast<uint32_t>(r) * a.table_blocks_per_row) *
                              kSlotThreads + threadIdx.x;
        fill_table_row(a.range_start, a.range_len, a.range_cum, a.num_ranges, a.range_stride,
                       a.table_k, a.table_out, a.table_out_stride, a.table_counts_out, r, q, flags);
    }
    raise_flags(a.err_flag, flags);
}

// One token per lane; the wave finds its tokens' requests (and, for ranges,
// the runs of the tokens of its first request) with wavefront searches.
// One token per lane; WIDE: more than 128 requests (two search levels).
template <int MODE, bool WIDE>
__device__ __forceinline__ void slot_mapping_tokens(const MapArgs &a)
{
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kSlotThreads + threadIdx.x;
    const bool in = t < a.max_num_tokens;  // every lane stays for the wave-wide searches
    // Loads are unconditional, at indices clamped into their arrays, and the values
    // masked at their use: the compiler moves a load under a branch to its use and
    // waits there for it and every load before it, which would serialize loads meant
    // to be in flight together.  The request search's first level, the positions
    // (all max_num_tokens of them are readable; a padded token's is ignored) and
    // the token count (a scalar load) go out together.  Ranges: each lane's run
    // count comes with its request, loaded beside the search's last level, so the
    // request's runs are one load further, not two.
    constexpr bool kCounts = MODE == kRanges;
    const WaveSamples qs = wave_samples<kCounts, WIDE>(a.qsl, a.num_reqs, a.num_ranges);
    const int64_t pv = a.positions[min(t, a.max_num_tokens - 1)];
    uint32_t nt_flag = 0, flags = 0;
    const int64_t num_tokens = device_num_tokens(a, nt_flag);
    const bool real = in && t < num_tokens;
    const int64_t keep = real ? ~int64_t{0} : 0;  // -1 for padded tokens, without a select on the load
    const int64_t p = (pv & keep) | ~keep;
    int32_t r_count = 0;
    const int32_t r = wave_search<kCounts, WIDE>(a.qsl, qs, t, real, a.num_ranges, &r_count);
    const int32_t bs = a.block_size;
    int64_t lb = 0;
    int32_t off = 0;
    // a token of another context-parallel rank is padding and reads nothing more
    const bool ok = real && r >= 0 && p >= 0 && locate(a, p, lb, off);
    const bool has_r = real && r >= 0;
    const uint64_t reals = __ballot(has_r);
    const int lane_a = reals ? __builtin_ctzll(reals) : 0;
    const int32_t lead_a = reals ? __builtin_amdgcn_readlane(r, lane_a) : 0;
    const int32_t r_safe = has_r ? r : lead_a;  // a real request of the wave for every lane
    int64_t b = -1;
    if (MODE == kPaged) {
        if (reals && a.table_stride > 0) {  // uniform
            const int64_t lb_in = ok && lb < a.table_stride ? lb : 0;
            const int32_t entry = a.block_table[static_cast<int64_t>(r_safe) * a.table_stride + lb_in];
            int64_t bound = a.table_stride;
            uint32_t count_flags = 0;
            if (a.num_blocks_per_req)
                bound = clamp_count(a.num_blocks_per_req[r_safe], a.table_stride, count_flags);
            if (ok) {
                flags |= count_flags;
                if (lb < bound) {
                    if (entry < 0) flags |= KVW_FLAG_BAD_BLOCK;
                    else b = entry;
                }
            }
        } else if (ok && a.num_blocks_per_req) {  // stride 0: no entry; the count is still checked
            uint32_t count_flags = 0;
            clamp_count(a.num_blocks_per_req[r], a.table_stride, count_flags);
            flags |= count_flags;
        }
    } else if (reals) {  // uniform
        // The count of each lane's request, then, together: the request's last run
        // (where decode positions and the end of a prefill chunk lie) and the first
        // search level of the rows of the wave's first and last requests when they
        // hold two lanes or more (a wave of consecutive tokens seldom spans more
        // requests); those lanes search their row together, the descriptors loaded
        // once for the wave's positions.  A lane of any other request outside its
        // last run (rare: a chunk that starts inside the wave) is settled by a
        // further cooperative search of its request's row.
        const int lane_b = 63 - __builtin_clzll(reals);
        const int32_t lead_b = __builtin_amdgcn_readlane(r, lane_b);
        uint32_t count_flags = 0;
        const int32_t count_a = __builtin_amdgcn_readlane(r_count, lane_a);  // lanes without a request take lead_a's
        const int32_t n_all =
            static_cast<int32_t>(clamp_count(has_r ? r_count : count_a, a.range_stride, count_flags));
        if (ok) flags |= count_flags;  // the count's flag, per token that uses it
        const int32_t n = ok ? n_all : 0;
        const int32_t n_a = __builtin_amdgcn_readlane(n_all, lane_a), n_b = __builtin_amdgcn_readlane(n_all, lane_b);
        if (a.range_stride > 0) {  // uniform; with no descriptor every slot is padding
            const bool two_a = __popcll(__ballot(has_r && r == lead_a)) >= 2;  // uniform
            const bool two_b = lead_b != lead_a && __popcll(__ballot(has_r && r == lead_b)) >= 2;
            const int64_t row_a = static_cast<int64_t>(lead_a) * a.range_stride;
            const int64_t row_b = static_cast<int64_t>(lead_b) * a.range_stride;
            const int64_t row = static_cast<int64_t>(r_safe) * a.range_stride;
            const int64_t i_last = row + (n_all > 0 ? n_all - 1 : 0);
            const int64_t c_last = a.range_cum[i_last], l_last = a.range_len[i_last],
                          s_last = a.range_start[i_last];
            const RunWindow win_a = run_window(a, row_a, two_a ? n_a : 0);
            const RunWindow win_b = run_window(a, row_b, two_b ? n_b : 0);
            // positions in their request's last run are settled at once; the
            // windows serve only the lanes left (none, for decode steps and for
            // chunks that lie in one run)
            asm volatile("" ::"v"(l_last), "v"(s_last));  // all three loaded here, together
            bool pending = n > 0;
            if (pending && lb >= c_last) {
                b = run_block(c_last, l_last, s_last, lb, flags);
                pending = false;
            }
            const bool in_a = two_a && pending && r == lead_a;
            const bool in_b = two_b && pending && r == lead_b;
            int64_t c = 0, l = 0, st = 0;
            if (__ballot(in_a)) {  // uniform
                const RunProbe pa = run_probe(a, row_a, win_a, n_a, lb, in_a);
                if (run_pick(pa, lb, in_a, c, l, st) >= 0 && in_a) b = run_block(c, l, st, lb, flags);
            }
            if (__ballot(in_b)) {  // uniform
                const RunProbe pb = run_probe(a, row_b, win_b, n_b, lb, in_b);
                if (run_pick(pb, lb, in_b, c, l, st) >= 0 && in_b) b = run_block(c, l, st, lb, flags);
            }
            if (in_a || in_b) pending = false;
            for (uint64_t left = __ballot(pending); left; left = __ballot(pending)) {  // uniform
                const int lane_c = __builtin_ctzll(left);
                const int32_t lead_c = __builtin_amdgcn_readlane(r, lane_c), n_c = __builtin_amdgcn_readlane(n_all, lane_c);
                const int64_t row_c = static_cast<int64_t>(lead_c) * a.range_stride;
                const bool in_c = pending && r == lead_c;
                const RunProbe pc = run_probe(a, row_c, run_window(a, row_c, n_c), n_c, lb, in_c);
                if (run_pick(pc, lb, in_c, c, l, st) >= 0 && in_c) b = run_block(c, l, st, lb, flags);
                if (in_c) pending = false;
            }
        }
    }
    if (in) a.slots_out[t] = b < 0 ? KVW_PAD_ID : b * bs + off;
    raise_flags(a.err_flag, flags | (t == 0 ? nt_flag : 0u));
}

// One-wave workgroups: a small batch's waves land on as many compute units,
// each with its own L1 and address units for the wave's gathers (a decode
// step of 256 tokens: four units, not one).  On cold caches this took range
// resolution from 8.1 to 6.6 µs per launch on a 256-request decode step and
// about 1 µs off the small prefill, mixed and 32-layer batches; the gather
// moved by under 0.5 µs either way.
template <int MODE>
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(MapArgs a)
{
    if (blockIdx.x >= a.slot_blocks) {  // uniform over the workgroup; no barriers below
        table_role<MODE>(a, blockIdx.x - a.slot_blocks);
        return;
    }
    if (a.num_reqs > 2 * kWave) slot_mapping_tokens<MODE, true>(a);  // uniform
    else slot_mapping_tokens<MODE, false>(a);
}



// One wave per (layer, token, plane, 1 KiB slice) item.  The token is
// wave-uniform; its slot is one scalar load, and the slice is read once the
// slot is known.  (Issuing the read together with the slot load was measured
// on 131,072 tokens of 2 KiB rows: no faster on a contiguous cache and 0.5%
// slower on a fully fragmented one, where the scattered writes bound the
// kernel and earlier reads compete with them.)  Items are ordered
// layer-major (blockIdx.y), then token, plane, slice, so consecutive waves
// stream through consecutive K/V rows and, for tokens of one block,
// consecutive cache slots.
// TPW > 1 (context parallelism, where most neighbouring tokens of a rank's
// batch are another rank's): one wave takes the same slice of TPW consecutive
// tokens and skips the padded ones, so far fewer waves start only to exit.
template <int TPW>
__global__ __launch_bounds__(kScatterThreads) void kv_scatter_kernel(const int64_t *slots,
                                                                     CopyArgs c, int32_t *err_flag)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t item = static_cast<uint64_t>(blockIdx.x) * kScatterWaves + wave;
    int32_t items_log2 = c.items_log2;
    asm("" : "+s"(items_log2) : "s"(slots));  // both argument lines in one round trip
    uint64_t g64;
    uint32_t r;
    if (items_log2 >= 0) {
        g64 = item >> items_log2;
        r = static_cast<uint32_t>(item & ((1u << items_log2) - 1));
    } else {
        g64 = item / c.items_per_token;
        r = static_cast<uint32_t>(item - g64 * c.items_per_token);
    }
    const uint32_t plane = r >= c.slices_per_row ? 1u : 0u;
    const uint32_t slice = r - plane * c.slices_per_row;
    const int64_t off = static_cast<int64_t>(slice) * kSliceBytes + static_cast<int64_t>(lane) * 16;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const uint64_t t64 = g64 * TPW + j;
        if (t64 >= static_cast<uint64_t>(c.max_num_tokens)) return;
        const int64_t t = static_cast<int64_t>(t64);
        const int64_t slot = slots[t];
        if (slot >= c.rows_per_layer) {  // beyond the cache: skipped, reported once per token
            if (blockIdx.y == 0 && r == 0 && lane == 0) raise_flags(err_flag, KVW_FLAG_SLOT_OOB);
            continue;
        }
        if (slot < 0 || off >= c.bytes_per_token) continue;
        const uint8_t *src = (plane ? c.value : c.key) + t * c.kv_token_stride + off;
        uint8_t *row = (plane ? c.v_cache : c.k_cache) + slot * c.bytes_per_token;  // wave-uniform
        // coordinate n = (l*B + slot/T)*T + slot%T = l*B*T + slot
        for (int64_t l = blockIdx.y; l < c.num_layers; l += gridDim.y)
            store16_through(row + l * c.rows_per_layer * c.bytes_per_token, static_cast<uint32_t>(off),
                            load16<KVW_NT_LOADS>(src + l * c.kv_layer_stride));
    }
}

// Rows shorter than a wave's 1 KiB: one wave copies one plane of up to
// rows_per_wave consecutive tokens (lane group g of lanes_per_row lanes takes
// token t0 + g), so a wave still moves up to 1 KiB; each lane reads its own
// token's slot.  EAGER (no context parallelism): each lane's row load goes out
// with its slot load, so the wave waits for the two together (2-3% faster at
// 256 and 512 B rows); under context parallelism most rows are another
// rank's, so a row is read only once its slot is known.
template <bool EAGER>
__global__ __launch_bounds__(kScatterThreads) void kv_scatter_small_kernel(const int64_t *slots,
                                                                           CopyArgs c,
                                                                           int32_t *err_flag)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint64_t item = static_cast<uint64_t>(blockIdx.x) * kScatterWaves + wave;
    const uint32_t plane = static_cast<uint32_t>(item & 1);
    uint32_t lanes_per_row = c.lanes_per_row;
    asm("" : "+s"(lanes_per_row) : "s"(slots));  // both argument lines in one round trip
    const uint32_t g = static_cast<uint32_t>(lane) / lanes_per_row;
    if (g >= c.rows_per_wave) return;
    const uint64_t t64 = (item >> 1) * c.rows_per_wave + g;
    if (t64 >= static_cast<uint64_t>(c.max_num_tokens)) return;
    const int64_t t = static_cast<int64_t>(t64);
    const int64_t off = static_cast<int64_t>(static_cast<uint32_t>(lane) - g * lanes_per_row) * 16;
    const uint8_t *src = (plane ? c.value : c.key) + t * c.kv_token_stride + off;
    const int64_t l0 = blockIdx.y;  // < num_layers: the grid has at most num_layers rows
    int64_t slot = slots[t];
    u32x4 first{};
    if (EAGER) {  // the row's first layer goes out before the slot is waited on
        first = load16<KVW_NT_LOADS>(src + l0 * c.kv_layer_stride);
        asm("" : "+v"(slot), "+v"(first));
    }
    if (slot >= c.rows_per_layer) {  // beyond the cache: skipped, reported once per token
        if (l0 == 0 && plane == 0 && off == 0) raise_flags(err_flag, KVW_FLAG_SLOT_OOB);
        return;
    }
    if (slot < 0) return;
    uint8_t *dst = (plane ? c.v_cache : c.k_cache) + slot * c.bytes_per_token + off;
    if (!EAGER) first = load16<KVW_NT_LOADS>(src + l0 * c.kv_layer_stride);
    store16_device(dst + l0 * c.rows_per_layer * c.bytes_per_token, first);
    for (int64_t l = l0 + gridDim.y; l < c.num_layers; l += gridDim.y)
        store16_device(dst + l * c.rows_per_layer * c.bytes_per_token,
                       load16<KVW_NT_LOADS>(src + l * c.kv_layer_stride));
}

// One wave per (token, plane) (PLANES = 1) or per token (PLANES = 2, both
// planes) and layer group (blockIdx.y); the wave resolves the slot with
// wave-uniform searches, then copies.  Small writes (PLANES = 2, one wave per
// token: half the slot resolutions, which wins where their latency dominates,
// a grid that does not fill the GPU twice) issue the loads of the token's rows
// for the group's first layer before resolving, so they are in flight during
// it.  Large writes (PLANES = 1: two waves per token keep more transfers in
// flight per byte) read a row only once its slot is known, like the two-kernel
// scatter, and store it through L2: 2% faster than reading ahead at 128K tokens
// on contiguous and on fully fragmented caches, where the scattered writes, not
// the waves' latency, set the pace.  Rows longer than CH KiB are copied in
// further CH KiB segments.  The wave that holds plane 0 reports the slot and
// the flags.
template <int MODE, int CH, int PLANES, bool ROWS>
__global__ __launch_bounds__(kFusedThreads) void kv_write_fused_kernel(MapArgs a, CopyArgs c)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kFusedWaves +
                         __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = PLANES == 2 ? item : item >> 1;
    const int plane0 = PLANES == 2 ? 0 : static_cast<int>(item & 1);  // first plane of the wave
    // Kernel arguments are scalar loads, and a wave's first ones miss the scalar
    // cache.  The compiler issues them where they are first used, so a prologue
    // with a branch would wait for one 64-byte line of them before asking for the
    // next.  Making the first branch's operand depend on a field of every line
    // the prologue reads sends them out in one round trip.
    int64_t max_tokens = a.max_num_tokens;
    asm("" : "+s"(max_tokens) : "s"(a.qsl), "s"(c.key), "s"(c.kv_token_stride));
    if (t >= max_tokens) return;  // whole wave: this kernel has no barrier
    const int l0 = blockIdx.y * c.layers_per_wave;
    const int l1 = min(c.num_layers, l0 + c.layers_per_wave);
    const int64_t bpt = c.bytes_per_token;
    const int64_t lane_off = static_cast<int64_t>(lane) * 16;
    const uint8_t *src[PLANES];
#pragma unroll
    for (int q = 0; q < PLANES; ++q)
        src[q] = (plane0 + q ? c.value : c.key) + t * c.kv_token_stride + lane_off;

    // Vector loads complete in order, and a load under a branch is waited on
    // before the branch joins.  So the request search's one vector load goes out
    // first (up to 128 requests: one level; for ranges with the requests' run
    // counts beside it), then (small writes) the rows' first loads, all
    // unconditional and independent of the token count: waiting for the search
    // then leaves the rows in flight while the slot is resolved with scalar
    // loads.  A padded token's rows are read too (they lie inside key/value) and
    // never stored; lanes past a row's end read inside the row.
    constexpr bool kCounts = MODE == kRanges;
    const bool one_level = a.num_reqs <= 2 * kWave;
    const UniformWindow qw = uniform_window<kCounts>(a.qsl, one_level ? a.num_reqs : 0, a.num_ranges);
    __builtin_amdgcn_sched_barrier(0);  // keep the search's load ahead of the rows'
    u32x4 row[PLANES][CH];
    if (ROWS && PLANES == 2) {  // launches with layers: l0 < l1
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int64_t off = min(lane_off + ch * kSliceBytes, bpt - 16) - lane_off;
#pragma unroll
            for (int q = 0; q < PLANES; ++q)
                row[q][ch] = load16<KVW_NT_LOADS>(src[q] + l0 * c.kv_layer_stride + off);
        }
    }
    uint32_t flags = 0;
    // the position and the token count go out together (scalar loads, after the
    // rows': any wait for a scalar load waits for all of them); positions holds
    // max_num_tokens entries, and a padded token's is read and ignored
    const int64_t pv = a.positions[t];
    const int64_t num_tokens = device_num_tokens(a, flags);
    if (t != 0) flags = 0;
    const bool real = t < num_tokens;
    const int64_t keep = real ? ~int64_t{0} : 0;  // -1 for padded tokens, without a select on the load
    const int64_t p = (pv & keep) | ~keep;
    // no branch on real before the position is used (a padded token has p = -1 and
    // gets the pad id): the compiler would move the position's load under it
    int32_t r, count = 0;
    if (one_level) {
        r = uniform_rank(qw, t);
        if (kCounts && r >= 0) count = uniform_entry(qw.c0, qw.c1, r);
    } else {
        r = wave_uniform_upper_index<kCounts>(a.qsl, a.num_reqs, t, a.num_ranges, &count);
    }
    int64_t slot = resolve_slot<MODE>(a, r, p, count, flags);
    const bool report = blockIdx.y == 0 && plane0 == 0;
    if (report && lane == 0 && a.slots_out) a.slots_out[t] = slot;
    if (slot >= c.rows_per_layer) {
        if (c.num_layers > 0) flags |= KVW_FLAG_SLOT_OOB;
        slot = KVW_PAD_ID;
    }
    if (report && lane == 0) raise_flags(a.err_flag, flags);
    if (slot < 0 || !real) return;
    if (ROWS && PLANES == 1) {  // large writes read a row once its slot is known
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) {
            const int64_t off = min(lane_off + ch * kSliceBytes, bpt - 16) - lane_off;
#pragma unroll
            for (int q = 0; q < PLANES; ++q)
                row[q][ch] = load16<KVW_NT_LOADS>(src[q] + l0 * c.kv_layer_stride + off);
        }
    }

    uint8_t *dst[PLANES];  // wave-uniform rows; each lane stores at lane_off within them
#pragma unroll
    for (int q = 0; q < PLANES; ++q) dst[q] = (plane0 + q ? c.v_cache : c.k_cache) + slot * bpt;
    // Large writes (one wave per token and plane) store through to memory, as the
    // scatter does.  Small ones (one wave per token, a single round of waves on the
    // GPU) keep the stores in L2: there the write-through traffic delayed the other
    // waves' cold metadata loads (range lookup on the 8,192-token mixed batch: 13.2
    // against 12.3 us of kernel time).
    const auto store_row = [](uint8_t *base, uint32_t off, u32x4 v) {
        if constexpr (PLANES == 1) store16_through(base, off, v);
        else store16<KVW_NT_STORES>(base + off, v);
    };
    for (int l = l0; l < l1; ++l) {
        const int64_t src_l = l * c.kv_layer_stride;
        const int64_t dst_l = static_cast<int64_t>(l) * c.rows_per_layer * bpt;  // l*B*T rows
        for (int64_t seg = 0; seg < bpt; seg += CH * kSliceBytes) {
            if (l != l0 || seg != 0) {
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    if (seg + lane_off + ch * kSliceBytes < bpt)
#pragma unroll
                        for (int q = 0; q < PLANES; ++q)
                            row[q][ch] = load16<KVW_NT_LOADS>(src[q] + src_l + seg + ch * kSliceBytes);
            }
#pragma unroll
            for (int ch = 0; ch < CH; ++ch)
                if (seg + lane_off + ch * kSliceBytes < bpt)
#pragma unroll
                    for (int q = 0; q < PLANES; ++q)
                        store_row(dst[q] + dst_l, static_cast<uint32_t>(lane_off + seg + ch * kSliceBytes),
                                  row[q][ch]);
        }
    }
}

// out[r][q] for q = i*k + j: ids[r][i]*k + j while i < count[r], else 0.
__global__ __launch_bounds__(kBlockThreads) void expand_blocks_kernel(
    const int32_t *ids, const int32_t *counts, int32_t rows, int32_t in_stride, int32_t k,
    int32_t *out, int32_t out_stride, int32_t *counts_out, int32_t *err_flag)
{
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    if (idx >= static_cast<int64_t>(rows) * out_stride) return;
    const int32_t r = static_cast<int32_t>(idx / out_stride);
    const int32_t q = static_cast<int32_t>(idx - static_cast<int64_t>(r) * out_stride);
    uint32_t flags = 0;
    expand_entry(ids, counts, in_stride, k, out, out_stride, counts_out, r, q, flags);
    raise_flags(err_flag, flags);
}

// (start, len, cum) -> (start*k, len*k, cum*k) for i < num_ranges[r]; 0 past it.
__global__ __launch_bounds__(kBlockThreads) void expand_ranges_kernel(
    const int32_t *start, const int32_t *len, const int32_t *cum, const int32_t *num_ranges,
    int32_t rows, int32_t stride, int32_t k, int32_t *o_start, int32_t *o_len, int32_t *o_cum,
    int32_t *o_num, int32_t *err_flag)
{
    const int32_t width = stride > 0 ? stride : 1;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    if (idx >= static_cast<int64_t>(rows) * width) return;
    const int32_t r = static_cast<int32_t>(idx / width);
    const int32_t i = static_cast<int32_t>(idx - static_cast<int64_t>(r) * width);
    uint32_t flags = 0;
    const int64_t n = clamp_count(num_ranges[r], stride, flags);
    if (i == 0) o_num[r] = static_cast<int32_t>(n);
    else flags = 0;  // the count is reported once per row
    if (i < stride) {
        const int64_t q = static_cast<int64_t>(r) * stride + i;
        int32_t s = 0, l = 0, c = 0;
        if (i < n) {
            if (expandable(start[q], k) && expandable(len[q], k) && expandable(cum[q], k)) {
                s = start[q] * k;
                l = len[q] * k;
                c = cum[q] * k;
            } else {
                flags |= KVW_FLAG_BAD_BLOCK;
            }
        }
        o_start[q] = s;
        o_len[q] = l;
        o_cum[q] = c;
    }
    raise_flags(err_flag, flags);
}

// Block table filled from range descriptors (see fill_table_row); the
// workgroups of a launch column share one row, looped over blockIdx.y.
__global__ __launch_bounds__(kBlockThreads) void fill_table_kernel(
    const int32_t *start, const int32_t *len, const int32_t *cum, const int32_t *num_ranges,
    int32_t rows, int32_t range_stride, int32_t k, int32_t *out, int32_t out_stride,
    int32_t *counts_out, int32_t *err_flag)
{
    const int64_t q = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    asm("" : "+s"(rows) : "s"(err_flag));  // both argument lines in one round trip
    for (int32_t r = blockIdx.y; r < rows; r += gridDim.y) {  // uniform over the workgroup
        uint32_t flags = 0;
        fill_table_row(start, len, cum, num_ranges, range_stride, k, out, out_stride, counts_out,
                       r, q, flags);
        raise_flags(err_flag, flags);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
using kvw_detail::check_cp;
using kvw_detail::fail;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kvw_status launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return KVW_OK;
}

unsigned grid_for(int64_t items, int64_t per_block)
{
    return static_cast<unsigned>((items + per_block - 1) / per_block);
}

#define KVW_REQUIRE(cond, ...)                                      \
    do {                                                            \
        if (!(cond)) return fail(KVW_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

// Checks shared by both slot-mapping calls and the fused write.
kvw_status check_mapping_common(const char *fn, const int32_t *qsl, int32_t num_reqs,
                                const int64_t *positions, int64_t max_num_tokens,
                                int32_t block_size, const int32_t *err_flag)
{
    KVW_REQUIRE(max_num_tokens >= 0 && max_num_tokens <= INT32_MAX,
                "%s: max_num_tokens %lld outside [0, 2^31)", fn, (long long)max_num_tokens);
    KVW_REQUIRE(num_reqs >= 0, "%s: num_reqs %d is negative", fn, num_reqs);
    KVW_REQUIRE(block_size > 0, "%s: block_size %d must be positive", fn, block_size);
    KVW_REQUIRE(!err_flag || aligned(err_flag, 4), "%s: err_flag misaligned", fn);
    if (max_num_tokens == 0) return KVW_OK;
    KVW_REQUIRE(qsl && aligned(qsl, 4), "%s: query_start_loc is NULL or misaligned", fn);
    KVW_REQUIRE(positions && aligned(positions, 8), "%s: positions is NULL or misaligned", fn);
    return KVW_OK;
}

kvw_status check_paged(const char *fn, int32_t num_reqs, const int32_t *block_table,
                       int32_t stride, const int32_t *num_blocks_per_req)
{
    KVW_REQUIRE(stride >= 0, "%s: block_table_stride %d is negative", fn, stride);
    KVW_REQUIRE(!(num_reqs > 0 && stride > 0) || block_table, "%s: block_table is NULL", fn);
    KVW_REQUIRE(!block_table || aligned(block_table, 4), "%s: block_table misaligned", fn);
    KVW_REQUIRE(!num_blocks_per_req || aligned(num_blocks_per_req, 4),
                "%s: num_blocks_per_req misaligned", fn);
    return KVW_OK;
}

kvw_status check_ranges(const char *fn, int32_t num_reqs, const int32_t *start, const int32_t *len,
                        const int32_t *cum, const int32_t *num_ranges, int32_t stride)
{
    KVW_REQUIRE(stride >= 0, "%s: range_stride %d is negative", fn, stride);
    if (stride > KVW_MAX_RANGE_STRIDE)
        return fail(KVW_ERR_RANGE_CAP, "%s: range_stride %d exceeds the cap of %d", fn, stride,
                    KVW_MAX_RANGE_STRIDE);
    if (num_reqs > 0) {
        KVW_REQUIRE(start && len && cum && num_ranges, "%s: a range descriptor array is NULL", fn);
        KVW_REQUIRE(aligned(start, 4) && aligned(len, 4) && aligned(cum, 4) && aligned(num_ranges, 4),
                    "%s: a range descriptor array is misaligned", fn);
    }
    return KVW_OK;
}

// Context-parallel parameters: world 0 means none; from 1 up the rank must lie
// in [0, world) and the interleave size divide block_size.
MapArgs make_map_args(const int32_t *qsl, int32_t num_reqs, const int64_t *positions,
                      int64_t max_num_tokens, int32_t block_size, int32_t cp_world,
                      int32_t cp_rank, int32_t cp_interleave, int32_t *err_flag)
{
    MapArgs a{};
    a.qsl = qsl;
    a.num_reqs = num_reqs;
    a.positions = positions;
    a.max_num_tokens = max_num_tokens;
    a.block_size = block_size;
    a.cp_world = cp_world > 1 ? cp_world : 1;
    a.cp_rank = cp_world > 1 ? cp_rank : 0;
    a.cp_interleave = cp_world > 1 ? cp_interleave : 1;
    a.err_flag = err_flag;
    return a;
}

// Workgroups that write the optional attention-side table next to the slots.
unsigned table_blocks(int mode, const MapArgs &a, int threads, uint32_t *per_row)
{
    *per_row = 0;
    if (!a.table_out || a.num_reqs == 0) return 0;
    if (mode == kPaged) return grid_for(static_cast<int64_t>(a.num_reqs) * a.table_out_stride, threads);
    *per_row = a.table_out_stride > 0 ? grid_for(a.table_out_stride, threads) : 1u;
    return *per_row * static_cast<unsigned>(a.num_reqs);
}

void launch_slot_mapping(int mode, const MapArgs &args, hipStream_t s)
{
    MapArgs a = args;
    a.slot_blocks = grid_for(a.max_num_tokens, kSlotThreads);
    const dim3 grid(a.slot_blocks + table_blocks(mode, a, kSlotThreads, &a.table_blocks_per_row));
    if (mode == kPaged) hipLaunchKernelGGL(slot_mapping_kernel<kPaged>, grid, dim3(kSlotThreads), 0, s, a);
    else hipLaunchKernelGGL(slot_mapping_kernel<kRanges>, grid, dim3(kSlotThreads), 0, s, a);
}

// The attention-side table on its own (the one-kernel schedule has no
// slot-mapping launch to ride on).
void launch_table(int mode, const MapArgs &a, hipStream_t s)
{
    uint32_t per_row;
    const unsigned blocks = table_blocks(mode, a, kBlockThreads, &per_row);
    if (!blocks) return;
    if (mode == kPaged) {
        hipLaunchKernelGGL(expand_blocks_kernel, dim3(blocks), dim3(kBlockThreads), 0, s, a.block_table,
                           a.num_blocks_per_req, a.num_reqs, a.table_stride, a.table_k, a.table_out,
                           a.table_out_stride, a.table_counts_out, a.err_flag);
    } else {
        const unsigned rows = static_cast<unsigned>(a.num_reqs) < kMaxGridY ? a.num_reqs : kMaxGridY;
        hipLaunchKernelGGL(fill_table_kernel, dim3(per_row, rows), dim3(kBlockThreads), 0, s,
                           a.range_start, a.range_len, a.range_cum, a.num_ranges, a.num_reqs,
                           a.range_stride, a.table_k, a.table_out, a.table_out_stride,
                           a.table_counts_out, a.err_flag);
    }
}

template <int MODE, int PLANES>
void launch_fused_shape(const MapArgs &a, const CopyArgs &c, unsigned groups, hipStream_t s)
{
    const dim3 grid(grid_for(PLANES == 2 ? a.max_num_tokens : 2 * a.max_num_tokens, kFusedWaves), groups);
    const dim3 block(kFusedThreads);
    if (c.num_layers == 0) {  // slots only: no row is read
        hipLaunchKernelGGL((kv_write_fused_kernel<MODE, 1, PLANES, false>), grid, block, 0, s, a, c);
        return;
    }
    switch (c.slices_per_row) {
    case 1: hipLaunchKernelGGL((kv_write_fused_kernel<MODE, 1, PLANES, true>), grid, block, 0, s, a, c); break;
    case 2: hipLaunchKernelGGL((kv_write_fused_kernel<MODE, 2, PLANES, true>), grid, block, 0, s, a, c); break;
    case 3: hipLaunchKernelGGL((kv_write_fused_kernel<MODE, 3, PLANES, true>), grid, block, 0, s, a, c); break;
    default: hipLaunchKernelGGL((kv_write_fused_kernel<MODE, kMaxSlicesPerLane, PLANES, true>), grid, block, 0, s, a, c);
    }
}

// One wave per token for writes of up to KVW_TOKEN_WAVE_MAX_ROWS token rows,
// one per (token, plane) above.
template <int MODE>
void launch_fused(const MapArgs &a, const CopyArgs &c, unsigned groups, hipStream_t s)
{
    if (a.max_num_tokens * static_cast<int64_t>(c.num_layers) <= KVW_TOKEN_WAVE_MAX_ROWS)
        launch_fused_shape<MODE, 2>(a, c, groups, s);
    else
        launch_fused_shape<MODE, 1>(a, c, groups, s);
}

}  // namespace

extern "C" {

int32_t kvw_abi_version(void) { return KVW_ABI_VERSION; }

size_t kvw_kv_write_args_size(void) { return sizeof(kvw_kv_write_args); }

kvw_status kvw_slot_mapping_paged(const int32_t *query_start_loc, int32_t num_reqs,
                                  const int64_t *positions, int64_t max_num_tokens,
                                  const int32_t *block_table, int32_t block_table_stride,
                                  const int32_t *num_blocks_per_req, int32_t block_size,
                                  int32_t cp_world_size, int32_t cp_rank,
                                  int32_t cp_interleave_size, int64_t *slot_mapping,
                                  int32_t *err_flag, void *stream)
{
    const char *fn = "kvw_slot_mapping_paged";
    kvw_status st = check_mapping_common(fn, query_start_loc, num_reqs, positions, max_num_tokens,
                                         block_size, err_flag);
    if (st != KVW_OK) return st;
    if ((st = check_cp(fn, block_size, cp_world_size, cp_rank, cp_interleave_size)) != KVW_OK)
        return st;
    if ((st = check_paged(fn, num_reqs, block_table, block_table_stride, num_blocks_per_req)) != KVW_OK)
        return st;
    if (max_num_tokens == 0) return KVW_OK;
    KVW_REQUIRE(slot_mapping && aligned(slot_mapping, 8), "%s: slot_mapping is NULL or misaligned", fn);
    MapArgs a = make_map_args(query_start_loc, num_reqs, positions, max_num_tokens, block_size,
                              cp_world_size, cp_rank, cp_interleave_size, err_flag);
    a.block_table = block_table;
    a.table_stride = block_table_stride;
    a.num_blocks_per_req = num_blocks_per_req;
    a.slots_out = slot_mapping;
    launch_slot_mapping(kPaged, a, reinterpret_cast<hipStream_t>(stream));
    return launched(fn);
}

kvw_status kvw_slot_mapping_ranges(const int32_t *query_start_loc, int32_t num_reqs,
                                   const int64_t *positions, int64_t max_num_tokens,
                                   const int32_t *range_start, const int32_t *range_len,
                                   const int32_t *range_cum, const int32_t *num_ranges,
                                   int32_t range_stride, int32_t block_size,
                                   int32_t cp_world_size, int32_t cp_rank,
                                   int32_t cp_interleave_size, int64_t *slot_mapping,
                                   int32_t *err_flag, void *stream)
{
    const char *fn = "kvw_slot_mapping_ranges";
    kvw_status st = check_mapping_common(fn, query_start_loc, num_reqs, positions, max_num_tokens,
                                         block_size, err_flag);
    if (st != KVW_OK) return st;
    if ((st = check_cp(fn, block_size, cp_world_size, cp_rank, cp_interleave_size)) != KVW_OK)
        return st;
    if ((st = check_ranges(fn, num_reqs, range_start, range_len, range_cum, num_ranges,
                           range_stride)) != KVW_OK)
        return st;
    if (max_num_tokens == 0) return KVW_OK;
    KVW_REQUIRE(slot_mapping && aligned(slot_mapping, 8), "%s: slot_mapping is NULL or misaligned", fn);
    MapArgs a = make_map_args(query_start_loc, num_reqs, positions, max_num_tokens, block_size,
                              cp_world_size, cp_rank, cp_interleave_size, err_flag);
    a.range_start = range_start;
    a.range_len = range_len;
    a.range_cum = range_cum;
    a.num_ranges = num_ranges;
    a.range_stride = range_stride;
    a.slots_out = slot_mapping;
    launch_slot_mapping(kRanges, a, reinterpret_cast<hipStream_t>(stream));
    return launched(fn);
}

kvw_status kvw_map_to_kernel_blocks(const int32_t *ids, const int32_t *counts, int32_t rows,
                                    int32_t in_stride, int32_t block_size,
                                    int32_t kernel_block_size, int32_t *out, int32_t out_stride,
                                    int32_t *err_flag, void *stream)
{
    const char *fn = "kvw_map_to_kernel_blocks";
    KVW_REQUIRE(block_size > 0 && kernel_block_size > 0 && block_size % kernel_block_size == 0,
                "%s: kernel block size %d does not divide block size %d", fn, kernel_block_size,
                block_size);
    const int64_t k = block_size / kernel_block_size;
    KVW_REQUIRE(rows >= 0 && in_stride >= 0, "%s: negative rows or in_stride", fn);
    KVW_REQUIRE(out_stride >= static_cast<int64_t>(in_stride) * k,
                "%s: out_stride %d below in_stride*k = %lld", fn, out_stride,
                (long long)(in_stride * k));
    KVW_REQUIRE(!err_flag || aligned(err_flag, 4), "%s: err_flag misaligned", fn);
    const int64_t total = static_cast<int64_t>(rows) * out_stride;
    if (total == 0) return KVW_OK;
    KVW_REQUIRE(total <= INT32_MAX, "%s: rows*out_stride too large", fn);
    KVW_REQUIRE(out && aligned(out, 4), "%s: out is NULL or misaligned", fn);
    KVW_REQUIRE(in_stride == 0 || (ids && aligned(ids, 4)), "%s: ids is NULL or misaligned", fn);
    KVW_REQUIRE(!counts || aligned(counts, 4), "%s: counts misaligned", fn);
    hipLaunchKernelGGL(expand_blocks_kernel, dim3(grid_for(total, kBlockThreads)), dim3(kBlockThreads),
                       0, reinterpret_cast<hipStream_t>(stream), ids, counts, rows, in_stride,
                       static_cast<int32_t>(k), out, out_stride, nullptr, err_flag);
    return launched(fn);
}

kvw_status kvw_map_ranges_to_kernel_blocks(const int32_t *range_start, const int32_t *range_len,
                                           const int32_t *range_cum, const int32_t *num_ranges,
                                           int32_t rows, int32_t range_stride, int32_t block_size,
                                           int32_t kernel_block_size, int32_t *out_start,
                                           int32_t *out_len, int32_t *out_cum,
                                           int32_t *out_num_ranges, int32_t *err_flag,
                                           void *stream)
{
    const char *fn = "kvw_map_ranges_to_kernel_blocks";
    KVW_REQUIRE(block_size > 0 && kernel_block_size > 0 && block_size % kernel_block_size == 0,
                "%s: kernel block size %d does not divide block size %d", fn, kernel_block_size,
                block_size);
    const int32_t k = block_size / kernel_block_size;
    KVW_REQUIRE(rows >= 0 && range_stride >= 0, "%s: negative rows or range_stride", fn);
    if (range_stride > KVW_MAX_RANGE_STRIDE)
        return fail(KVW_ERR_RANGE_CAP, "%s: range_stride %d exceeds the cap of %d", fn, range_stride,
                    KVW_MAX_RANGE_STRIDE);
    KVW_REQUIRE(!err_flag || aligned(err_flag, 4), "%s: err_flag misaligned", fn);
    if (rows == 0) return KVW_OK;
    const int32_t *ins[] = {range_start, range_len, range_cum};
    const int32_t *outs[] = {out_start, out_len, out_cum};
    for (int i = 0; i < 3; ++i) {
        KVW_REQUIRE(range_stride == 0 || (ins[i] && aligned(ins[i], 4)),
                    "%s: an input descriptor array is NULL or misaligned", fn);
        KVW_REQUIRE(range_stride == 0 || (outs[i] && aligned(outs[i], 4)),
                    "%s: an output descriptor array is NULL or misaligned", fn);
    }
    KVW_REQUIRE(num_ranges && aligned(num_ranges, 4) && out_num_ranges && aligned(out_num_ranges, 4),
                "%s: num_ranges or out_num_ranges is NULL or misaligned", fn);
    const int64_t total = static_cast<int64_t>(rows) * (range_stride > 0 ? range_stride : 1);
    KVW_REQUIRE(total <= INT32_MAX, "%s: rows*range_stride too large", fn);
    hipLaunchKernelGGL(expand_ranges_kernel, dim3(grid_for(total, kBlockThreads)), dim3(kBlockThreads),
                       0, reinterpret_cast<hipStream_t>(stream), range_start, range_len, range_cum,
                       num_ranges, rows, range_stride, k, out_start, out_len, out_cum,
                       out_num_ranges, err_flag);
    return launched(fn);
}

kvw_status kvw_ranges_to_block_table(const int32_t *range_start, const int32_t *range_len,
                                     const int32_t *range_cum, const int32_t *num_ranges,
                                     int32_t rows, int32_t range_stride, int32_t block_size,
                                     int32_t kernel_block_size, int32_t *block_table,
                                     int32_t block_table_stride, int32_t *num_blocks_per_req,
                                     int32_t *err_flag, void *stream)
{
    const char *fn = "kvw_ranges_to_block_table";
    KVW_REQUIRE(block_size > 0 && kernel_block_size > 0 && block_size % kernel_block_size == 0,
                "%s: kernel block size %d does not divide block size %d", fn, kernel_block_size,
                block_size);
    const int32_t k = block_size / kernel_block_size;
    KVW_REQUIRE(rows >= 0 && range_stride >= 0 && block_table_stride >= 0,
                "%s: negative rows, range_stride or block_table_stride", fn);
    if (range_stride > KVW_MAX_RANGE_STRIDE)
        return fail(KVW_ERR_RANGE_CAP, "%s: range_stride %d exceeds the cap of %d", fn, range_stride,
                    KVW_MAX_RANGE_STRIDE);
    KVW_REQUIRE(!err_flag || aligned(err_flag, 4), "%s: err_flag misaligned", fn);
    if (rows == 0) return KVW_OK;
    KVW_REQUIRE(num_ranges && aligned(num_ranges, 4), "%s: num_ranges is NULL or misaligned", fn);
    const int32_t *ins[] = {range_start, range_len, range_cum};
    for (const int32_t *p : ins)
        KVW_REQUIRE(range_stride == 0 || (p && aligned(p, 4)),
                    "%s: a range descriptor array is NULL or misaligned", fn);
    KVW_REQUIRE(block_table_stride == 0 || (block_table && aligned(block_table, 4)),
                "%s: block_table is NULL or misaligned", fn);
    KVW_REQUIRE(!num_blocks_per_req || aligned(num_blocks_per_req, 4),
                "%s: num_blocks_per_req misaligned", fn);
    // at least one workgroup per row: its first lane writes the count and the row's flags
    const dim3 grid(block_table_stride > 0 ? grid_for(block_table_stride, kBlockThreads) : 1u,
                    static_cast<unsigned>(rows) < kMaxGridY ? static_cast<unsigned>(rows) : kMaxGridY);
    hipLaunchKernelGGL(fill_table_kernel, grid, dim3(kBlockThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), range_start, range_len, range_cum,
                       num_ranges, rows, range_stride, k, block_table, block_table_stride,
                       num_blocks_per_req, err_flag);
    return launched(fn);
}

kvw_status kvw_kv_write(const kvw_kv_write_args *args, void *stream)
{
    const char *fn = "kvw_kv_write";
    KVW_REQUIRE(args, "%s: args is NULL", fn);
    const kvw_kv_write_args &g = *args;
    KVW_REQUIRE(g.mode == KVW_SLOTS_PRECOMPUTED || g.mode == KVW_SLOTS_PAGED || g.mode == KVW_SLOTS_RANGES,
                "%s: unknown mode %d", fn, g.mode);
    KVW_REQUIRE(g.max_num_tokens >= 0 && g.max_num_tokens <= INT32_MAX,
                "%s: max_num_tokens %lld outside [0, 2^31)", fn, (long long)g.max_num_tokens);
    KVW_REQUIRE(g.num_layers >= 0, "%s: num_layers is negative", fn);
    KVW_REQUIRE(g.num_blocks >= 0, "%s: num_blocks is negative", fn);
    KVW_REQUIRE(g.block_size > 0, "%s: block_size %d must be positive", fn, g.block_size);
    KVW_REQUIRE(g.bytes_per_token > 0 && g.bytes_per_token % 16 == 0 && g.bytes_per_token <= INT32_MAX,
                "%s: bytes_per_token %lld must be a positive multiple of 16 below 2^31", fn,
                (long long)g.bytes_per_token);
    KVW_REQUIRE(g.num_blocks <= INT64_MAX / g.block_size, "%s: num_blocks*block_size overflows", fn);
    const int64_t rows_per_layer = g.num_blocks * g.block_size;
    KVW_REQUIRE(g.num_layers == 0 || rows_per_layer <= INT64_MAX / g.num_layers / g.bytes_per_token,
                "%s: cache size overflows int64", fn);
    KVW_REQUIRE(!g.err_flag || aligned(g.err_flag, 4), "%s: err_flag misaligned", fn);

    kvw_status st = KVW_OK;
    const bool fused = g.mode != KVW_SLOTS_PRECOMPUTED;
    if (fused) {
        st = check_mapping_common(fn, g.query_start_loc, g.num_reqs, g.positions, g.max_num_tokens,
                                  g.block_size, g.err_flag);
        if (st != KVW_OK) return st;
        st = (g.mode == KVW_SLOTS_PAGED)
                 ? check_paged(fn, g.num_reqs, g.block_table, g.block_table_stride, g.num_blocks_per_req)
                 : check_ranges(fn, g.num_reqs, g.range_start, g.range_len, g.range_cum, g.num_ranges,
                                g.range_stride);
        if (st != KVW_OK) return st;
        st = check_cp(fn, g.block_size, g.cp_world_size, g.cp_rank, g.cp_interleave_size);
        if (st != KVW_OK) return st;
        KVW_REQUIRE(!g.slot_mapping_out || aligned(g.slot_mapping_out, 8),
                    "%s: slot_mapping_out misaligned", fn);
        KVW_REQUIRE(g.schedule == KVW_SCHEDULE_AUTO || g.schedule == KVW_SCHEDULE_TWO_KERNELS ||
                        g.schedule == KVW_SCHEDULE_ONE_KERNEL,
                    "%s: unknown schedule %d", fn, g.schedule);
        KVW_REQUIRE(g.schedule != KVW_SCHEDULE_TWO_KERNELS || g.slot_mapping_out,
                    "%s: the two-kernel schedule needs slot_mapping_out", fn);
        if (g.table_out) {
            KVW_REQUIRE(aligned(g.table_out, 4) && (!g.table_counts_out || aligned(g.table_counts_out, 4)),
                        "%s: table_out or table_counts_out misaligned", fn);
            KVW_REQUIRE(g.table_block_size > 0 && g.block_size % g.table_block_size == 0,
                        "%s: table_block_size %d does not divide block_size %d", fn,
                        g.table_block_size, g.block_size);
            KVW_REQUIRE(g.table_out_stride > 0, "%s: table_out_stride must be positive", fn);
            KVW_REQUIRE(g.mode != KVW_SLOTS_PAGED ||
                            g.table_out_stride >= static_cast<int64_t>(g.block_table_stride) *
                                                      (g.block_size / g.table_block_size),
                        "%s: table_out_stride below block_table_stride * k", fn);
            KVW_REQUIRE(static_cast<int64_t>(g.num_reqs) * g.table_out_stride <= INT32_MAX,
                        "%s: num_reqs * table_out_stride too large", fn);
        }
    } else {
        KVW_REQUIRE(!g.table_out, "%s: table_out needs the paged or range mode", fn);
    }
    if (g.max_num_tokens == 0) {  // no token rows; the attention-side table is still written
        if (fused && g.table_out) {
            MapArgs t = make_map_args(g.query_start_loc, g.num_reqs, g.positions, 0, g.block_size, 0,
                                      0, 0, g.err_flag);
            t.block_table = g.block_table;
            t.table_stride = g.block_table_stride;
            t.num_blocks_per_req = g.num_blocks_per_req;
            t.range_start = g.range_start;
            t.range_len = g.range_len;
            t.range_cum = g.range_cum;
            t.num_ranges = g.num_ranges;
            t.range_stride = g.range_stride;
            t.table_out = g.table_out;
            t.table_counts_out = g.table_counts_out;
            t.table_out_stride = g.table_out_stride;
            t.table_k = g.block_size / g.table_block_size;
            launch_table(g.mode, t, reinterpret_cast<hipStream_t>(stream));
            return launched(fn);
        }
        return KVW_OK;
    }
    if (!fused)
        KVW_REQUIRE(g.slot_mapping_in && aligned(g.slot_mapping_in, 8),
                    "%s: slot_mapping_in is NULL or misaligned", fn);
    if (g.num_layers > 0) {
        KVW_REQUIRE(g.key && g.value && g.k_cache && g.v_cache, "%s: a K/V or cache pointer is NULL", fn);
        KVW_REQUIRE(aligned(g.key, 16) && aligned(g.value, 16) && aligned(g.k_cache, 16) &&
                        aligned(g.v_cache, 16),
                    "%s: K/V and cache pointers must be 16-byte aligned", fn);
        KVW_REQUIRE(g.kv_layer_stride >= 0 && g.kv_token_stride >= 0 && g.kv_layer_stride % 16 == 0 &&
                        g.kv_token_stride % 16 == 0,
                    "%s: K/V strides must be non-negative multiples of 16", fn);
    }

    CopyArgs c{};
    c.key = static_cast<const uint8_t *>(g.key);
    c.value = static_cast<const uint8_t *>(g.value);
    c.k_cache = static_cast<uint8_t *>(g.k_cache);
    c.v_cache = static_cast<uint8_t *>(g.v_cache);
    c.kv_layer_stride = g.kv_layer_stride;
    c.kv_token_stride = g.kv_token_stride;
    c.rows_per_layer = rows_per_layer;
    c.bytes_per_token = g.bytes_per_token;
    c.max_num_tokens = g.max_num_tokens;
    c.num_layers = g.num_layers;
    c.layers_per_wave = 1;
    c.slices_per_row = static_cast<uint32_t>((g.bytes_per_token + kSliceBytes - 1) / kSliceBytes);
    c.items_per_token = 2 * c.slices_per_row;
    c.items_log2 = -1;
    for (int b = 0; b < 31; ++b)
        if (c.items_per_token == (1u << b)) c.items_log2 = b;
    const unsigned layer_grid =
        g.num_layers < 1 ? 1u : (static_cast<unsigned>(g.num_layers) < kMaxGridY ? g.num_layers : kMaxGridY);
    // Scatter shape.  Rows under 1 KiB: a wave copies one plane of several
    // tokens.  Context parallelism: a wave takes one slice of up to four
    // consecutive tokens, most of which may be another rank's.
    const bool small_rows = g.bytes_per_token < kSliceBytes;
    const int32_t cp = fused && g.cp_world_size > 1 ? g.cp_world_size : 1;
    const int tpw = small_rows ? 1 : (cp >= 4 ? 4 : (cp >= 2 ? 2 : 1));
    int64_t scatter_waves;
    if (small_rows) {
        c.lanes_per_row = static_cast<uint32_t>(g.bytes_per_token / 16);
        c.rows_per_wave = static_cast<uint32_t>(kWave) / c.lanes_per_row;
        scatter_waves = 2 * ((g.max_num_tokens + c.rows_per_wave - 1) / c.rows_per_wave);
    } else {
        scatter_waves = (g.max_num_tokens + tpw - 1) / tpw * static_cast<int64_t>(c.items_per_token);
    }
    const int64_t scatter_blocks = (scatter_waves + kScatterWaves - 1) / kScatterWaves;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    MapArgs a = make_map_args(g.query_start_loc, g.num_reqs, g.positions, g.max_num_tokens,
                              g.block_size, fused ? g.cp_world_size : 0, g.cp_rank,
                              g.cp_interleave_size, g.err_flag);
    a.block_table = g.block_table;
    a.table_stride = g.block_table_stride;
    a.num_blocks_per_req = g.num_blocks_per_req;
    a.range_start = g.range_start;
    a.range_len = g.range_len;
    a.range_cum = g.range_cum;
    a.num_ranges = g.num_ranges;
    a.range_stride = g.range_stride;
    a.slots_out = g.slot_mapping_out;
    if (fused && g.table_out) {
        a.table_out = g.table_out;
        a.table_counts_out = g.table_counts_out;
        a.table_out_stride = g.table_out_stride;
        a.table_k = g.block_size / g.table_block_size;
    }

    const bool two_pass =
        !fused || (g.slot_mapping_out != nullptr &&
                   (g.schedule == KVW_SCHEDULE_TWO_KERNELS ||
                    (g.schedule == KVW_SCHEDULE_AUTO &&
                     g.max_num_tokens * static_cast<int64_t>(g.num_layers) >= KVW_TWO_KERNEL_MIN_ROWS)));
    if (two_pass && g.num_layers > 0 && scatter_blocks > static_cast<int64_t>(kMaxGridX))
        return fail(KVW_ERR_UNSUPPORTED, "%s: %lld token rows of %lld bytes exceed one launch", fn,
                    (long long)g.max_num_tokens, (long long)g.bytes_per_token);
    if (two_pass) {
        // slots (unless given), then the slice-granular scatter that reads them
        if (fused) {
            launch_slot_mapping(g.mode, a, s);
            if (kvw_status e = launched(fn); e != KVW_OK) return e;
        }
        if (g.num_layers == 0) return KVW_OK;
        const int64_t *slots = fused ? g.slot_mapping_out : g.slot_mapping_in;
        const dim3 grid(static_cast<unsigned>(scatter_blocks), layer_grid);
        if (small_rows && cp > 1)
            hipLaunchKernelGGL(kv_scatter_small_kernel<false>, grid, dim3(kScatterThreads), 0, s,
                               slots, c, g.err_flag);
        else if (small_rows)
            hipLaunchKernelGGL(kv_scatter_small_kernel<true>, grid, dim3(kScatterThreads), 0, s,
                               slots, c, g.err_flag);
        else if (tpw == 4)
            hipLaunchKernelGGL(kv_scatter_kernel<4>, grid, dim3(kScatterThreads), 0, s, slots, c,
                               g.err_flag);
        else if (tpw == 2)
            hipLaunchKernelGGL(kv_scatter_kernel<2>, grid, dim3(kScatterThreads), 0, s, slots, c,
                               g.err_flag);
        else
            hipLaunchKernelGGL(kv_scatter_kernel<1>, grid, dim3(kScatterThreads), 0, s, slots, c,
                               g.err_flag);
        return launched(fn);
    }
    // fused mode without a slot-mapping output: one kernel, one wave per token
    // (after the attention-side table, if asked for, in a launch of its own)
    launch_table(g.mode, a, s);
    if (g.num_layers > static_cast<int32_t>(kMaxGridY)) c.layers_per_wave = g.num_layers / kMaxGridY + 1;
    const unsigned groups =
        g.num_layers < 1 ? 1u : static_cast<unsigned>((g.num_layers + c.layers_per_wave - 1) / c.layers_per_wave);
    if (g.mode == KVW_SLOTS_PAGED) launch_fused<kPaged>(a, c, groups, s);
    else launch_fused<kRanges>(a, c, groups, s);
    return launched(fn);
}

}  // extern "C"
