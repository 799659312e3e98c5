// Device helpers shared by the kernels of libkvw.so (kvw.hip, decode_attention.hip):
// wave constants, sticky flags, count clamping, 16-byte memory access and the
// wavefront-level search.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvw.h"

namespace {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void raise_flags(int32_t *err, uint32_t flags)
{
    if (err && flags) atomicOr(err, static_cast<int>(flags));
}

__device__ __forceinline__ int64_t clamp_count(int32_t c, int32_t stride, uint32_t &flags)
{
    if (c < 0) { flags |= KVW_FLAG_COUNT; return 0; }
    if (c > stride) { flags |= KVW_FLAG_COUNT; return stride; }
    return c;
}

__device__ __forceinline__ bool expandable(int64_t id, int64_t k)
{
    return id >= 0 && id * k + (k - 1) <= INT32_MAX;
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const uint8_t *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else return *reinterpret_cast<const u32x4 *>(p);
}

template <bool NT>
__device__ __forceinline__ void store16(uint8_t *p, u32x4 v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    else *reinterpret_cast<u32x4 *>(p) = v;
}

// 16 bytes to base + off for a wave-uniform base (off: the lane's offset, below
// 2^31), stored at device scope and non-temporal: the line is written through
// the XCD's L2 to memory rather than held there dirty, and streamed.  A buffer
// store with the cache-policy bits (SC1 | NT), so the compiler sees the store.
// Measured on the K/V scatter of 2 KiB rows, each call writing lines the call
// before did not: 3-4% faster than a non-temporal store that L2 holds, at every
// destination layout from contiguous to one 64 KiB block per run.
constexpr int kCpolNt = 2, kCpolSc1 = 16;
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw (untyped) buffer access on gfx9-family parts

__device__ __forceinline__ void store16_through(uint8_t *base, uint32_t off, u32x4 v)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, kBufferRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, kCpolSc1 | kCpolNt);
}

// 16 bytes to p (any lane's own address) at device scope, without the
// non-temporal hint: written through L2 and left to the memory-side cache.  For
// rows under 1 KiB, where a wave's stores land in several rows: measured with
// each call writing lines the call before did not, 5-6% faster than a
// non-temporal store at 512 B rows and up to 11% at 256 B (fragmented cache).
// A global store in assembly, since no builtin sets SC1 on a per-lane address;
// the trailing nop gives the wait state that a later vector write to the store's
// data registers needs, which the compiler does not track for an assembly store.
__device__ __forceinline__ void store16_device(uint8_t *p, u32x4 v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// ---- wavefront-level search -------------------------------------------------
// The 64 lanes of a wave hold 64 evenly spaced entries of a sorted array (one
// vector load) and each lane ranks its own key among them with a 6-step
// ds_bpermute search, which touches no memory.  A second load of the window
// that holds every lane's answer finishes the search, so two dependent loads
// replace the ~log2(n) of a per-lane binary search: the request of a token is
// found in query_start_loc this way, and the run of a position in range_cum
// (the range descriptors are loaded once for the consecutive positions of a
// wave, not once per position).

// Number of lanes whose sample is <= x; samples are non-decreasing over the
// lanes and lanes without a sample hold INT64_MAX.  Every lane runs every
// shuffle (a permute that reads an inactive lane gets no defined value).
__device__ __forceinline__ int wave_rank(int64_t sample, int64_t x)
{
    const bool all = __shfl(sample, kWave - 1) <= x;
    int cnt = 0;
#pragma unroll
    for (int b = kWave / 2; b >= 1; b >>= 1) {
        const int64_t probe = __shfl(sample, cnt + b - 1);
        cnt += probe <= x ? b : 0;
    }
    return all ? kWave : cnt;
}

// Minimum and maximum over the wave (every lane active), by the device
// library's DPP reductions: row shifts within 16-lane rows, then across rows.
__device__ __forceinline__ int32_t wave_min(int32_t v) { return __ockl_wfred_min_i32(v); }

__device__ __forceinline__ int32_t wave_max(int32_t v) { return __ockl_wfred_max_i32(v); }

// First level of a wavefront search of the sorted v[0, n): up to 128 entries
// in registers, two per lane.  For n <= 128 these are all of v; otherwise 64
// evenly spaced samples, v[lane * step] with step = ceil(n / 64).  Split from
// the rest of the search so that a caller can issue these loads together with
// other independent ones (the compiler keeps loads in flight across code that
// does not use them).
//
// With COMP, a companion array c indexed like v (at least n entries) is loaded
// beside the search's last level, and the search also returns c[i] for the i
// it finds: a value keyed by the same index (a request's descriptor count,
// found with the request) then costs no dependent load of its own.
struct WaveSamples {
    int32_t r0, r1;  // raw entries (lane, lane + 64; or the lane's sample), clamped loads
    int32_t n, step; // step 0: the samples are v itself
    int32_t c0, c1;  // COMP, step 0: c at the entries of r0 and r1
};

// Entry v as a 64-bit key where the lane holds one, INT64_MAX where it holds
// none.  A max, not a select: the compiler turns a select whose operand is a
// load into a branch with the load moved under it, which then waits for the
// load (and every load issued before it) at the branch.
__device__ __forceinline__ int64_t entry_or_max(int32_t v, bool has)
{
    return max(static_cast<int64_t>(v), has ? INT64_MIN : INT64_MAX);
}

// WIDE (n > 128: samples, then a window) or not (n <= 128: the whole of v) is
// chosen by the caller, uniformly, before any load, so that each variant is
// straight-line code from its loads to their use: the compiler moves a load
// past a branch to the block that uses it, and there waits for it together
// with every load issued before it.  The loads are at indices clamped into v
// and masked at their use, so v must hold at least one entry even when n is 0
// (query_start_loc always does; wave_upper_index checks n for other arrays).
template <bool COMP = false, bool WIDE = false>
__device__ __forceinline__ WaveSamples wave_samples(const int32_t *v, int32_t n,
                                                    const int32_t *c = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t last = max(n - 1, 0);
    WaveSamples s{0, 0, n, 0, 0, 0};
    if constexpr (WIDE) {
        s.step = max((n + kWave - 1) / kWave, 1);
        s.r0 = v[min(lane * s.step, last)];
    } else {
        const int32_t i0 = min(lane, last), i1 = min(lane + kWave, last);
        if (COMP) {
            const int32_t *cc = n > 0 ? c : v;  // c may be absent when there is no entry
            s.c0 = cc[i0];
            s.c1 = cc[i1];
        }
        s.r0 = v[i0];
        s.r1 = v[i1];
    }
    return s;
}

// Entry j (0 <= j < 128, per lane) of a 128-entry window held two per lane:
// w0 holds entries 0..63, w1 entries 64..127.  Every lane runs both shuffles.
__device__ __forceinline__ int32_t window_entry(int32_t w0, int32_t w1, int32_t j)
{
    const int32_t a = __shfl(w0, j & (kWave - 1)), b = __shfl(w1, j & (kWave - 1));
    return j < kWave ? a : b;
}

// Largest i in [0, n) with v[i] <= x (this lane's key), or -1; v sorted, s
// from wave_samples<COMP, WIDE>(v, n, c).  Every lane of the wave calls it with
// the same v and samples; lanes with part == false get -1 and do not shape the
// search.  WIDE: when the lanes' answers lie too far apart for one 128-entry
// window, each lane finishes with a binary search inside its own 1/64 bucket.
// With COMP, c_out receives c[i] (0 with no answer).
template <bool COMP = false, bool WIDE = false>
__device__ __forceinline__ int32_t wave_search(const int32_t *v, const WaveSamples &s, int64_t x,
                                               bool part, const int32_t *c = nullptr,
                                               int32_t *c_out = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    int32_t lo = 0;
    int64_t s0, s1;
    int32_t w0 = s.c0, w1 = s.c1;
    if constexpr (!WIDE) {  // n <= 128 (n <= 0: every entry masked, no answer)
        s0 = entry_or_max(s.r0, lane < s.n);
        s1 = entry_or_max(s.r1, lane + kWave < s.n);
    } else {
        if (COMP) *c_out = 0;
        const int cnt = wave_rank(entry_or_max(s.r0, lane * s.step < s.n), x);
        int32_t b_lo = INT32_MAX, b_hi = INT32_MIN;  // this lane's bucket [b_lo, b_hi)
        if (part && cnt > 0) {
            b_lo = (cnt - 1) * s.step;
            b_hi = min(cnt * s.step, s.n);
        }
        const int32_t u_lo = wave_min(b_lo), u_hi = wave_max(b_hi);
        if (u_lo == INT32_MAX) return -1;  // no taking-part lane has an answer
        if (u_hi - u_lo > 2 * kWave) {
            if (!part || cnt == 0) return -1;
            int32_t a = b_lo, h = b_hi;  // v[a] <= x
            while (h - a > 1) {
                const int32_t mid = (a + h) >> 1;
                if (v[mid] <= x) a = mid; else h = mid;
            }
            if (COMP) *c_out = c[a];
            return a;
        }
        // window of at most 128 entries: two per lane, loaded together (len >= 1)
        lo = u_lo;
        const int32_t len = u_hi - u_lo;
        const int32_t i0 = lo + min(lane, len - 1), i1 = lo + min(lane + kWave, len - 1);
        if (COMP) {
            w0 = c[i0];
            w1 = c[i1];
        }
        s0 = entry_or_max(v[i0], lane < len);
        s1 = entry_or_max(v[i1], lane + kWave < len);
    }
    int cnt = wave_rank(s0, x);
    const int cnt1 = wave_rank(s1, x);
    if (cnt == kWave) cnt += cnt1;
    const bool hit = part && cnt > 0;
    if (COMP) {
        const int32_t e = window_entry(w0, w1, hit ? cnt - 1 : 0);
        *c_out = hit ? e : 0;
    }
    return hit ? lo + cnt - 1 : -1;
}

// Largest i in [0, n) with v[i] <= x (this lane's key), or -1; v sorted.
// Both levels in one call, the variant chosen from n; with COMP also c[i] in
// c_out.
template <bool COMP = false>
__device__ __forceinline__ int32_t wave_upper_index(const int32_t *v, int32_t n, int64_t x, bool part,
                                                    const int32_t *c = nullptr,
                                                    int32_t *c_out = nullptr)
{
    if (n <= 0) {  // uniform; v may hold no entry at all (a row of zero width)
        if (COMP) *c_out = 0;
        return -1;
    }
    if (n > 2 * kWave)
        return wave_search<COMP, true>(v, wave_samples<COMP, true>(v, n, c), x, part, c, c_out);
    return wave_search<COMP, false>(v, wave_samples<COMP, false>(v, n, c), x, part, c, c_out);
}

// Entry i (wave-uniform, 0 <= i < 128) of a window held two per lane.
__device__ __forceinline__ int32_t uniform_entry(int32_t w0, int32_t w1, int32_t i)
{
    return i < kWave ? __builtin_amdgcn_readlane(w0, i) : __builtin_amdgcn_readlane(w1, i - kWave);
}

// The same search for a key x that is equal on every lane (one token per
// wave): the entries <= x form a prefix of the sorted v, so a level is one
// vector load of up to 128 entries (two per lane) and the popcount of a
// ballot, with no shuffles.  One level covers n <= 128 and two n <= 16,384.
// The result is wave-uniform; with COMP, c_out receives c[i] (0 with none),
// loaded beside the last level.
template <bool COMP = false>
__device__ __forceinline__ int32_t wave_uniform_upper_index(const int32_t *v, int32_t n, int64_t x,
                                                            const int32_t *c = nullptr,
                                                            int32_t *c_out = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (COMP) *c_out = 0;
    if (n <= 0) return -1;
    int32_t lo = 0, len = n;
    // loads are unconditional at clamped indices (see wave_samples)
    while (len > 2 * kWave) {
        const int32_t step = (len + 2 * kWave - 1) / (2 * kWave);
        const int32_t i0 = lane * step, i1 = (lane + kWave) * step;
        const int64_t v0 = v[lo + min(i0, len - 1)], v1 = v[lo + min(i1, len - 1)];
        const bool p0 = i0 < len && v0 <= x;
        const bool p1 = i1 < len && v1 <= x;
        const int32_t cnt = __builtin_amdgcn_readfirstlane(
            static_cast<int32_t>(__popcll(__ballot(p0)) + __popcll(__ballot(p1))));
        if (cnt == 0) return -1;  // v[lo] > x: only possible at the first level
        lo += (cnt - 1) * step;
        len = min(step, len - (cnt - 1) * step);
    }
    const int32_t i0 = lo + min(lane, len - 1), i1 = lo + min(lane + kWave, len - 1);
    int32_t w0 = 0, w1 = 0;
    if (COMP) {
        w0 = c[i0];
        w1 = c[i1];
    }
    const int64_t v0 = v[i0];
    const int64_t v1 = len > kWave ? v[i1] : INT64_MAX;  // uniform
    const bool p0 = lane < len && v0 <= x;
    const bool p1 = lane + kWave < len && v1 <= x;
    const int32_t cnt = __builtin_amdgcn_readfirstlane(
        static_cast<int32_t>(__popcll(__ballot(p0)) + __popcll(__ballot(p1))));
    if (cnt == 0) return -1;
    if (COMP) *c_out = uniform_entry(w0, w1, cnt - 1);
    return lo + cnt - 1;
}

// The wave-uniform search of a sorted v with n <= 128 entries in two phases:
// uniform_window issues its one vector load (two entries per lane, clamped
// into v) and uniform_rank counts the entries <= x with ballots.  Issued
// before other vector loads, the window can be waited on while those stay in
// flight (vector loads complete in order).  With COMP the window also holds
// the companion c at the same indices, and uniform_entry(w.c0, w.c1, i)
// gives c[i].
struct UniformWindow {
    int32_t v0, v1;  // kept 32-bit: a widening right after the load would wait for it
    int32_t n;
    int32_t c0, c1;
};

// Loads are unconditional (no branch to join) at indices clamped into v, which
// must hold at least one entry; n <= 0 gives an empty window.  The companion is
// read only below n (with n <= 0 the loads go to v instead).
template <bool COMP = false>
__device__ __forceinline__ UniformWindow uniform_window(const int32_t *v, int32_t n,
                                                        const int32_t *c = nullptr)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t last = n > 0 ? n - 1 : 0;
    const int32_t i0 = min(lane, last), i1 = min(lane + kWave, last);
    UniformWindow w{0, 0, n, 0, 0};
    if (COMP) {
        const int32_t *cc = n > 0 ? c : v;
        w.c0 = cc[i0];
        w.c1 = cc[i1];
    }
    w.v0 = v[i0];
    w.v1 = v[i1];
    return w;
}

// Largest i < n with v[i] <= x (x wave-uniform), or -1.
__device__ __forceinline__ int32_t uniform_rank(const UniformWindow &w, int64_t x)
{
    const int lane = threadIdx.x & (kWave - 1);
    const bool p0 = lane < w.n && static_cast<int64_t>(w.v0) <= x;
    const bool p1 = lane + kWave < w.n && static_cast<int64_t>(w.v1) <= x;
    const int32_t cnt = __builtin_amdgcn_readfirstlane(
        static_cast<int32_t>(__popcll(__ballot(p0)) + __popcll(__ballot(p1))));
    return cnt == 0 ? -1 : cnt - 1;
}

// Logical block lb and in-block offset off of position p >= 0 on this rank.
// Without context parallelism (world <= 1) lb = p / bs and off = p % bs.  With
// W ranks and interleave I the ranks deal positions in chunks of I, round
// robin; a table entry covers a virtual block of bs*W positions, of which each
// rank keeps its own, in order, in its block of bs slots:
//   owner = (p / I) % W,  lb = p / (bs*W),  o = p % (bs*W),
//   off = (o / (I*W)) * I + o % I.
// Returns false when another rank holds p.  bs*W fits an int32 (host check).
__device__ __forceinline__ bool cp_locate(int64_t p, int32_t block_size, int32_t world,
                                          int32_t rank, int32_t interleave, int64_t &lb,
                                          int32_t &off)
{
    const uint32_t bs = static_cast<uint32_t>(block_size);
    if (world <= 1) {
        if (p <= INT32_MAX) {
            const uint32_t q = static_cast<uint32_t>(p) / bs;
            lb = q;
            off = static_cast<int32_t>(static_cast<uint32_t>(p) - q * bs);
        } else {
            lb = p / block_size;
            off = static_cast<int32_t>(p - lb * block_size);
        }
        return true;
    }
    const int64_t w = world, il = interleave, span = static_cast<int64_t>(bs) * w;
    int64_t o;
    if (p <= INT32_MAX) {
        const uint32_t up = static_cast<uint32_t>(p);
        if ((up / static_cast<uint32_t>(il)) % static_cast<uint32_t>(w) != static_cast<uint32_t>(rank))
            return false;
        const uint32_t q = up / static_cast<uint32_t>(span);
        lb = q;
        o = up - q * static_cast<uint32_t>(span);
    } else {
        if ((p / il) % w != rank) return false;
        lb = p / span;
        o = p - lb * span;
    }
    const uint32_t uo = static_cast<uint32_t>(o), ui = static_cast<uint32_t>(il);
    off = static_cast<int32_t>((uo / (ui * static_cast<uint32_t>(w))) * ui + uo % ui);
    return true;
}

}  // namespace
