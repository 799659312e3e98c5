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

__device__ __forceinline__ int32_t wave_min(int32_t v)
{
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int32_t wave_max(int32_t v)
{
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// First level of a wavefront search of the sorted v[0, n): up to 128 entries
// in registers, two per lane.  For n <= 128 these are all of v; otherwise 64
// evenly spaced samples, v[lane * step] with step = ceil(n / 64).  Split from
// the rest of the search so that a caller can issue these loads together with
// other independent ones (the compiler keeps loads in flight across code that
// does not use them).
struct WaveSamples {
    int64_t s0, s1;  // INT64_MAX where a lane holds no entry
    int32_t n, step; // step 0: the samples are v itself
};

__device__ __forceinline__ WaveSamples wave_samples(const int32_t *v, int32_t n)
{
    // loads are unconditional, at indices clamped into v, and masked afterwards: a load
    // under a per-lane branch makes the compiler wait for it before the branch joins
    const int lane = threadIdx.x & (kWave - 1);
    WaveSamples s{INT64_MAX, INT64_MAX, n, 0};
    if (n <= 0) return s;  // uniform
    if (n > 2 * kWave) {
        s.step = (n + kWave - 1) / kWave;
        const int32_t idx = lane * s.step;
        const int64_t x = v[min(idx, n - 1)];
        if (idx < n) s.s0 = x;
    } else {
        const int64_t x0 = v[min(lane, n - 1)], x1 = v[min(lane + kWave, n - 1)];
        if (lane < n) s.s0 = x0;
        if (lane + kWave < n) s.s1 = x1;
    }
    return s;
}

// Largest i in [0, n) with v[i] <= x (this lane's key), or -1; v sorted, s
// from wave_samples(v, n).  Every lane of the wave calls it with the same v
// and samples; lanes with part == false get -1 and do not shape the search.
// When the lanes' answers lie too far apart for one 128-entry window, each
// lane finishes with a binary search inside its own 1/64 bucket.
__device__ int32_t wave_search(const int32_t *v, const WaveSamples &s, int64_t x, bool part)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (s.n <= 0) return -1;
    int32_t lo = 0, len = s.n;
    int64_t s0 = s.s0, s1 = s.s1;
    if (s.step > 0) {
        const int cnt = wave_rank(s0, x);
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
            return a;
        }
        // window of at most 128 entries: two per lane, loaded together (len >= 1)
        lo = u_lo;
        len = u_hi - u_lo;
        const int64_t x0 = v[lo + min(lane, len - 1)], x1 = v[lo + min(lane + kWave, len - 1)];
        s0 = lane < len ? x0 : INT64_MAX;
        s1 = lane + kWave < len ? x1 : INT64_MAX;
    }
    int cnt = wave_rank(s0, x);
    const int cnt1 = wave_rank(s1, x);
    if (cnt == kWave) cnt += cnt1;
    return (part && cnt > 0) ? lo + cnt - 1 : -1;
}

// Largest i in [0, n) with v[i] <= x (this lane's key), or -1; v sorted.
// The two levels of wave_samples and wave_search in one call.
__device__ __forceinline__ int32_t wave_upper_index(const int32_t *v, int32_t n, int64_t x, bool part)
{
    return wave_search(v, wave_samples(v, n), x, part);
}

// The same search for a key x that is equal on every lane (one token per
// wave): the entries <= x form a prefix of the sorted v, so a level is one
// vector load of up to 128 entries (two per lane) and the popcount of a
// ballot, with no shuffles.  One level covers n <= 128 and two n <= 16,384.
// With LAST, v[n - 1] is loaded alongside the first level and, when <= x,
// answers at once (a key in the last run skips the second level).  The
// result is wave-uniform.
template <bool LAST = false>
__device__ __forceinline__ int32_t wave_uniform_upper_index(const int32_t *v, int32_t n, int64_t x)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (n <= 0) return -1;
    int32_t lo = 0, len = n;
    const int64_t last = LAST ? static_cast<int64_t>(v[n - 1]) : INT64_MAX;
    bool first = true;
    // loads are unconditional at clamped indices (see wave_samples)
    while (len > 2 * kWave) {
        const int32_t step = (len + 2 * kWave - 1) / (2 * kWave);
        const int32_t i0 = lane * step, i1 = (lane + kWave) * step;
        const int64_t v0 = v[lo + min(i0, len - 1)], v1 = v[lo + min(i1, len - 1)];
        const bool p0 = i0 < len && v0 <= x;
        const bool p1 = i1 < len && v1 <= x;
        if (LAST && first && last <= x) return n - 1;
        first = false;
        const int32_t cnt = __builtin_amdgcn_readfirstlane(
            static_cast<int32_t>(__popcll(__ballot(p0)) + __popcll(__ballot(p1))));
        if (cnt == 0) return -1;  // v[lo] > x: only possible at the first level
        lo += (cnt - 1) * step;
        len = min(step, len - (cnt - 1) * step);
    }
    const int64_t v0 = v[lo + min(lane, len - 1)];
    const int64_t v1 = len > kWave ? v[lo + min(lane + kWave, len - 1)] : INT64_MAX;  // uniform
    const bool p0 = lane < len && v0 <= x;
    const bool p1 = lane + kWave < len && v1 <= x;
    const int32_t cnt = __builtin_amdgcn_readfirstlane(
        static_cast<int32_t>(__popcll(__ballot(p0)) + __popcll(__ballot(p1))));
    return cnt == 0 ? -1 : lo + cnt - 1;
}

// The wave-uniform search of a sorted v with n <= 128 entries in two phases:
// uniform_window issues its one vector load (two entries per lane, clamped
// into v) and uniform_rank counts the entries <= x with ballots.  Issued
// before other vector loads, the window can be waited on while those stay in
// flight (vector loads complete in order).
struct UniformWindow {
    int32_t v0, v1;  // kept 32-bit: a widening right after the load would wait for it
    int32_t n;
};

// Loads are unconditional (no branch to join) at indices clamped into v, which
// must hold at least one entry; n <= 0 gives an empty window.
__device__ __forceinline__ UniformWindow uniform_window(const int32_t *v, int32_t n)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t last = n > 0 ? n - 1 : 0;
    return UniformWindow{v[min(lane, last)], v[min(lane + kWave, last)], n};
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
