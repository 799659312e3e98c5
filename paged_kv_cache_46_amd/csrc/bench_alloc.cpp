// Host benchmark of the range allocator and the checked coordinate offset,
// calling libkvw.so through its C ABI (include/kvw_alloc.h).  The offset
// scenarios use the header's inline form, as a per-token host loop would; one
// more scenario times the same offset through the library call.
//
// Harness as in "Range-addressed KV cache blocks for the vLLM serving
// engine", "Benchmark Methodology" (host benchmark): each scenario runs
// `iterations` calls per round over `rounds` rounds with one warmup call per
// round, on a steady clock, and reports the mean and standard deviation
// across rounds of the nanoseconds per call.  Scenarios follow that page's
// "Measured Results" table; the layout is its coordinate layout (32 layers,
// 64K blocks, 32 tokens per block, 2048 bytes per token).
//
// Usage: bench_alloc [iterations] [rounds]   -- one JSON object per line.

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <type_traits>
#include <vector>

#include "kvw_alloc.h"

namespace {

constexpr int64_t kLayers = 32, kBlocks = 65536, kTokens = 32, kBytes = 2048;

struct Result {
    double mean, stddev;
};

volatile int64_t g_sink;  // keeps results observable

// The checked offset as a per-token host loop calls it: inline from the
// header, or (kLibrary) through the shared library's kvw_coord_offset.
template <bool kLibrary>
inline kvw_status coord_offset(int64_t layer, int64_t block, int64_t token, int64_t *off)
{
    return kLibrary ? kvw_coord_offset(layer, block, token, kLayers, kBlocks, kTokens, kBytes, off)
                    : kvw_coord_offset_inline(layer, block, token, kLayers, kBlocks, kTokens,
                                              kBytes, off);
}

void check(kvw_status st, const char *what)
{
    if (st != KVW_OK) {
        std::fprintf(stderr, "%s failed (%d): %s\n", what, static_cast<int>(st), kvw_last_error());
        std::exit(1);
    }
}

// setup(round) runs untimed before each round; call(i) is one timed call
// (a template parameter, so the loop makes a direct call); per_call divides a
// round's time (ns per call, or per token for walks).
template <typename Setup, typename Call>
Result run(int64_t iterations, int rounds, Setup &&setup, Call &&call, double per_call)
{
    std::vector<double> ns(rounds);
    for (int r = 0; r < rounds; ++r) {
        setup(r);
        call(-1);  // warmup
        const auto t0 = std::chrono::steady_clock::now();
        for (int64_t i = 0; i < iterations; ++i) call(i);
        const auto t1 = std::chrono::steady_clock::now();
        ns[r] = std::chrono::duration<double, std::nano>(t1 - t0).count() / (iterations * per_call);
    }
    double m = 0, v = 0;
    for (double x : ns) m += x;
    m /= rounds;
    for (double x : ns) v += (x - m) * (x - m);
    return {m, rounds > 1 ? std::sqrt(v / (rounds - 1)) : 0.0};
}

void emit(const char *name, const char *unit, const char *what, int64_t iterations, int rounds,
          Result r)
{
    std::printf("{\"scenario\": \"%s\", \"mean_ns\": %.3f, \"stddev_ns\": %.3f, \"unit\": \"%s\", "
                "\"iterations\": %lld, \"rounds\": %d, \"what\": \"%s\"}\n",
                name, r.mean, r.stddev, unit, static_cast<long long>(iterations), rounds, what);
    std::fflush(stdout);
}

}  // namespace

int main(int argc, char **argv)
{
    const int64_t iters = argc > 1 ? std::atoll(argv[1]) : 200000;
    const int rounds = argc > 2 ? std::atoi(argv[2]) : 20;

    // map/offset single: one checked closed-form offset, at a varying coordinate
    auto offset_single = [&](auto library, const char *name, const char *what) {
        int64_t seed = 12345;
        auto call = [&](int64_t i) {
            seed = seed * 6364136223846793005LL + 1442695040888963407LL;  // vary the coordinate
            const uint64_t u = static_cast<uint64_t>(seed) >> 11;
            int64_t off = 0;
            coord_offset<decltype(library)::value>(static_cast<int64_t>(u % kLayers),
                                                   static_cast<int64_t>((u >> 5) % kBlocks),
                                                   static_cast<int64_t>((u >> 21) % kTokens), &off);
            g_sink = off + i;
        };
        emit(name, "ns/op", what, iters, rounds, run(iters, rounds, [](int) {}, call, 1.0));
    };
    offset_single(std::false_type{}, "map/offset single", "one checked closed-form offset");
    offset_single(std::true_type{}, "map/offset single, library call",
                  "the same through the shared library (kvw_coord_offset)");
    // map/offset decode walk: one new token per step of a request holding a contiguous range
    {
        int64_t pos = 0;
        const int64_t start = 1000;
        auto call = [&](int64_t) {
            const int64_t p = pos++ % (kTokens * 4096);
            int64_t off = 0;
            coord_offset<false>(7, start + p / kTokens, p % kTokens, &off);
            g_sink = off;
        };
        emit("map/offset decode walk", "ns/op", "one new token per step", iters, rounds,
             run(iters, rounds, [](int) {}, call, 1.0));
    }
    // map/offset context walk 4k: prefill walk of one 4,096-token request
    {
        const int64_t walk = 4096, start = 2000, calls = std::max<int64_t>(1, iters / walk);
        auto call = [&](int64_t) {
            int64_t acc = 0, off = 0;
            for (int64_t p = 0; p < walk; ++p) {
                coord_offset<false>(3, start + p / kTokens, p % kTokens, &off);
                acc += off;
            }
            g_sink = acc;
        };
        emit("map/offset context walk 4k", "ns/token", "prefill walk of one request", calls, rounds,
             run(calls, rounds, [](int) {}, call, static_cast<double>(walk)));
    }

    kvw_alloc *a = nullptr;
    check(kvw_alloc_create(kBlocks, 1, 1, 1024, &a), "create");
    // a pool in use: 512 requests of 64 blocks, every other one released (256 holes)
    for (int r = 0; r < 512; ++r) check(kvw_alloc_extend(a, r, 64), "fill");
    for (int r = 0; r < 512; r += 2) check(kvw_alloc_release(a, r), "hole");

    // alloc/allocate release: one allocate (16 blocks: a 512-token prompt) plus one release
    {
        auto call = [&](int64_t) {
            kvw_alloc_extend(a, 600, 16);
            kvw_alloc_release(a, 600);
        };
        emit("alloc/allocate release", "ns/cycle", "one allocate plus one release", iters, rounds,
             run(iters, rounds, [](int) {}, call, 1.0));
    }
    // alloc/grow in place: decode growth, one block per 32 tokens (rollover every 32 steps)
    {
        int64_t tokens = 0;
        auto setup = [&](int) {
            kvw_alloc_release(a, 601);
            tokens = 0;
        };
        auto call = [&](int64_t) {
            if (tokens % kTokens == 0) {
                if (tokens >= kTokens * 2048) {  // a 64K-token context: start over
                    kvw_alloc_release(a, 601);
                    tokens = 0;
                }
                kvw_alloc_extend(a, 601, 1);
            }
            ++tokens;
        };
        emit("alloc/grow in place", "ns/step", "decode growth, rollover every 32 steps", iters,
             rounds, run(iters, rounds, setup, call, 1.0));
        kvw_alloc_release(a, 601);
    }
    // alloc/prefix acquire release: one prefix share cycle on a cached 8-block range
    {
        check(kvw_alloc_extend(a, 602, 8), "prefix");
        check(kvw_alloc_cache_insert(a, 42, 602, 0, 8), "prefix insert");
        auto call = [&](int64_t) {
            kvw_alloc_cache_acquire(a, 42, 603);
            kvw_alloc_release(a, 603);
        };
        emit("alloc/prefix acquire release", "ns/cycle", "one prefix share cycle", iters, rounds,
             run(iters, rounds, [](int) {}, call, 1.0));
        kvw_alloc_release(a, 602);
        int64_t n;
        kvw_alloc_cache_evict(a, 1 << 30, &n);
    }
    // alloc/evict cache only: LRU eviction of one cache-only range
    {
        const int64_t per_round = std::min<int64_t>(iters, 20000);
        auto setup = [&](int r) {
            // per_round + 1 cache-only 1-block ranges (one for the warmup call)
            for (int64_t i = 0; i <= per_round; ++i) {
                check(kvw_alloc_extend(a, 700, 1), "evict setup");
                check(kvw_alloc_cache_insert(a, (static_cast<uint64_t>(r) << 32) | i, 700,
                                             0, 1), "evict insert");
                check(kvw_alloc_release(a, 700), "evict release");
            }
        };
        auto call = [&](int64_t) {
            int64_t n;
            kvw_alloc_cache_evict(a, 1, &n);
            g_sink = n;
        };
        emit("alloc/evict cache only", "ns/evict", "LRU eviction of a cache-only range", per_round,
             rounds, run(per_round, rounds, setup, call, 1.0));
    }
    kvw_alloc_destroy(a);
    return 0;
}
