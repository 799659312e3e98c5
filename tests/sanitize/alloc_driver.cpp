// Drives the range allocator (paged_kv_cache_46_amd/csrc/range_alloc.cpp) through a long,
// seeded mix of valid and invalid calls and checks what any state must satisfy.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py (host code only),
// so an out-of-bounds access, a leak or undefined arithmetic ends the run with an error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvw_alloc.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next()
{  // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
int64_t below(int64_t n) { return static_cast<int64_t>(next() % static_cast<uint64_t>(n)); }

int g_failures = 0;
void expect(bool ok, const char *what, long step)
{
    if (!ok && g_failures++ < 10) std::fprintf(stderr, "step %ld: %s\n", step, what);
}

void run(int64_t num_blocks, int32_t align, int64_t first, int32_t rows, long steps)
{
    kvw_alloc *a = nullptr;
    if (kvw_alloc_create(num_blocks, align, first, rows, &a) != KVW_OK) {
        std::fprintf(stderr, "create failed: %s\n", kvw_last_error());
        std::exit(2);
    }
    kvw_alloc_stats st0;
    kvw_alloc_get_stats(a, &st0);
    std::vector<int64_t> starts(num_blocks + 1), lens(num_blocks + 1);
    for (long i = 0; i < steps; ++i) {
        const int32_t row = static_cast<int32_t>(below(rows + 1)) - (below(50) == 0 ? 1 : 0);
        const int op = static_cast<int>(below(100));
        kvw_status s;
        if (op < 45) {
            int64_t n = align * below(12);
            if (below(40) == 0) n = below(3) - 1;  // negative or unaligned now and then
            s = kvw_alloc_extend(a, row, n);
        } else if (op < 62) {
            s = kvw_alloc_release(a, row);
        } else if (op < 78) {
            s = kvw_alloc_cache_insert(a, static_cast<uint64_t>(below(40)), row, align * below(8),
                                       align * (below(4) + (below(30) == 0 ? -1 : 0)));
        } else if (op < 92) {
            s = kvw_alloc_cache_acquire(a, static_cast<uint64_t>(below(48)), row);
        } else {
            int64_t k = -1;
            s = kvw_alloc_cache_evict(a, below(4) - (below(20) == 0 ? 1 : 0), &k);
        }
        expect(s >= KVW_OK && s <= KVW_ERR_NOT_FOUND, "unknown status", i);
        // the accounting always adds up
        kvw_alloc_stats st;
        kvw_alloc_get_stats(a, &st);
        int64_t nruns = 0, free_sum = 0;
        kvw_alloc_free_runs(a, num_blocks + 1, starts.data(), lens.data(), &nruns);
        for (int64_t r = 0; r < nruns; ++r) {
            free_sum += lens[r];
            expect(lens[r] > 0 && starts[r] % align == 0, "bad free run", i);
            if (r) expect(starts[r - 1] + lens[r - 1] < starts[r], "free runs not coalesced", i);
        }
        expect(free_sum == st.free_blocks && nruns == st.free_runs, "free accounting", i);
        expect(st.usable_blocks == st0.usable_blocks, "usable changed", i);
        for (int32_t r = 0; r < rows; ++r) {  // every row's extents are aligned and in the pool
            int32_t n = 0;
            kvw_alloc_row_extents(a, r, static_cast<int32_t>(num_blocks), starts.data(), lens.data(),
                                  &n);
            for (int32_t e = 0; e < n; ++e)
                expect(starts[e] % align == 0 && lens[e] % align == 0 && lens[e] > 0 &&
                           starts[e] + lens[e] <= num_blocks, "bad extent", i);
        }
        expect(st.free_blocks + st.cache_only_blocks <= st.usable_blocks, "over-count", i);
        if (i % 997 == 0) {  // exports of every row, both shapes
            std::vector<int32_t> ids(rows), s32(rows * 64), l32(rows * 64), c32(rows * 64), nr(rows);
            for (int32_t r = 0; r < rows; ++r) ids[r] = r;
            kvw_alloc_ranges(a, ids.data(), rows, 64, s32.data(), l32.data(), c32.data(), nr.data());
            std::vector<int32_t> table(static_cast<size_t>(rows) * num_blocks), counts(rows);
            kvw_alloc_block_table(a, ids.data(), rows, static_cast<int32_t>(num_blocks),
                                  table.data(), counts.data());
        }
    }
    int64_t evicted = 0;
    for (int32_t r = 0; r < rows; ++r) kvw_alloc_release(a, r);
    kvw_alloc_cache_evict(a, INT64_MAX, &evicted);
    kvw_alloc_stats st;
    kvw_alloc_get_stats(a, &st);
    expect(st.free_blocks == st.usable_blocks && st.free_runs == (st.usable_blocks ? 1 : 0),
           "pool not whole after releasing everything", steps);
    kvw_alloc_destroy(a);
}

}  // namespace

int main()
{
    run(97, 1, 1, 4, 60000);
    run(200, 4, 3, 6, 60000);
    run(64, 8, 0, 3, 30000);
    run(5, 2, 7, 2, 2000);  // no usable chunk at all
    int64_t off = 0;
    expect(kvw_coord_offset(31, 65535, 31, 32, 65536, 32, 2048, &off) == KVW_OK, "offset", 0);
    expect(kvw_coord_offset(1, 0, 0, 2, INT64_MAX / 2, 4, 1024, &off) == KVW_ERR_UNSUPPORTED,
           "offset overflow", 0);
    expect(kvw_coord_offset(-1, 0, 0, 2, 2, 2, 2, &off) == KVW_ERR_INVALID_ARG, "negative", 0);
    if (g_failures) return 1;
    std::printf("OK\n");
    return 0;
}
