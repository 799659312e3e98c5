// Contiguous-range block allocator (host side) and the checked coordinate
// offset of the write path; the contract is include/kvw_alloc.h.
//
// Sources: "Range-addressed KV cache blocks for the vLLM serving engine",
// sections "The allocator: contiguous ranges as the closed form" (aligned
// ranges, an always-coalesced free list, growth in place, merging on append,
// prefix sharing by reference, LRU eviction of cache-only ranges, request and
// cache references kept apart) and "The Coordinate Approach" (the offset).
//
// Free space is kept per chunk (`alignment` blocks) as coalesced runs with
// boundary tags: run_len[c] is the length of the free run that starts at
// chunk c (0 if none does) and run_head[c] is start + 1 at a run's last chunk
// (0 elsewhere), so freeing a span finds both neighbours in O(1).  A max
// segment tree over run_len finds the leftmost run of at least k chunks --
// first fit -- in one root-to-leaf descent.  Taking the head of a run, or
// freeing a span next to a run, changes two leaves; the leaf whose new value
// is the larger is written first, so the second leaf-to-root walk stops where
// the two paths meet.  After creation nothing is heap-allocated except when a
// row's extent list, the extent pool or the cache map outgrows its capacity.
// The prefix cache's key -> extent map is open addressing with linear probing
// over a power-of-two table at most half full (no per-entry heap node, no
// division to find a bucket), with deletion by backward shift, so no
// tombstones accumulate.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kvw_alloc.h"
#include "kvw_error.h"

using kvw_detail::fail;

namespace {

struct Extent {
    int32_t start = 0;     // first chunk
    int32_t len = 0;       // chunks
    int32_t refs = 0;      // request references (row listings)
    int32_t prev = -1;     // LRU links while cache-only
    int32_t next = -1;
    bool cached = false;   // held by the prefix cache under `key`
    uint64_t key = 0;
};

// Cache key -> extent id.  Empty slots hold id -1.  Keys and ids sit in two
// arrays, so a probe run reads densely packed keys (one array of slots holding
// both was measured slower).  The hash is the 64-bit finalizer of MurmurHash3
// (a fixed bijection with good avalanche), so keys that differ only in high
// bits still spread over the table.
class KeyMap {
public:
    KeyMap() { rehash(1024); }

    size_t size() const { return count_; }

    // the id stored under key, or -1
    int32_t find(uint64_t key) const
    {
        for (size_t i = home(key);; i = (i + 1) & mask_) {
            if (ids_[i] < 0) return -1;
            if (keys_[i] == key) return ids_[i];
        }
    }

    // key must not be present; may throw std::bad_alloc when the table grows
    void insert(uint64_t key, int32_t id)
    {
        if (2 * (count_ + 1) > ids_.size()) rehash(2 * ids_.size());
        place(key, id);
        ++count_;
    }

    // key must be present
    void erase(uint64_t key)
    {
        size_t i = home(key);
        while (keys_[i] != key || ids_[i] < 0) i = (i + 1) & mask_;
        // backward shift: pull later entries of the probe run into the hole
        // when their home does not lie cyclically in (hole, slot]
        for (size_t j = (i + 1) & mask_; ids_[j] >= 0; j = (j + 1) & mask_) {
            const size_t h = home(keys_[j]);
            const bool stays = i <= j ? (i < h && h <= j) : (i < h || h <= j);
            if (stays) continue;
            keys_[i] = keys_[j];
            ids_[i] = ids_[j];
            i = j;
        }
        ids_[i] = -1;
        --count_;
    }

private:
    static uint64_t mix(uint64_t k)
    {
        k ^= k >> 33;
        k *= 0xff51afd7ed558ccdULL;
        k ^= k >> 33;
        k *= 0xc4ceb9fe1a85ec53ULL;
        k ^= k >> 33;
        return k;
    }
    size_t home(uint64_t key) const { return static_cast<size_t>(mix(key)) & mask_; }

    void place(uint64_t key, int32_t id)
    {
        size_t i = home(key);
        while (ids_[i] >= 0) i = (i + 1) & mask_;
        keys_[i] = key;
        ids_[i] = id;
    }

    void rehash(size_t cap)
    {
        std::vector<uint64_t> keys(cap);
        std::vector<int32_t> ids(cap, -1);
        keys.swap(keys_);
        ids.swap(ids_);
        mask_ = cap - 1;
        for (size_t i = 0; i < ids.size(); ++i)
            if (ids[i] >= 0) place(keys[i], ids[i]);
    }

    std::vector<uint64_t> keys_;
    std::vector<int32_t> ids_;
    size_t mask_ = 0, count_ = 0;
};

}  // namespace

struct kvw_alloc {
    int64_t num_blocks = 0;
    int32_t align = 1;
    int32_t align_log2 = -1;  // log2(align) when align is a power of two
    int32_t c0 = 0;        // first usable chunk
    int32_t nchunks = 0;   // usable chunks end here
    int32_t max_rows = 0;
    int32_t leaves = 1;    // segment-tree leaf count (power of two)
    std::vector<int32_t> run_len, run_head, tree;
    int64_t free_chunks = 0, free_runs = 0;
    std::vector<Extent> ext;
    std::vector<int32_t> spare;  // unused extent ids
    int64_t live = 0;
    std::vector<std::vector<int32_t>> rows;
    KeyMap cache;
    int32_t lru_head = -1, lru_tail = -1;
    int64_t cache_only_chunks = 0;

    // -- free space --------------------------------------------------------
    // The running maximum stays in a register and only the sibling is loaded,
    // so no level waits on the store made at the level below.
    void set_leaf(int32_t c, int32_t v)
    {
        run_len[c] = v;
        int32_t i = c + leaves;
        tree[i] = v;
        int32_t m = v;
        while (i > 1) {
            m = std::max(m, tree[i ^ 1]);
            i >>= 1;
            if (tree[i] == m) break;
            tree[i] = m;
        }
    }

    // Leftmost run start with at least k free chunks, or -1.  The descent is
    // branch-free: the left/right choice is data-dependent and would mispredict.
    int32_t first_fit(int64_t k) const
    {
        if (tree[1] < k) return -1;
        int32_t i = 1;
        while (i < leaves) i = 2 * i + static_cast<int32_t>(tree[2 * i] < k);
        return i - leaves;
    }

    // Blocks -> chunks; false when n is not a multiple of the alignment.
    bool to_chunks(int64_t n, int64_t &k) const
    {
        if (align_log2 >= 0) {
            if (n & (static_cast<int64_t>(align) - 1)) return false;
            k = n >> align_log2;
            return true;
        }
        if (n % align) return false;
        k = n / align;
        return true;
    }

    // Allocate the first k chunks of the free run starting at s.
    void take_head(int32_t s, int32_t k)
    {
        const int32_t L = run_len[s];
        if (L > k) {
            set_leaf(s + k, L - k);  // the larger new value first
            run_head[s + L - 1] = s + k + 1;
        } else {
            run_head[s + L - 1] = 0;
            --free_runs;
        }
        set_leaf(s, 0);
        free_chunks -= k;
    }

    // Return chunks [s, s+k) and merge them with free neighbours.
    void give(int32_t s, int32_t k)
    {
        const int32_t left = (s > c0 && run_head[s - 1]) ? run_head[s - 1] - 1 : -1;
        const int32_t right = (s + k < nchunks) ? run_len[s + k] : 0;
        const int32_t start = left >= 0 ? left : s;
        const int32_t end = s + k + right;
        if (left >= 0) run_head[s - 1] = 0;
        set_leaf(start, end - start);  // the larger new value first
        if (right) set_leaf(s + k, 0);
        run_head[end - 1] = start + 1;
        free_runs += 1 - (left >= 0 ? 1 : 0) - (right ? 1 : 0);
        free_chunks += k;
    }

    // -- extents and the LRU list ---------------------------------------------
    int32_t new_extent(int32_t start, int32_t len)
    {
        int32_t id;
        if (!spare.empty()) {
            id = spare.back();
            spare.pop_back();
        } else {
            id = static_cast<int32_t>(ext.size());
            ext.emplace_back();
        }
        Extent &e = ext[id];
        e = Extent{};
        e.start = start;
        e.len = len;
        e.refs = 1;
        ++live;
        return id;
    }

    void drop_extent(int32_t id)
    {
        spare.push_back(id);
        --live;
    }

    void lru_push(int32_t id)
    {
        Extent &e = ext[id];
        e.prev = lru_tail;
        e.next = -1;
        if (lru_tail >= 0) ext[lru_tail].next = id;
        else lru_head = id;
        lru_tail = id;
        cache_only_chunks += e.len;
    }

    void lru_unlink(int32_t id)
    {
        Extent &e = ext[id];
        if (e.prev >= 0) ext[e.prev].next = e.next;
        else lru_head = e.next;
        if (e.next >= 0) ext[e.next].prev = e.prev;
        else lru_tail = e.prev;
        e.prev = e.next = -1;
        cache_only_chunks -= e.len;
    }

    void evict_oldest()
    {
        const int32_t id = lru_head;
        lru_unlink(id);
        Extent &e = ext[id];
        cache.erase(e.key);
        give(e.start, e.len);
        drop_extent(id);
    }
};

namespace {

constexpr int64_t kMaxBlocks = INT32_MAX;

bool row_ok(const kvw_alloc *a, int32_t row) { return a && row >= 0 && row < a->max_rows; }

// Physically adjacent extents of a row merge into one range.
template <typename F>
int64_t for_each_range(const kvw_alloc *a, int32_t row, F &&f)
{
    int64_t n = 0, cum = 0, cur_start = -1, cur_len = 0;
    for (int32_t id : a->rows[row]) {
        const Extent &e = a->ext[id];
        if (cur_start >= 0 && cur_start + cur_len == e.start) {
            cur_len += e.len;
        } else {
            if (cur_start >= 0) {
                f(cur_start, cur_len, cum);
                cum += cur_len;
                ++n;
            }
            cur_start = e.start;
            cur_len = e.len;
        }
    }
    if (cur_start >= 0) {
        f(cur_start, cur_len, cum);
        ++n;
    }
    return n;
}

}  // namespace

extern "C" {

kvw_status kvw_alloc_create(int64_t num_blocks, int32_t alignment, int64_t first_block,
                            int32_t max_rows, kvw_alloc **out)
{
    const char *fn = "kvw_alloc_create";
    if (!out) return fail(KVW_ERR_INVALID_ARG, "%s: out is NULL", fn);
    *out = nullptr;
    if (num_blocks <= 0 || num_blocks > kMaxBlocks || alignment < 1 || first_block < 0 ||
        max_rows < 1)
        return fail(KVW_ERR_INVALID_ARG,
                    "%s: need 0 < num_blocks <= 2^31-1, alignment >= 1, first_block >= 0, "
                    "max_rows >= 1 (got %lld, %d, %lld, %d)",
                    fn, (long long)num_blocks, alignment, (long long)first_block, max_rows);
    try {
        auto *a = new kvw_alloc();
        a->num_blocks = num_blocks;
        a->align = alignment;
        if ((alignment & (alignment - 1)) == 0)
            a->align_log2 = __builtin_ctz(static_cast<unsigned>(alignment));
        a->nchunks = static_cast<int32_t>(num_blocks / alignment);
        a->c0 = static_cast<int32_t>(std::min<int64_t>((first_block + alignment - 1) / alignment,
                                                       a->nchunks));
        a->max_rows = max_rows;
        while (a->leaves < a->nchunks) a->leaves <<= 1;
        a->run_len.assign(static_cast<size_t>(a->nchunks) + 1, 0);
        a->run_head.assign(static_cast<size_t>(a->nchunks) + 1, 0);
        a->tree.assign(2 * static_cast<size_t>(a->leaves), 0);
        a->rows.resize(max_rows);
        for (auto &r : a->rows) r.reserve(8);
        a->ext.reserve(1024);
        a->spare.reserve(1024);
        if (a->c0 < a->nchunks) {
            a->set_leaf(a->c0, a->nchunks - a->c0);
            a->run_head[a->nchunks - 1] = a->c0 + 1;
            a->free_chunks = a->nchunks - a->c0;
            a->free_runs = 1;
        }
        *out = a;
        return KVW_OK;
    } catch (const std::bad_alloc &) {
        return fail(KVW_ERR_UNSUPPORTED, "%s: out of host memory", fn);
    }
}

void kvw_alloc_destroy(kvw_alloc *a) { delete a; }

kvw_status kvw_alloc_extend(kvw_alloc *a, int32_t row, int64_t num_blocks)
{
    const char *fn = "kvw_alloc_extend";
    if (!row_ok(a, row)) return fail(KVW_ERR_INVALID_ARG, "%s: no allocator or row %d", fn, row);
    int64_t k;
    if (num_blocks < 0 || !a->to_chunks(num_blocks, k))
        return fail(KVW_ERR_INVALID_ARG, "%s: %lld blocks is not a non-negative multiple of %d",
                    fn, (long long)num_blocks, a->align);
    if (k == 0) return KVW_OK;
    if (a->free_chunks < k) {
        if (a->free_chunks + a->cache_only_chunks < k)
            return fail(KVW_ERR_NO_SPACE, "%s: %lld blocks wanted, %lld free and %lld evictable",
                        fn, (long long)num_blocks, (long long)(a->free_chunks * a->align),
                        (long long)(a->cache_only_chunks * a->align));
        while (a->free_chunks < k) a->evict_oldest();
    }
    try {
        std::vector<int32_t> &r = a->rows[row];
        const int32_t kk = static_cast<int32_t>(k);
        if (!r.empty()) {
            Extent &e = a->ext[r.back()];
            const int32_t end = e.start + e.len;
            if (e.refs == 1 && !e.cached && end < a->nchunks && a->run_len[end] >= kk) {
                a->take_head(end, kk);  // growth in place
                e.len += kk;
                return KVW_OK;
            }
        }
        r.reserve(r.size() + 1);
        int32_t s = a->first_fit(kk);
        if (s >= 0) {
            a->take_head(s, kk);
            r.push_back(a->new_extent(s, kk));
            return KVW_OK;
        }
        // no run is long enough: the lowest runs, whole, the last as far as needed
        int32_t need = kk;
        while (need > 0) {
            s = a->first_fit(1);
            const int32_t t = std::min(a->run_len[s], need);
            a->take_head(s, t);
            r.push_back(a->new_extent(s, t));
            need -= t;
        }
        return KVW_OK;
    } catch (const std::bad_alloc &) {
        return fail(KVW_ERR_UNSUPPORTED, "%s: out of host memory", fn);
    }
}

kvw_status kvw_alloc_release(kvw_alloc *a, int32_t row)
{
    if (!row_ok(a, row)) return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_release: bad row %d", row);
    for (int32_t id : a->rows[row]) {
        Extent &e = a->ext[id];
        if (--e.refs > 0) continue;
        if (e.cached) {
            a->lru_push(id);
        } else {
            a->give(e.start, e.len);
            a->drop_extent(id);
        }
    }
    a->rows[row].clear();
    return KVW_OK;
}

kvw_status kvw_alloc_cache_insert(kvw_alloc *a, uint64_t key, int32_t row, int64_t first,
                                  int64_t count)
{
    const char *fn = "kvw_alloc_cache_insert";
    if (!row_ok(a, row)) return fail(KVW_ERR_INVALID_ARG, "%s: no allocator or row %d", fn, row);
    if (first < 0 || count <= 0 || first % a->align || count % a->align)
        return fail(KVW_ERR_INVALID_ARG, "%s: blocks [%lld, +%lld) are not aligned to %d", fn,
                    (long long)first, (long long)count, a->align);
    if (a->cache.find(key) >= 0) return fail(KVW_ERR_INVALID_ARG, "%s: key already cached", fn);
    const int64_t fc = first / a->align, cc = count / a->align;
    std::vector<int32_t> &r = a->rows[row];
    int64_t off = 0;
    size_t i = 0;
    for (; i < r.size(); ++i) {
        const Extent &e = a->ext[r[i]];
        if (off <= fc && fc + cc <= off + e.len) break;
        off += e.len;
    }
    if (i == r.size())
        return fail(KVW_ERR_INVALID_ARG, "%s: blocks [%lld, +%lld) are not inside one extent",
                    fn, (long long)first, (long long)count);
    const int32_t id = r[i];
    if (a->ext[id].cached) return fail(KVW_ERR_INVALID_ARG, "%s: extent already cached", fn);
    try {
        const int32_t head = static_cast<int32_t>(fc - off);
        const int32_t mid = static_cast<int32_t>(cc);
        const int32_t tail = a->ext[id].len - head - mid;
        if (head || tail) {
            // extents are shared only through the cache: this row is the one holder
            r.reserve(r.size() + 2);
            a->ext.reserve(a->ext.size() + 2);
            const int32_t start = a->ext[id].start;
            if (tail) r.insert(r.begin() + i + 1, a->new_extent(start + head + mid, tail));
            if (head) r.insert(r.begin() + i, a->new_extent(start, head));
            a->ext[id].start = start + head;
            a->ext[id].len = mid;
        }
        a->cache.insert(key, id);
        a->ext[id].cached = true;
        a->ext[id].key = key;
        return KVW_OK;
    } catch (const std::bad_alloc &) {
        return fail(KVW_ERR_UNSUPPORTED, "%s: out of host memory", fn);
    }
}

kvw_status kvw_alloc_cache_acquire(kvw_alloc *a, uint64_t key, int32_t row)
{
    const char *fn = "kvw_alloc_cache_acquire";
    if (!row_ok(a, row)) return fail(KVW_ERR_INVALID_ARG, "%s: no allocator or row %d", fn, row);
    const int32_t id = a->cache.find(key);
    if (id < 0) return fail(KVW_ERR_NOT_FOUND, "%s: key not cached", fn);
    try {
        a->rows[row].push_back(id);
    } catch (const std::bad_alloc &) {
        return fail(KVW_ERR_UNSUPPORTED, "%s: out of host memory", fn);
    }
    Extent &e = a->ext[id];
    if (e.refs == 0) a->lru_unlink(id);
    ++e.refs;
    return KVW_OK;
}

kvw_status kvw_alloc_cache_evict(kvw_alloc *a, int64_t max_extents, int64_t *evicted)
{
    if (!a || max_extents < 0)
        return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_cache_evict: no allocator or negative count");
    int64_t k = 0;
    while (k < max_extents && a->lru_head >= 0) {
        a->evict_oldest();
        ++k;
    }
    if (evicted) *evicted = k;
    return KVW_OK;
}

kvw_status kvw_alloc_ranges(const kvw_alloc *a, const int32_t *rows, int32_t n,
                            int32_t range_stride, int32_t *start, int32_t *len, int32_t *cum,
                            int32_t *num_ranges)
{
    const char *fn = "kvw_alloc_ranges";
    if (!a || n < 0 || range_stride < 0 || (n > 0 && (!rows || !num_ranges)) ||
        (n > 0 && range_stride > 0 && (!start || !len || !cum)))
        return fail(KVW_ERR_INVALID_ARG, "%s: bad arguments", fn);
    for (int32_t i = 0; i < n; ++i) {
        if (!row_ok(a, rows[i])) return fail(KVW_ERR_INVALID_ARG, "%s: bad row %d", fn, rows[i]);
        const int64_t c = for_each_range(a, rows[i], [](int64_t, int64_t, int64_t) {});
        if (c > range_stride)
            return fail(KVW_ERR_RANGE_CAP, "%s: row %d has %lld ranges, more than %d", fn, rows[i],
                        (long long)c, range_stride);
    }
    const int64_t A = a->align;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t base = static_cast<int64_t>(i) * range_stride;
        int64_t j = 0;
        const int64_t c = for_each_range(a, rows[i], [&](int64_t s, int64_t l, int64_t cu) {
            start[base + j] = static_cast<int32_t>(s * A);
            len[base + j] = static_cast<int32_t>(l * A);
            cum[base + j] = static_cast<int32_t>(cu * A);
            ++j;
        });
        for (; j < range_stride; ++j) start[base + j] = len[base + j] = cum[base + j] = 0;
        num_ranges[i] = static_cast<int32_t>(c);
    }
    return KVW_OK;
}

kvw_status kvw_alloc_block_table(const kvw_alloc *a, const int32_t *rows, int32_t n,
                                 int32_t stride, int32_t *table, int32_t *counts)
{
    const char *fn = "kvw_alloc_block_table";
    if (!a || n < 0 || stride < 0 || (n > 0 && !rows) || (n > 0 && stride > 0 && !table))
        return fail(KVW_ERR_INVALID_ARG, "%s: bad arguments", fn);
    const int64_t A = a->align;
    for (int32_t i = 0; i < n; ++i) {
        if (!row_ok(a, rows[i])) return fail(KVW_ERR_INVALID_ARG, "%s: bad row %d", fn, rows[i]);
        int64_t blocks = 0;
        for (int32_t id : a->rows[rows[i]]) blocks += a->ext[id].len * A;
        if (blocks > stride)
            return fail(KVW_ERR_RANGE_CAP, "%s: row %d holds %lld blocks, more than %d", fn,
                        rows[i], (long long)blocks, stride);
    }
    for (int32_t i = 0; i < n; ++i) {
        int32_t *out = table + static_cast<int64_t>(i) * stride;
        int64_t q = 0;
        for (int32_t id : a->rows[rows[i]]) {
            const Extent &e = a->ext[id];
            for (int64_t b = e.start * A; b < (e.start + static_cast<int64_t>(e.len)) * A; ++b)
                out[q++] = static_cast<int32_t>(b);
        }
        if (counts) counts[i] = static_cast<int32_t>(q);
        for (; q < stride; ++q) out[q] = 0;
    }
    return KVW_OK;
}

kvw_status kvw_alloc_row_extents(const kvw_alloc *a, int32_t row, int32_t max, int64_t *starts,
                                 int64_t *lens, int32_t *count)
{
    if (!row_ok(a, row) || max < 0 || (max > 0 && (!starts || !lens)))
        return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_row_extents: bad arguments");
    const std::vector<int32_t> &r = a->rows[row];
    for (size_t i = 0; i < r.size() && static_cast<int64_t>(i) < max; ++i) {
        starts[i] = static_cast<int64_t>(a->ext[r[i]].start) * a->align;
        lens[i] = static_cast<int64_t>(a->ext[r[i]].len) * a->align;
    }
    if (count) *count = static_cast<int32_t>(r.size());
    return KVW_OK;
}

kvw_status kvw_alloc_free_runs(const kvw_alloc *a, int64_t max, int64_t *starts, int64_t *lens,
                               int64_t *count)
{
    if (!a || max < 0 || (max > 0 && (!starts || !lens)))
        return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_free_runs: bad arguments");
    int64_t k = 0;
    for (int32_t c = a->c0; c < a->nchunks;) {
        if (a->run_len[c]) {
            if (k < max) {
                starts[k] = static_cast<int64_t>(c) * a->align;
                lens[k] = static_cast<int64_t>(a->run_len[c]) * a->align;
            }
            ++k;
            c += a->run_len[c];
        } else {
            ++c;
        }
    }
    if (count) *count = k;
    return KVW_OK;
}

kvw_status kvw_alloc_lru(const kvw_alloc *a, int64_t max, int64_t *starts, int64_t *lens,
                         int64_t *count)
{
    if (!a || max < 0 || (max > 0 && (!starts || !lens)))
        return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_lru: bad arguments");
    int64_t k = 0;
    for (int32_t id = a->lru_head; id >= 0; id = a->ext[id].next, ++k) {
        if (k < max) {
            starts[k] = static_cast<int64_t>(a->ext[id].start) * a->align;
            lens[k] = static_cast<int64_t>(a->ext[id].len) * a->align;
        }
    }
    if (count) *count = k;
    return KVW_OK;
}

kvw_status kvw_alloc_get_stats(const kvw_alloc *a, kvw_alloc_stats *out)
{
    if (!a || !out) return fail(KVW_ERR_INVALID_ARG, "kvw_alloc_get_stats: NULL argument");
    out->usable_blocks = static_cast<int64_t>(a->nchunks - a->c0) * a->align;
    out->free_blocks = a->free_chunks * a->align;
    out->cache_only_blocks = a->cache_only_chunks * a->align;
    out->free_runs = a->free_runs;
    out->extents = a->live;
    out->cache_entries = static_cast<int64_t>(a->cache.size());
    return KVW_OK;
}

kvw_status kvw_coord_offset(int64_t layer, int64_t block, int64_t token, int64_t num_layers,
                            int64_t num_blocks, int64_t block_size, int64_t bytes_per_token,
                            int64_t *offset)
{
    const kvw_status st = kvw_coord_offset_inline(layer, block, token, num_layers, num_blocks,
                                                  block_size, bytes_per_token, offset);
    if (st == KVW_ERR_INVALID_ARG) return fail(st, "kvw_coord_offset: coordinate out of range");
    if (st != KVW_OK) return fail(st, "kvw_coord_offset: offset overflows int64");
    return KVW_OK;
}

}  // extern "C"
