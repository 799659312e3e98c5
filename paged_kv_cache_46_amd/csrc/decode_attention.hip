// Decode attention over the paged cache: the read path, one query token per
// request (contract: kvw_decode_attention in include/kvw.h).
//
// Sources: "Range-addressed KV cache blocks for the vLLM serving engine",
// "The block-table access pattern" (the attention kernels resolve each
// position's block again) and "The Direction" (M7: range arithmetic in the
// attention kernels).  The attention is the standard scaled dot product.
//
// The work is HBM-bound.  Per position a wave reads 256 B of K and 256 B of V
// for its key/value head and does 2 * G * 128 multiply-adds (G query heads per
// key/value head): about G/2 flop per byte, under 20 TFLOP/s of fp32 vector
// work at 8 TB/s, so matrix cores would buy nothing.
//
// decode_partial_kernel<MODE, G>: one workgroup per (256-position chunk,
// request), one wave per key/value head.
//   0. The workgroup resolves the slots of its positions once, into LDS:
//      the block-table gather (PAGED) or range arithmetic with the wavefront
//      search over range_cum (RANGES).  Every head then reads them from LDS.
//   1. Scores: 16 lanes per position, 8 head dims (16 B of K) per lane; the
//      lane's G query rows sit in registers, pre-scaled; a 4-step xor shuffle
//      sums the 16 partial dot products.  Scores go to LDS.
//   2. The chunk's maximum and exponentials per query head, in LDS.
//   3. Values: the same lane layout accumulates p * V in registers; two xor
//      shuffles fold the four position groups of a wave.  The chunk's
//      (max, sum, weighted values) go to the workspace.
// decode_combine_kernel: per (query head, request), one thread per head dim
// merges the chunks with the usual rescaling by exp(m_c - max m).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kvw.h"
#include "kvw_device.h"
#include "kvw_error.h"

using kvw_detail::fail;

namespace {

constexpr int kChunk = 256;                          // positions per workgroup
constexpr int kHeadDim = 128;                        // supported head_dim
constexpr int kLanesPerRow = kHeadDim / 8;           // 16 lanes x 8 bf16
constexpr int kRowsPerPass = kWave / kLanesPerRow;   // 4 positions per wave pass
constexpr int kUnroll = 4;                           // passes whose loads are issued together
constexpr int kMaxKvHeads = 16;
constexpr int kMaxQHeads = 32;                       // score tile: 32 KiB of LDS

struct DecodeArgs {
    const uint16_t *q;
    const int32_t *context_lens;
    const int32_t *block_table;
    const int32_t *num_blocks_per_req;
    const int32_t *range_start;
    const int32_t *range_len;
    const int32_t *range_cum;
    const int32_t *num_ranges;
    const uint8_t *k_cache;
    const uint8_t *v_cache;
    float *out;
    float *ws_acc;  // [num_reqs][splits][num_q_heads][head_dim]
    float *ws_ml;   // [num_reqs][splits][num_q_heads][2]: chunk max, chunk sum
    int32_t *err_flag;
    int64_t cache_rows;
    int32_t num_reqs;
    int32_t max_context;
    int32_t block_size;
    int32_t table_stride;
    int32_t range_stride;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t splits;
    float scale;
};

__device__ __forceinline__ int32_t context_of(const DecodeArgs &a, int32_t r, uint32_t &flags)
{
    int32_t n = a.context_lens[r];
    if (n < 0) { n = 0; flags |= KVW_FLAG_COUNT; }
    if (n > a.max_context) { n = a.max_context; flags |= KVW_FLAG_COUNT; }
    return n;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Threads per workgroup: one wave per key/value head, at most 16 and at most
// 32 / G (so the G-row register tiles fit the per-thread budget).
template <int G>
constexpr int partial_threads() { return kWave * (G <= 2 ? kMaxKvHeads : kMaxQHeads / G); }

template <int MODE, int G>
__global__ __launch_bounds__(partial_threads<G>()) void decode_partial_kernel(DecodeArgs a)
{
    extern __shared__ float s_p[];           // [num_kv_heads * G][kChunk] scores, then weights
    __shared__ int64_t s_slot[kChunk];
    const int32_t r = blockIdx.y;
    const int32_t c = blockIdx.x;
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);  // a clamp is reported by the combine launch
    flags = 0;
    const int64_t c0 = static_cast<int64_t>(c) * kChunk;
    if (c0 >= n) return;  // uniform over the workgroup: no barrier is skipped by part of it
    const int32_t cnt = static_cast<int32_t>(n - c0 < kChunk ? n - c0 : kChunk);
    const int32_t bs = a.block_size;

    // 0. slots of this chunk's positions, resolved once for every head
    for (int base = 0; base < kChunk; base += blockDim.x) {  // uniform trip count
        const int t = base + static_cast<int>(threadIdx.x);
        const bool in = t < cnt;
        const int64_t p = c0 + t;
        const int64_t lb = in ? p / bs : 0;
        int64_t b = -1;
        if (MODE == KVW_SLOTS_PAGED) {
            if (in) {
                int64_t bound = a.table_stride;
                if (a.num_blocks_per_req)
                    bound = clamp_count(a.num_blocks_per_req[r], a.table_stride, flags);
                if (lb < bound) {
                    b = a.block_table[static_cast<int64_t>(r) * a.table_stride + lb];
                    if (b < 0) { flags |= KVW_FLAG_BAD_BLOCK; b = -1; }
                }
            }
        } else {
            uint32_t nflags = 0;
            const int32_t nr = static_cast<int32_t>(clamp_count(a.num_ranges[r], a.range_stride, nflags));
            if (in) flags |= nflags;
            const int64_t row = static_cast<int64_t>(r) * a.range_stride;
            const int32_t i = wave_upper_index(a.range_cum + row, nr, lb, in);  // every lane calls
            if (in && i >= 0) {
                const int64_t cm = a.range_cum[row + i];
                if (lb >= cm && lb < cm + a.range_len[row + i]) {
                    b = static_cast<int64_t>(a.range_start[row + i]) + (lb - cm);
                    if (b < 0) { flags |= KVW_FLAG_BAD_BLOCK; b = -1; }
                }
            }
        }
        int64_t slot = b < 0 ? -1 : b * bs + (p - lb * bs);
        if (slot >= a.cache_rows) { flags |= KVW_FLAG_SLOT_OOB; slot = -1; }
        if (t < kChunk) s_slot[t] = slot;
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;       // key/value head of this wave
    const int sub = lane % kLanesPerRow;     // which 8 head dims
    const int grp = lane / kLanesPerRow;     // which of the pass's 4 positions
    const int hq0 = w * G;                   // first query head of the group
    const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * kHeadDim * 2;
    const int64_t head_off = static_cast<int64_t>(w) * kHeadDim * 2 + sub * 16;
    float *sp = s_p + static_cast<int64_t>(hq0) * kChunk;

    // 1. scores
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const u32x4 qw = load16<false>(reinterpret_cast<const uint8_t *>(
            a.q + (static_cast<int64_t>(r) * a.num_q_heads + hq0 + g) * kHeadDim + sub * 8));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            qv[g][2 * k] = bf16_lo(qw[k]) * a.scale;
            qv[g][2 * k + 1] = bf16_hi(qw[k]) * a.scale;
        }
    }
    for (int base = 0; base < cnt; base += kRowsPerPass * kUnroll) {
        u32x4 kw[kUnroll];
        int64_t sl[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + u * kRowsPerPass + grp;
            sl[u] = tok < cnt ? s_slot[tok] : -1;
            kw[u] = sl[u] >= 0 ? load16<true>(a.k_cache + sl[u] * row_bytes + head_off) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + u * kRowsPerPass + grp;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    s += qv[g][2 * k] * bf16_lo(kw[u][k]) + qv[g][2 * k + 1] * bf16_hi(kw[u][k]);
                s += __shfl_xor(s, 8);
                s += __shfl_xor(s, 4);
                s += __shfl_xor(s, 2);
                s += __shfl_xor(s, 1);
                if (sub == 0 && tok < cnt) sp[g * kChunk + tok] = sl[u] >= 0 ? s : -INFINITY;
            }
        }
    }
    __syncthreads();

    // 2. maximum and exponentials per query head of the group
    float m[G], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = -INFINITY;
        for (int t = lane; t < cnt; t += kWave) mx = fmaxf(mx, sp[g * kChunk + t]);
#pragma unroll
        for (int o = kWave / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float sum = 0.f;
        for (int t = lane; t < cnt; t += kWave) {
            const float e = mx == -INFINITY ? 0.f : expf(sp[g * kChunk + t] - mx);
            sp[g * kChunk + t] = e;
            sum += e;
        }
#pragma unroll
        for (int o = kWave / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
        m[g] = mx;
        l[g] = sum;
    }
    __syncthreads();

    // 3. weighted values
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[g][k] = 0.f;
    for (int base = 0; base < cnt; base += kRowsPerPass * kUnroll) {
        u32x4 vw[kUnroll];
        int toks[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tok = base + u * kRowsPerPass + grp;
            const int64_t slot = tok < cnt ? s_slot[tok] : -1;
            toks[u] = slot >= 0 ? tok : -1;
            vw[u] = slot >= 0 ? load16<true>(a.v_cache + slot * row_bytes + head_off) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (toks[u] < 0) continue;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = sp[g * kChunk + toks[u]];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc[g][2 * k] += p * bf16_lo(vw[u][k]);
                    acc[g][2 * k + 1] += p * bf16_hi(vw[u][k]);
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            acc[g][k] += __shfl_xor(acc[g][k], 16);
            acc[g][k] += __shfl_xor(acc[g][k], 32);
        }
    const int64_t part = (static_cast<int64_t>(r) * a.splits + c) * a.num_q_heads + hq0;
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float *dst = a.ws_acc + (part + g) * kHeadDim + sub * 8;
#pragma unroll
            for (int k = 0; k < 8; ++k) dst[k] = acc[g][k];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            a.ws_ml[(part + g) * 2] = m[g];
            a.ws_ml[(part + g) * 2 + 1] = l[g];
        }
    }
    raise_flags(a.err_flag, flags);
}

// out[r][h][d] from the chunks of request r: sum_c e^(m_c - M) acc_c[d] / sum_c e^(m_c - M) l_c.
// This launch covers every request whatever max_context is, so it reports a clamped length.
__global__ __launch_bounds__(kHeadDim) void decode_combine_kernel(DecodeArgs a)
{
    const int32_t h = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);
    if (h == 0 && d == 0) raise_flags(a.err_flag, flags);
    const int32_t chunks = (n + kChunk - 1) / kChunk;
    const int64_t base = static_cast<int64_t>(r) * a.splits * a.num_q_heads + h;
    float mx = -INFINITY;
    for (int32_t c = 0; c < chunks; ++c) {
        const int64_t i = base + static_cast<int64_t>(c) * a.num_q_heads;
        if (a.ws_ml[i * 2 + 1] > 0.f) mx = fmaxf(mx, a.ws_ml[i * 2]);
    }
    float num = 0.f, den = 0.f;
    for (int32_t c = 0; c < chunks; ++c) {
        const int64_t i = base + static_cast<int64_t>(c) * a.num_q_heads;
        const float lc = a.ws_ml[i * 2 + 1];
        if (!(lc > 0.f)) continue;
        const float e = expf(a.ws_ml[i * 2] - mx);
        den += e * lc;
        num += e * a.ws_acc[i * kHeadDim + d];
    }
    a.out[(static_cast<int64_t>(r) * a.num_q_heads + h) * kHeadDim + d] = den > 0.f ? num / den : 0.f;
}

int64_t splits_for(int32_t max_context) { return (static_cast<int64_t>(max_context) + kChunk - 1) / kChunk; }

bool aligned_to(const void *p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

template <int MODE>
void launch_partial(int group, dim3 grid, dim3 block, size_t lds, hipStream_t s, const DecodeArgs &a)
{
    switch (group) {
    case 1: hipLaunchKernelGGL((decode_partial_kernel<MODE, 1>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((decode_partial_kernel<MODE, 2>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((decode_partial_kernel<MODE, 4>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((decode_partial_kernel<MODE, 8>), grid, block, lds, s, a); break;
    }
}

}  // namespace

extern "C" {

int64_t kvw_decode_workspace_size(int32_t num_reqs, int32_t max_context, int32_t num_q_heads,
                                  int32_t head_dim)
{
    if (num_reqs < 0 || max_context < 0 || num_q_heads < 0 || head_dim < 0) return -1;
    return static_cast<int64_t>(num_reqs) * splits_for(max_context) * num_q_heads *
           (head_dim + 2) * static_cast<int64_t>(sizeof(float));
}

size_t kvw_decode_args_size(void) { return sizeof(kvw_decode_args); }

kvw_status kvw_decode_attention(const kvw_decode_args *args, void *stream)
{
    const char *fn = "kvw_decode_attention";
    if (!args) return fail(KVW_ERR_INVALID_ARG, "%s: args is NULL", fn);
    const kvw_decode_args &g = *args;
    if (g.mode != KVW_SLOTS_PAGED && g.mode != KVW_SLOTS_RANGES)
        return fail(KVW_ERR_INVALID_ARG, "%s: mode %d is neither paged nor ranges", fn, g.mode);
    if (g.num_reqs < 0 || g.max_context < 0 || g.block_size <= 0 || g.num_blocks < 0 ||
        g.num_q_heads <= 0 || g.num_kv_heads <= 0 || g.num_reqs > 65535)
        return fail(KVW_ERR_INVALID_ARG, "%s: a size is out of range", fn);
    if (g.head_dim != kHeadDim || g.num_kv_heads > kMaxKvHeads || g.num_q_heads > kMaxQHeads ||
        g.num_q_heads % g.num_kv_heads != 0)
        return fail(KVW_ERR_UNSUPPORTED, "%s: head_dim %d, %d query / %d key-value heads not supported",
                    fn, g.head_dim, g.num_q_heads, g.num_kv_heads);
    const int group = g.num_q_heads / g.num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(KVW_ERR_UNSUPPORTED, "%s: %d query heads per key/value head not supported", fn,
                    group);
    if (g.num_blocks > INT64_MAX / g.block_size / g.num_kv_heads / (kHeadDim * 2))
        return fail(KVW_ERR_INVALID_ARG, "%s: cache size overflows", fn);
    if (g.err_flag && !aligned_to(g.err_flag, 4))
        return fail(KVW_ERR_INVALID_ARG, "%s: err_flag misaligned", fn);
    if (g.num_reqs == 0) return KVW_OK;
    if (!g.q || !aligned_to(g.q, 16) || !g.context_lens || !aligned_to(g.context_lens, 4) ||
        !g.out || !aligned_to(g.out, 4))
        return fail(KVW_ERR_INVALID_ARG, "%s: q, context_lens or out is NULL or misaligned", fn);
    if (g.max_context > 0 &&
        (!g.k_cache || !g.v_cache || !aligned_to(g.k_cache, 16) || !aligned_to(g.v_cache, 16)))
        return fail(KVW_ERR_INVALID_ARG, "%s: a cache pointer is NULL or misaligned", fn);
    if (g.mode == KVW_SLOTS_PAGED) {
        if (g.block_table_stride < 0 || (g.block_table_stride > 0 && !g.block_table) ||
            (g.block_table && !aligned_to(g.block_table, 4)) ||
            (g.num_blocks_per_req && !aligned_to(g.num_blocks_per_req, 4)))
            return fail(KVW_ERR_INVALID_ARG, "%s: block table arguments are invalid", fn);
    } else {
        if (g.range_stride < 0) return fail(KVW_ERR_INVALID_ARG, "%s: range_stride is negative", fn);
        if (g.range_stride > KVW_MAX_RANGE_STRIDE)
            return fail(KVW_ERR_RANGE_CAP, "%s: range_stride %d exceeds the cap of %d", fn,
                        g.range_stride, KVW_MAX_RANGE_STRIDE);
        if (!g.range_start || !g.range_len || !g.range_cum || !g.num_ranges ||
            !aligned_to(g.range_start, 4) || !aligned_to(g.range_len, 4) ||
            !aligned_to(g.range_cum, 4) || !aligned_to(g.num_ranges, 4))
            return fail(KVW_ERR_INVALID_ARG, "%s: a range descriptor array is NULL or misaligned", fn);
    }
    const int64_t need = kvw_decode_workspace_size(g.num_reqs, g.max_context, g.num_q_heads, g.head_dim);
    if (need > 0 && (!g.workspace || !aligned_to(g.workspace, 16) || g.workspace_bytes < need))
        return fail(KVW_ERR_INVALID_ARG, "%s: workspace of %lld bytes needed", fn, (long long)need);

    DecodeArgs a{};
    a.q = static_cast<const uint16_t *>(g.q);
    a.context_lens = g.context_lens;
    a.block_table = g.block_table;
    a.num_blocks_per_req = g.num_blocks_per_req;
    a.range_start = g.range_start;
    a.range_len = g.range_len;
    a.range_cum = g.range_cum;
    a.num_ranges = g.num_ranges;
    a.k_cache = static_cast<const uint8_t *>(g.k_cache);
    a.v_cache = static_cast<const uint8_t *>(g.v_cache);
    a.out = g.out;
    a.splits = static_cast<int32_t>(splits_for(g.max_context));
    a.ws_acc = static_cast<float *>(g.workspace);
    a.ws_ml = a.ws_acc + static_cast<int64_t>(g.num_reqs) * a.splits * g.num_q_heads * kHeadDim;
    a.err_flag = g.err_flag;
    a.cache_rows = g.num_blocks * g.block_size;
    a.num_reqs = g.num_reqs;
    a.max_context = g.max_context;
    a.block_size = g.block_size;
    a.table_stride = g.block_table_stride;
    a.range_stride = g.range_stride;
    a.num_q_heads = g.num_q_heads;
    a.num_kv_heads = g.num_kv_heads;
    a.scale = g.scale;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (a.splits > 0) {
        const dim3 grid(static_cast<unsigned>(a.splits), static_cast<unsigned>(g.num_reqs));
        const dim3 block(static_cast<unsigned>(g.num_kv_heads * kWave));
        const size_t lds = static_cast<size_t>(g.num_q_heads) * kChunk * sizeof(float);
        if (g.mode == KVW_SLOTS_PAGED) launch_partial<KVW_SLOTS_PAGED>(group, grid, block, lds, s, a);
        else launch_partial<KVW_SLOTS_RANGES>(group, grid, block, lds, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    hipLaunchKernelGGL(decode_combine_kernel, dim3(static_cast<unsigned>(g.num_q_heads),
                                                   static_cast<unsigned>(g.num_reqs)),
                       dim3(kHeadDim), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KVW_OK;
}

}  // extern "C"
