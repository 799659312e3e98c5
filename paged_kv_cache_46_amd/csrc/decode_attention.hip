// Decode attention over the paged cache: the read path, one query token per
// request (contract: kvw_decode_attention in include/kvw.h).
//
// Sources: "Range-addressed KV cache blocks for the vLLM serving engine",
// "The block-table access pattern" (the attention kernels resolve each
// position's block again) and "The Direction" (M7: range arithmetic in the
// attention kernels).  The attention is the standard scaled dot product.
//
// The work is HBM-bound on paper: per position a wave reads 256 B of K and
// 256 B of V for its key/value head and does 2 * G * 128 multiply-adds (G
// query heads per key/value head), G flop per byte: 32 TFLOP/s at 8 TB/s for
// G = 4.  That is 40% of the fp32 vector rate without packed math, so the
// vector instructions per position are kept few.  For G = 4 and 8 the q.k
// products run on matrix cores (decode_partial_mfma_kernel); for G = 1 and 2
// on v_dot2c_f32_bf16 straight from the bf16 pairs with 16-lane sums on DPP
// adds (decode_partial_kernel).  The exponentials run on v_exp_f32 in base 2,
// and the running maximum is only moved when it grows by more than 2^8.
//
// decode_partial_kernel<MODE, G, L> (G = 1, 2) and decode_partial_mfma_kernel<MODE, G>
// (G = 4, 8): one workgroup per (chunk of 256, 512, 1024 or 2048 positions, request),
// one wave per key/value head, L = 16 lanes per position row for P.V.  At G = 8
// with more than 4 key/value heads, two workgroups share a chunk, half the heads
// each (grid z).
//   0. The workgroup resolves the slots of its positions once, into LDS: the
//      block-table gather (PAGED) or range arithmetic with the wavefront
//      search over range_cum (RANGES).  Positions that hold nothing here
//      (another context-parallel rank's, pad slots) are dropped and the rest
//      packed in order.  Every head reads them from LDS.
//   1. One pass over the chunk: 16 lanes per position, 8 head dims (16 B of
//      K and of V) per lane, four positions per wave and U positions per lane
//      group in flight.  Each lane group keeps, per query head, a running
//      maximum m (log2 units), sum l and weighted values acc (online softmax).
//   2. The four lane groups are merged with cross-row shuffles and the
//      chunk's (m, l, acc) go to the workspace.
// decode_plan_kernel: for batches of 32 requests or more, one workgroup lists
// the (request, chunk) pairs that hold positions: every full chunk first, then
// the requests' last, partial chunks from the longest down (16 length
// classes), so that the short ones fill the last round of workgroups.  The
// partial kernel then takes its pair from the list.  The order decides only
// the schedule: each pair has its own place in the workspace.
// decode_combine_kernel: per (query head, request), 256 threads merge the
// chunks with the rescaling by 2^(m_c - max m): eight slices of the chunks,
// four head dims per thread.  decode_combine_small_kernel: the same with one
// wave per (query head, request) when no request has more than 16 chunks.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kvw.h"
#include "kvw_device.h"
#include "kvw_error.h"

using kvw_detail::fail;

namespace {

constexpr int kMaxChunk = 2048;                      // positions per workgroup, at most
constexpr int kMinChunk = 256;                       // ... and at least; the workspace is sized per 256
constexpr int kPlanThreads = 1024;                   // the plan kernel's one workgroup
constexpr int kTailClasses = 16;                     // length classes of the partial chunks
constexpr int kCombineThreads = 256;                 // combine workgroup: 8 chunk slices x 32 threads
constexpr int kSmallChunks = 16;                     // chunks per request, at most, for the one-wave combine
constexpr int32_t kPlanMinReqs = 32;                 // batches this large get a work list
constexpr int64_t kAutoMinGroups = 256;              // the automatic chunk keeps a workgroup per CU
constexpr int kHeadDim = 128;                        // supported head_dim
constexpr int kRowLanes = 16;                        // lanes per position row of one head (8 was
                                                     // slower: fewer instructions, fewer waves)
constexpr int kMaxKvHeads = 16;                      // 8 when G = 8 (register budget, below)
constexpr float kRescaleLog2 = 8.f;                  // move the running max past this growth
constexpr float kNoMax = -1e30f;                     // running max before any position: finite, so
                                                     // a masked score's weight 2^(-inf - m) is 0
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
    float *ws_ml;   // [num_reqs][splits][num_q_heads][2]: chunk max (log2 units), chunk sum
    int2 *units;         // work list (request, chunk), or NULL: the grid is (chunk, request)
    int32_t *unit_count; // entries of the work list
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
    int32_t chunk;      // positions per workgroup
    int32_t cp_world;   // context parallelism: world size (<= 1: none), this rank, interleave
    int32_t cp_rank;
    int32_t cp_interleave;
    float *lse_out;     // [num_reqs][num_q_heads] natural-log normalizer, or NULL
    float scale_log2;  // scale * log2(e): scores in base-2 exponent units
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

// max(x, the same register of another lane of its row), picked by a DPP control.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x)
{
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY),
                                                               __float_as_int(x), CTRL, 0xF, 0xF,
                                                               false)));
}

// Maximum over the 16 lanes of a row, left in every lane (the pattern of row_sum).
__device__ __forceinline__ float row_max16(float x)
{
    x = dpp_max<0xB1>(x);
    x = dpp_max<0x4E>(x);
    x = dpp_max<0x141>(x);
    x = dpp_max<0x140>(x);
    return x;
}

// x + the same register of another lane of its row, picked by a DPP control.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the L lanes of a row (L = 8 or 16), left in every lane: pair swap,
// quad swap, the mirror inside each half row, then (L = 16) inside the row.
template <int L>
__device__ __forceinline__ float row_sum(float x)
{
    x = dpp_add<0xB1>(x);                   // quad_perm [1,0,3,2]
    x = dpp_add<0x4E>(x);                   // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);                  // row_half_mirror
    if (L == 16) x = dpp_add<0x140>(x);     // row_mirror
    return x;
}

// s + q . k over 8 head dims, from the bf16 pairs.  Each vector element is
// copied to a scalar before the bit cast: a bit cast applied to the element
// expression itself reads the vector's first element.
__device__ __forceinline__ float dot8(const u32x4 &q, const u32x4 &k, float s)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t qi = q[i], ki = k[i];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qi),
                                            __builtin_bit_cast(bf16x2, ki), s, false);
    }
    return s;
}

// Positions in flight per lane group (register budget): 8 at 16 lanes per row,
// 4 at 8 lanes per row, where a lane holds twice the head dims.
template <int L>
constexpr int unroll_of() { return L == 16 ? 8 : 4; }

// Threads per workgroup: one wave per key/value head, at most 16, or 8 for G = 8
// whose 8-row register tiles need more than the 128 VGPRs a 16-wave workgroup
// leaves each wave.
template <int G>
constexpr int partial_threads() { return kWave * (G <= 4 ? kMaxKvHeads : kMaxKvHeads / 2); }

// The slots of positions c0 .. c0+span-1 of request r, resolved once for every
// head and packed into s_slot in position order; returns how many there are.  A
// position that holds nothing here (another context-parallel rank's, or a pad
// slot) takes no place.  Each wave counts its held positions (ballot); the counts
// of the waves before it give its offset.  Every thread of the workgroup calls it.
template <int MODE>
__device__ int32_t stage_slots(const DecodeArgs &a, int32_t r, int64_t c0, int32_t span,
                               int64_t *s_slot, int32_t *s_wave_count, uint32_t &flags)
{
    const int32_t bs = a.block_size;
    const int nwaves = static_cast<int>(blockDim.x) / kWave;
    const int wave_id = static_cast<int>(threadIdx.x) / kWave;
    const int lane_id = static_cast<int>(threadIdx.x) & (kWave - 1);
    int32_t cnt = 0;  // held positions packed so far: the same value in every thread
    for (int base = 0; base < span; base += blockDim.x) {  // uniform trip count
        const int t = base + static_cast<int>(threadIdx.x);
        const bool in = t < span;
        const int64_t p = c0 + t;
        int64_t lb = 0;
        int32_t off = 0;
        // a position of another context-parallel rank holds nothing here: skipped, no flag
        const bool mine = in && cp_locate(p, bs, a.cp_world, a.cp_rank, a.cp_interleave, lb, off);
        int64_t b = -1;
        if (MODE == KVW_SLOTS_PAGED) {
            if (mine) {
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
            if (mine) flags |= nflags;
            const int64_t row = static_cast<int64_t>(r) * a.range_stride;
            const int32_t i = wave_upper_index(a.range_cum + row, nr, lb, mine);  // every lane calls
            if (mine && i >= 0) {
                const int64_t cm = a.range_cum[row + i];
                if (lb >= cm && lb < cm + a.range_len[row + i]) {
                    b = static_cast<int64_t>(a.range_start[row + i]) + (lb - cm);
                    if (b < 0) { flags |= KVW_FLAG_BAD_BLOCK; b = -1; }
                }
            }
        }
        int64_t slot = b < 0 ? -1 : b * bs + off;
        if (slot >= a.cache_rows) { flags |= KVW_FLAG_SLOT_OOB; slot = -1; }
        const bool held = in && slot >= 0;
        const uint64_t mask = __ballot(held);
        if (lane_id == 0) s_wave_count[wave_id] = __popcll(mask);
        __syncthreads();
        int32_t at = cnt;
        for (int i = 0; i < wave_id; ++i) at += s_wave_count[i];
        if (held) s_slot[at + __popcll(mask & ((uint64_t{1} << lane_id) - 1))] = slot;
        for (int i = 0; i < nwaves; ++i) cnt += s_wave_count[i];
        __syncthreads();  // the counts are rewritten by the next round
    }
    return cnt;
}

template <int MODE, int G, int L>
__global__ __launch_bounds__(partial_threads<G>()) void decode_partial_kernel(DecodeArgs a)
{
    static_assert(G == 1 || G == 2, "4 and 8 query heads per key/value head take the matrix-core kernel");
    // G = 2 keeps 6 positions per lane group in flight: 8 would not fit 128 VGPRs
    constexpr int U = G == 2 ? 6 : unroll_of<L>();
    constexpr int NV = kHeadDim / (L * 8);   // 16-byte pieces of a row per lane (1 or 2)
    constexpr int DPL = NV * 8;              // head dims per lane
    constexpr int RPP = kWave / L;           // positions per wave load
    __shared__ int64_t s_slot[kMaxChunk];
    int32_t r, c;
    if (a.units) {
        if (static_cast<int32_t>(blockIdx.x) >= *a.unit_count) return;  // uniform
        const int2 rc = a.units[blockIdx.x];
        r = rc.x;
        c = rc.y;
    } else {
        r = blockIdx.y;
        c = blockIdx.x;
    }
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);  // a clamp is reported by the combine launch
    flags = 0;
    const int64_t c0 = static_cast<int64_t>(c) * a.chunk;
    if (c0 >= n) return;  // uniform over the workgroup: no barrier is skipped by part of it
    const int32_t span = static_cast<int32_t>(n - c0 < a.chunk ? n - c0 : a.chunk);

    // 0. slots of this chunk's positions, resolved once for every head, packed in LDS
    __shared__ int32_t s_wave_count[kMaxKvHeads];
    const int32_t cnt = stage_slots<MODE>(a, r, c0, span, s_slot, s_wave_count, flags);

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;       // key/value head of this wave
    const int sub = lane % L;                // which DPL head dims
    const int grp = lane / L;                // which of the RPP positions of a wave load
    const int hq0 = w * G;                   // first query head of the group
    const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * kHeadDim * 2;
    const int64_t head_off = static_cast<int64_t>(w) * kHeadDim * 2 + sub * DPL * 2;
    const uint8_t *kb = a.k_cache + head_off;
    const uint8_t *vb = a.v_cache + head_off;

    u32x4 qw[G][NV];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < NV; ++j)
            qw[g][j] = load16<false>(reinterpret_cast<const uint8_t *>(
                a.q + (static_cast<int64_t>(r) * a.num_q_heads + hq0 + g) * kHeadDim + sub * DPL + 8 * j));

    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNoMax;
        l[g] = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[g][k] = 0.f;
    }

    // 1. one pass: scores, running maximum, weights and weighted values
    for (int base = 0; base < cnt; base += RPP * U) {  // uniform trip count
        u32x4 kw[U][NV], vw[U][NV];
        bool ok[U];
        // All K loads, then all V loads, none under a branch (a lane without a
        // position reads row 0, in the cache whenever the chunk holds a position, and
        // drops the value): the scores then wait only for K while V is in flight.
        int64_t sl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = base + u * RPP + grp;
            const int64_t s_ = tok < cnt ? s_slot[tok] : -1;
            ok[u] = s_ >= 0;
            sl[u] = ok[u] ? s_ : 0;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const u32x4 t = load16<true>(kb + sl[u] * row_bytes + 16 * j);
                kw[u][j] = ok[u] ? t : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const u32x4 t = load16<true>(vb + sl[u] * row_bytes + 16 * j);
                vw[u][j] = ok[u] ? t : u32x4{0, 0, 0, 0};
            }
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float t = 0.f;
#pragma unroll
                for (int j = 0; j < NV; ++j) t = dot8(qw[g][j], kw[u][j], t);
                t = row_sum<L>(t) * a.scale_log2;  // every lane
                sc[u][g] = ok[u] ? t : -INFINITY;
            }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = sc[0][g];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
            if (mx > m[g] + kRescaleLog2) {  // also at the first position (m = kNoMax)
                const float alpha = __builtin_amdgcn_exp2f(m[g] - mx);
                l[g] *= alpha;
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[g][k] *= alpha;
                m[g] = mx;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[DPL];
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    vf[8 * j + 2 * k] = bf16_lo(vw[u][j][k]);
                    vf[8 * j + 2 * k + 1] = bf16_hi(vw[u][j][k]);
                }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = __builtin_amdgcn_exp2f(sc[u][g] - m[g]);  // 0 for a masked score
                l[g] += p;
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[g][k] += p * vf[k];
            }
        }
    }

    // 2. merge the lane groups (cross-row shuffles), then store the chunk's partials.  A group
    // that saw no position keeps m = kNoMax and l = 0, so its factor is 0 or multiplies zeros.
#pragma unroll
    for (int o = L; o < kWave; o <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], o);
            const float lo = __shfl_xor(l[g], o);
            const float mm = fmaxf(m[g], mo);
            const float ea = __builtin_amdgcn_exp2f(m[g] - mm);
            const float eb = __builtin_amdgcn_exp2f(mo - mm);
            l[g] = l[g] * ea + lo * eb;
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[g][k] = acc[g][k] * ea + __shfl_xor(acc[g][k], o) * eb;
            m[g] = mm;
        }
    }
    const int64_t part = (static_cast<int64_t>(r) * a.splits + c) * a.num_q_heads + hq0;
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float *dst = a.ws_acc + (part + g) * kHeadDim + sub * DPL;
#pragma unroll
            for (int k = 0; k < DPL; ++k) dst[k] = acc[g][k];
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

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a)
{
    __shared__ int32_t s_full, s_full_cur, s_total;
    __shared__ int32_t s_cls[kTailClasses], s_base[kTailClasses], s_cur[kTailClasses];
    const int tid = threadIdx.x;
    if (tid == 0) { s_full = 0; s_full_cur = 0; }
    if (tid < kTailClasses) { s_cls[tid] = 0; s_cur[tid] = 0; }
    __syncthreads();
    for (int32_t r = tid; r < a.num_reqs; r += kPlanThreads) {
        uint32_t unused = 0;
        const int32_t n = context_of(a, r, unused);  // clamps are reported by the combine launch
        const int32_t nf = n / a.chunk, rem = n % a.chunk;
        if (nf) atomicAdd(&s_full, nf);
        if (rem) atomicAdd(&s_cls[(rem - 1) * kTailClasses / a.chunk], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int32_t base = s_full;
        for (int k = kTailClasses - 1; k >= 0; --k) {
            s_base[k] = base;
            base += s_cls[k];
        }
        s_total = base;
    }
    __syncthreads();
    for (int32_t r = tid; r < a.num_reqs; r += kPlanThreads) {
        uint32_t unused = 0;
        const int32_t n = context_of(a, r, unused);
        const int32_t nf = n / a.chunk, rem = n % a.chunk;
        if (nf) {
            const int32_t at = atomicAdd(&s_full_cur, nf);
            for (int32_t i = 0; i < nf; ++i) a.units[at + i] = make_int2(r, i);
        }
        if (rem) {
            const int k = (rem - 1) * kTailClasses / a.chunk;
            a.units[s_base[k] + atomicAdd(&s_cur[k], 1)] = make_int2(r, nf);
        }
    }
    if (tid == 0) *a.unit_count = s_total;
}

// q.k on matrix cores for G = 4 or 8 query heads per key/value head (one wave
// per key/value head, tiles of 16 positions).  The scores of a tile are one
// 16 x 16 product over 4 steps of 32 head dims (v_mfma_f32_16x16x32_bf16: lane
// l holds the query rows' dims 8*(l/16) .. +8 of step k as the A operand, the K
// row of position l%16 as the B operand, and gets scores of rows 4*(l/16) .. +3,
// column l%16).  The G query heads fill rows 0..G-1; the other rows are zero and
// masked.  The
// softmax runs in that layout (a row's maximum over the tile's 16 positions by
// DPP, one exponential per lane and row), and the weights and the rescale factors
// go through a per-wave LDS tile to the P.V lanes, which accumulate in fp32 on
// the vector units as in decode_partial_kernel (16 lanes per position row).
template <int MODE, int G>
__global__ __launch_bounds__(partial_threads<G>()) void decode_partial_mfma_kernel(DecodeArgs a)
{
    constexpr int kTile = 16;
    constexpr int kWaves = partial_threads<G>() / kWave;
    __shared__ int64_t s_slot[kMaxChunk];
    __shared__ int32_t s_wave_count[kMaxKvHeads];
    __shared__ __attribute__((aligned(16))) float s_p[kWaves][kTile][16];  // [position][row]
    __shared__ __attribute__((aligned(16))) float s_alpha[kWaves][16];
    int32_t r, c;
    if (a.units) {
        if (static_cast<int32_t>(blockIdx.x) >= *a.unit_count) return;  // uniform
        const int2 rc = a.units[blockIdx.x];
        r = rc.x;
        c = rc.y;
    } else {
        r = blockIdx.y;
        c = blockIdx.x;
    }
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);  // a clamp is reported by the combine launch
    flags = 0;
    const int64_t c0 = static_cast<int64_t>(c) * a.chunk;
    if (c0 >= n) return;  // uniform over the workgroup
    const int32_t span = static_cast<int32_t>(n - c0 < a.chunk ? n - c0 : a.chunk);
    const int32_t cnt = stage_slots<MODE>(a, r, c0, span, s_slot, s_wave_count, flags);

    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;       // wave of the workgroup: its LDS tile
    // key/value head of this wave: the workgroups of a chunk split the heads (blockIdx.z)
    const int kvh = static_cast<int>(blockIdx.z * (blockDim.x / kWave)) + w;
    if (kvh >= a.num_kv_heads) return;       // no block-wide barrier follows the staging
    const int col = lane % kTile;            // MFMA side: position of the tile; P.V side: dims
    const int rg = lane / kTile;             // MFMA side: rows 4*rg .. +3; P.V side: position group
    const int hq0 = kvh * G;
    const int64_t row_bytes = static_cast<int64_t>(a.num_kv_heads) * kHeadDim * 2;
    const uint8_t *kbase = a.k_cache + static_cast<int64_t>(kvh) * kHeadDim * 2 + rg * 16;
    const uint8_t *vbase = a.v_cache + static_cast<int64_t>(kvh) * kHeadDim * 2 + col * 16;

    bf16x8 qa[4];  // A operand: query row col, dims 32*k + 8*rg .. +8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (col < G)
            v = load16<false>(reinterpret_cast<const uint8_t *>(
                a.q + (static_cast<int64_t>(r) * a.num_q_heads + hq0 + col) * kHeadDim + 32 * k + 8 * rg));
        qa[k] = __builtin_bit_cast(bf16x8, v);
    }
    float m[4];                   // MFMA side: running maximum of rows 4*rg + i
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = kNoMax;
    float l[G], acc[G][8];        // P.V side
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[g][k] = 0.f;
    }
    float *tile = &s_p[w][0][0];
    float *alpha_row = &s_alpha[w][0];

    // K of the first tile (position col) as the B operand.  Within a chunk that
    // holds a position (cnt > 0, uniform) every load below is unconditional: a
    // lane without a position reads row 0, which is then in the cache, and drops
    // the value.  Loads under a per-lane branch would make the compiler wait for
    // all of them before the first product; in straight code it waits only for
    // the loads the product needs.  A chunk with no position reads nothing (the
    // cache may then have no rows at all).
    int64_t slk = col < cnt ? s_slot[col] : -1;
    u32x4 kw[4] = {};
    if (cnt > 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 t = load16<false>(kbase + (slk >= 0 ? slk : 0) * row_bytes + 64 * k);
            kw[k] = slk >= 0 ? t : u32x4{0, 0, 0, 0};
        }
    }
    for (int tb = 0; tb < cnt; tb += kTile) {  // uniform trip count
        // loads: K of position tb + col as the B operand, V of positions tb + 4u + rg.
        // One K load covers 64 B of each of 16 rows, so every 128 B line is split
        // over two loads: K goes through the cache with the default policy (with
        // the streaming hint 2% of the lines were fetched twice).  V loads cover
        // whole rows and keep the hint (without it the kernel is 11% slower).
        // This tile's K (kw, slot slk) was loaded during the previous tile; the next
        // tile's K goes out here, after this tile's V, and arrives while this tile's
        // scores, softmax and P.V run.
        u32x4 vw[4], kn[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tv = tb + 4 * u + rg;
            const int64_t slv = tv < cnt ? s_slot[tv] : -1;
            const u32x4 t = load16<true>(vbase + (slv >= 0 ? slv : 0) * row_bytes);
            vw[u] = slv >= 0 ? t : u32x4{0, 0, 0, 0};
        }
        const int tn = tb + kTile + col;
        const int64_t sln = tn < cnt ? s_slot[tn] : -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 t = load16<false>(kbase + (sln >= 0 ? sln : 0) * row_bytes + 64 * k);
            kn[k] = sln >= 0 ? t : u32x4{0, 0, 0, 0};
        }
        // scores of the tile: rows 4*rg + i, column col
        f32x4 sc4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            sc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], __builtin_bit_cast(bf16x8, kw[k]),
                                                          sc4, 0, 0, 0);
        float p[4], alpha[4];
        bool moved = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sc = (slk >= 0 && 4 * rg + i < G) ? sc4[i] * a.scale_log2 : -INFINITY;
            const float mx = row_max16(sc);
            alpha[i] = 1.f;
            if (mx > m[i] + kRescaleLog2) {  // also at the first position (m = kNoMax)
                alpha[i] = __builtin_amdgcn_exp2f(m[i] - mx);
                m[i] = mx;
                moved = true;
            }
            p[i] = __builtin_amdgcn_exp2f(sc - m[i]);  // 0 for a masked score
        }
        // to the P.V side: weights [position][row] and the rows' rescale factors
        *reinterpret_cast<f32x4 *>(tile + col * 16 + 4 * rg) = f32x4{p[0], p[1], p[2], p[3]};
        if (col == 0) *reinterpret_cast<f32x4 *>(alpha_row + 4 * rg) = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (__ballot(moved)) {  // uniform: some row of the wave moved its maximum
            float al[G];
#pragma unroll
            for (int j = 0; j < G / 4; ++j) {
                const f32x4 aj = *reinterpret_cast<const f32x4 *>(alpha_row + 4 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i) al[4 * j + i] = aj[i];
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                l[g] *= al[g];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[g][k] *= al[g];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float pv[G];
#pragma unroll
            for (int j = 0; j < G / 4; ++j) {
                const f32x4 pj = *reinterpret_cast<const f32x4 *>(tile + (4 * u + rg) * 16 + 4 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[4 * j + i] = pj[i];
            }
            float vf[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vf[2 * k] = bf16_lo(vw[u][k]);
                vf[2 * k + 1] = bf16_hi(vw[u][k]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                l[g] += pv[g];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[g][k] += pv[g] * vf[k];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the tile is rewritten by the next iteration
#pragma unroll
        for (int k = 0; k < 4; ++k) kw[k] = kn[k];
        slk = sln;
    }

    // the four P.V position groups share each row's maximum: plain sums across them
#pragma unroll
    for (int o = kTile; o < kWave; o <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            l[g] += __shfl_xor(l[g], o);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[g][k] += __shfl_xor(acc[g][k], o);
        }
    }
    const int64_t part = (static_cast<int64_t>(r) * a.splits + c) * a.num_q_heads + hq0;
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float *dst = a.ws_acc + (part + g) * kHeadDim + col * 8;
#pragma unroll
            for (int k = 0; k < 8; ++k) dst[k] = acc[g][k];
        }
    }
    if (col == 0 && 4 * rg < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a.ws_ml[(part + 4 * rg + i) * 2] = m[i];
            a.ws_ml[(part + 4 * rg + i) * 2 + 1] = l[4 * rg + i];
        }
    }
    raise_flags(a.err_flag, flags);
}

// out[r][h][d] from the chunks of request r:
//   sum_c 2^(m_c - M) acc_c[d] / sum_c 2^(m_c - M) l_c,  M = max of m_c over chunks with l_c > 0.
// Two load phases, so that few memory round trips stand between launch and result:
//   1. every thread reads the (m, l) of chunks tid, tid + 256, ... and the
//      workgroup's maximum M follows from wave shuffles and one barrier;
//   2. thread (slice, quad) sums, over chunks slice, slice + 8, ..., the weighted
//      acc of head dims 4*quad .. +3 (one 16-byte load per chunk, 16 chunks in
//      flight) and the weighted l; the eight slices are added in LDS.
// This launch covers every request whatever max_context is, so it reports a
// clamped length.
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a)
{
    constexpr int kQuads = kHeadDim / 4;
    constexpr int kSlices = kCombineThreads / kQuads;
    __shared__ float s_max[kCombineThreads / kWave];
    __shared__ __attribute__((aligned(16))) float s_num[kSlices][kHeadDim];
    __shared__ float s_den[kSlices];
    const int32_t h = blockIdx.x, r = blockIdx.y;
    const int tid = threadIdx.x, quad = tid % kQuads, slice = tid / kQuads;
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);
    if (h == 0 && tid == 0) raise_flags(a.err_flag, flags);
    const int32_t chunks = static_cast<int32_t>((static_cast<int64_t>(n) + a.chunk - 1) / a.chunk);
    const int64_t base = static_cast<int64_t>(r) * a.splits * a.num_q_heads + h;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + base;  // (m, l) of chunk c at c*Hq
    const int64_t step = a.num_q_heads;

    float mx = -INFINITY;
    for (int32_t c = tid; c < chunks; c += kCombineThreads) {
        const float2 v = ml[c * step];
        if (v.y > 0.f) mx = fmaxf(mx, v.x);
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & (kWave - 1)) == 0) s_max[tid / kWave] = mx;
    __syncthreads();
    mx = s_max[0];
#pragma unroll
    for (int i = 1; i < kCombineThreads / kWave; ++i) mx = fmaxf(mx, s_max[i]);

    float num0 = 0.f, num1 = 0.f, num2 = 0.f, num3 = 0.f, den = 0.f;
    const f32x4 *acc = reinterpret_cast<const f32x4 *>(a.ws_acc + base * kHeadDim) + quad;
    const int64_t acc_step = static_cast<int64_t>(a.num_q_heads) * (kHeadDim / 4);
#pragma unroll 16
    for (int32_t c = slice; c < chunks; c += kSlices) {
        const float2 v = ml[c * step];
        const f32x4 x = acc[c * acc_step];
        const float e = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
        num0 += e * x[0];
        num1 += e * x[1];
        num2 += e * x[2];
        num3 += e * x[3];
        den += e * v.y;
    }
    *reinterpret_cast<f32x4 *>(&s_num[slice][4 * quad]) = f32x4{num0, num1, num2, num3};
    if (quad == 0) s_den[slice] = den;
    __syncthreads();
    if (tid < kHeadDim) {
        float sum = s_num[0][tid], dsum = s_den[0];
#pragma unroll
        for (int i = 1; i < kSlices; ++i) {
            sum += s_num[i][tid];
            dsum += s_den[i];
        }
        a.out[(static_cast<int64_t>(r) * a.num_q_heads + h) * kHeadDim + tid] = dsum > 0.f ? sum / dsum : 0.f;
        // log sum_j e^(s_j) = ln 2 * (M + log2(den)), scores in base-2 units; -inf with no position
        if (a.lse_out && tid == 0)
            a.lse_out[static_cast<int64_t>(r) * a.num_q_heads + h] =
                dsum > 0.f ? (mx + log2f(dsum)) * kLn2 : -INFINITY;
    }
}

// The same merge when no request has more than kSmallChunks chunks: one wave per
// (query head, request), two head dims per lane, four query heads per workgroup.
// Every lane reads the (m, l) of all the request's chunks (one address per load,
// shared by the wave), so the maximum needs no exchange between lanes, and the
// acc loads do not wait for it: one memory round trip and no barrier, where the
// general kernel's 256-thread workgroup per head is mostly idle at a few chunks.
// The sums run over the chunks in order.  Reports a clamped length like the
// general kernel.
__global__ __launch_bounds__(kCombineThreads) void decode_combine_small_kernel(DecodeArgs a)
{
    const int32_t h = static_cast<int32_t>(blockIdx.x) * (kCombineThreads / kWave) +
                      static_cast<int32_t>(threadIdx.x) / kWave;
    const int32_t r = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t flags = 0;
    const int32_t n = context_of(a, r, flags);
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_flags(a.err_flag, flags);
    if (h >= a.num_q_heads) return;  // uniform over the wave; nothing below waits on others
    const int32_t chunks = static_cast<int32_t>((static_cast<int64_t>(n) + a.chunk - 1) / a.chunk);
    const int64_t base = static_cast<int64_t>(r) * a.splits * a.num_q_heads + h;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + base;
    const float2 *acc = reinterpret_cast<const float2 *>(a.ws_acc + base * kHeadDim) + lane;
    const int64_t step = a.num_q_heads;
    const int64_t acc_step = static_cast<int64_t>(a.num_q_heads) * (kHeadDim / 2);
    float2 v[kSmallChunks], x[kSmallChunks];
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c) {
        v[c] = make_float2(0.f, 0.f);
        x[c] = make_float2(0.f, 0.f);
        if (c < chunks) {
            v[c] = ml[c * step];
            x[c] = acc[c * acc_step];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c)
        if (v[c].y > 0.f) mx = fmaxf(mx, v[c].x);
    float num0 = 0.f, num1 = 0.f, den = 0.f;
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c) {
        const float e = v[c].y > 0.f ? __builtin_amdgcn_exp2f(v[c].x - mx) : 0.f;
        num0 += e * x[c].x;
        num1 += e * x[c].y;
        den += e * v[c].y;
    }
    // out is only 4-byte aligned: two scalar stores
    float *dst = a.out + (static_cast<int64_t>(r) * a.num_q_heads + h) * kHeadDim + 2 * lane;
    dst[0] = den > 0.f ? num0 / den : 0.f;
    dst[1] = den > 0.f ? num1 / den : 0.f;
    // log sum_j e^(s_j) = ln 2 * (M + log2(den)), scores in base-2 units; -inf with no position
    if (a.lse_out && lane == 0)
        a.lse_out[static_cast<int64_t>(r) * a.num_q_heads + h] =
            den > 0.f ? (mx + log2f(den)) * kLn2 : -INFINITY;
}

// out[r][h][d] = sum_p e^(lse_p - L) out_p[r][h][d], L = log sum_p e^(lse_p), over the parts'
// stacked results; a part with lse -inf (no position) adds nothing; no part with a position
// gives 0 and -inf.
__global__ __launch_bounds__(1024) void decode_merge_kernel(int32_t parts, int32_t num_reqs,
                                                            int32_t num_q_heads, int32_t head_dim,
                                                            const float *outs, const float *lses,
                                                            float *out, float *lse_out)
{
    const int32_t h = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
    const int64_t row = static_cast<int64_t>(r) * num_q_heads + h;
    const int64_t part_rows = static_cast<int64_t>(num_reqs) * num_q_heads;
    float mx = -INFINITY;
    for (int32_t p = 0; p < parts; ++p) mx = fmaxf(mx, lses[p * part_rows + row]);
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
        for (int32_t p = 0; p < parts; ++p) {
            const float e = __builtin_amdgcn_exp2f((lses[p * part_rows + row] - mx) * kLog2e);
            den += e;
            num += e * outs[(p * part_rows + row) * head_dim + d];
        }
    }
    out[row * head_dim + d] = den > 0.f ? num / den : 0.f;
    if (lse_out && d == 0) lse_out[row] = den > 0.f ? mx + log2f(den) * kLn2 : -INFINITY;
}

int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

// The automatic chunk length: the longest of 2048, 1024, 512 and 256 positions
// that still gives every compute unit a workgroup, num_reqs * ceil(max_context /
// chunk) >= 256.  Longer chunks spread each workgroup's fixed cost (slot staging,
// the partial's write) over more positions; fewer workgroups than compute units
// leave some idle.  A batch of 32 requests or more, which gets the work list,
// stops at 1024: its requests are often uneven, and longer chunks leave its last
// round of workgroups partly empty (the 256-request decode step with contexts
// U[1, 8192] is 4% slower at 2048).  Only num_reqs and max_context are known here.
int32_t auto_chunk(int32_t num_reqs, int32_t max_context)
{
    int32_t c = num_reqs < kPlanMinReqs ? kMaxChunk : kMaxChunk / 2;
    while (c > kMinChunk && static_cast<int64_t>(num_reqs) * ceil_div(max_context, c) < kAutoMinGroups) c /= 2;
    return c;
}

bool aligned_to(const void *p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; }

template <int MODE>
void launch_partial(int group, dim3 grid, dim3 block, size_t lds, hipStream_t s, const DecodeArgs &a)
{
    switch (group) {
    case 1: hipLaunchKernelGGL((decode_partial_kernel<MODE, 1, kRowLanes>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((decode_partial_kernel<MODE, 2, kRowLanes>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((decode_partial_mfma_kernel<MODE, 4>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((decode_partial_mfma_kernel<MODE, 8>), grid, block, lds, s, a); break;
    }
}

// The workspace of kvw_decode_attention_noalloc: one array per GPU, held from the
// library's load on that GPU until the process ends.  Host code never passes
// `scratch` itself (on the host the name is a stand-in, not a device address):
// static_workspace() looks up each GPU's address once, with that GPU current.
static __device__ __align__(256) uint8_t scratch[KVW_DECODE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of this GPU's `scratch` (the GPU of `stream`, or the current
// one for the null stream).
kvw_status static_workspace(hipStream_t stream, const char *fn, void **out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: no device for the stream: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVW_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(KVW_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(KVW_ERR_HIP, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(e));
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr)
            return fail(KVW_ERR_HIP, "%s: hipGetSymbolAddress of the static workspace on device %d: %s",
                        fn, dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KVW_OK;
}

}  // namespace

extern "C" {

int64_t kvw_decode_workspace_size(int32_t num_reqs, int32_t max_context, int32_t num_q_heads,
                                  int32_t head_dim)
{
    if (num_reqs < 0 || max_context < 0 || num_q_heads < 0 || head_dim < 0) return -1;
    // chunk partials (head_dim sums, max, sum per query head) and one work-list entry per chunk,
    // counted per 256 positions so that every chunk length fits; then the list's length.
    // -1 when the size does not fit int64.
    int64_t per_chunk = 0, chunks = 0, bytes = 0;
    if (__builtin_mul_overflow(static_cast<int64_t>(num_q_heads),
                               (static_cast<int64_t>(head_dim) + 2) * static_cast<int64_t>(sizeof(float)),
                               &per_chunk) ||
        __builtin_add_overflow(per_chunk, static_cast<int64_t>(sizeof(int2)), &per_chunk) ||
        __builtin_mul_overflow(static_cast<int64_t>(num_reqs), ceil_div(max_context, kMinChunk), &chunks) ||
        __builtin_mul_overflow(chunks, per_chunk, &bytes) || __builtin_add_overflow(bytes, int64_t{16}, &bytes))
        return -1;
    return bytes;
}

size_t kvw_decode_args_size(void) { return sizeof(kvw_decode_args); }

kvw_status kvw_decode_merge(int32_t num_parts, int32_t num_reqs, int32_t num_q_heads,
                            int32_t head_dim, const float *outs, const float *lses, float *out,
                            float *lse_out, void *stream)
{
    const char *fn = "kvw_decode_merge";
    if (num_parts < 1 || num_reqs < 0 || num_reqs > 65535 || num_q_heads <= 0 ||
        num_q_heads > 65535 || head_dim <= 0 || head_dim > 1024)
        return fail(KVW_ERR_INVALID_ARG, "%s: a size is out of range", fn);
    if (num_reqs == 0) return KVW_OK;
    if (!outs || !lses || !out || !aligned_to(outs, 4) || !aligned_to(lses, 4) ||
        !aligned_to(out, 4) || (lse_out && !aligned_to(lse_out, 4)))
        return fail(KVW_ERR_INVALID_ARG, "%s: a pointer is NULL or misaligned", fn);
    hipLaunchKernelGGL(decode_merge_kernel,
                       dim3(static_cast<unsigned>(num_q_heads), static_cast<unsigned>(num_reqs)),
                       dim3(static_cast<unsigned>(head_dim)), 0, reinterpret_cast<hipStream_t>(stream),
                       num_parts, num_reqs, num_q_heads, head_dim, outs, lses, out, lse_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KVW_OK;
}

// kvw_decode_attention with the workspace from args (use_static false) or from
// this GPU's static array (kvw_decode_attention_noalloc).
static kvw_status decode_attention_run(const kvw_decode_args *args, void *stream, const char *fn,
                                       bool use_static)
{
    if (!args) return fail(KVW_ERR_INVALID_ARG, "%s: args is NULL", fn);
    const kvw_decode_args &g = *args;
    if (g.mode != KVW_SLOTS_PAGED && g.mode != KVW_SLOTS_RANGES)
        return fail(KVW_ERR_INVALID_ARG, "%s: mode %d is neither paged nor ranges", fn, g.mode);
    if (g.num_reqs < 0 || g.max_context < 0 || g.block_size <= 0 || g.num_blocks < 0 ||
        g.num_q_heads <= 0 || g.num_kv_heads <= 0 || g.num_reqs > 65535)
        return fail(KVW_ERR_INVALID_ARG, "%s: a size is out of range", fn);
    if (g.head_dim != kHeadDim || g.num_kv_heads > kMaxKvHeads || g.num_q_heads % g.num_kv_heads != 0)
        return fail(KVW_ERR_UNSUPPORTED, "%s: head_dim %d, %d query / %d key-value heads not supported",
                    fn, g.head_dim, g.num_q_heads, g.num_kv_heads);
    const int group = g.num_q_heads / g.num_kv_heads;
    if ((group != 1 && group != 2 && group != 4 && group != 8) ||
        g.num_kv_heads > (group <= 4 ? kMaxKvHeads : kMaxKvHeads / 2))
        return fail(KVW_ERR_UNSUPPORTED, "%s: %d query heads over %d key/value heads not supported",
                    fn, g.num_q_heads, g.num_kv_heads);
    if (g.num_blocks > INT64_MAX / g.block_size / g.num_kv_heads / (kHeadDim * 2))
        return fail(KVW_ERR_INVALID_ARG, "%s: cache size overflows", fn);
    if (g.chunk_positions != 0 && g.chunk_positions != 256 && g.chunk_positions != 512 &&
        g.chunk_positions != 1024 && g.chunk_positions != 2048)
        return fail(KVW_ERR_INVALID_ARG, "%s: chunk_positions %d is not 0, 256, 512, 1024 or 2048",
                    fn, g.chunk_positions);
    if (g.err_flag && !aligned_to(g.err_flag, 4))
        return fail(KVW_ERR_INVALID_ARG, "%s: err_flag misaligned", fn);
    if (g.lse_out && !aligned_to(g.lse_out, 4))
        return fail(KVW_ERR_INVALID_ARG, "%s: lse_out misaligned", fn);
    {
        const kvw_status st = kvw_detail::check_cp(fn, g.block_size, g.cp_world_size, g.cp_rank,
                                                    g.cp_interleave_size);
        if (st != KVW_OK) return st;
    }
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
    const int32_t chunk = g.chunk_positions ? g.chunk_positions : auto_chunk(g.num_reqs, g.max_context);
    const int32_t splits = static_cast<int32_t>(ceil_div(g.max_context, chunk));
    const int64_t units = static_cast<int64_t>(g.num_reqs) * splits;
    const bool plan = g.num_reqs >= kPlanMinReqs && units <= INT32_MAX;
    void *workspace = g.workspace;
    if (!use_static) {
        const int64_t need = kvw_decode_workspace_size(g.num_reqs, g.max_context, g.num_q_heads, g.head_dim);
        if (need < 0) return fail(KVW_ERR_INVALID_ARG, "%s: the workspace size overflows", fn);
        if (need > 0 && (!g.workspace || !aligned_to(g.workspace, 16) || g.workspace_bytes < need))
            return fail(KVW_ERR_INVALID_ARG, "%s: workspace of %lld bytes needed", fn, (long long)need);
    } else {
        // what this call's chunks need: partials, then the work list and its length
        const int64_t need = units * g.num_q_heads * (kHeadDim + 2) * static_cast<int64_t>(sizeof(float)) +
                             (plan ? units * static_cast<int64_t>(sizeof(int2)) + 4 : 0);
        if (need > KVW_DECODE_STATIC_WORKSPACE_BYTES)
            return fail(KVW_ERR_UNSUPPORTED, "%s: %lld bytes of workspace needed, the static one holds %lld",
                        fn, (long long)need, (long long)KVW_DECODE_STATIC_WORKSPACE_BYTES);
        const kvw_status st = static_workspace(reinterpret_cast<hipStream_t>(stream), fn, &workspace);
        if (st != KVW_OK) return st;
    }

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
    a.chunk = chunk;
    a.cp_world = g.cp_world_size;
    a.cp_rank = g.cp_rank;
    a.cp_interleave = g.cp_interleave_size > 0 ? g.cp_interleave_size : 1;
    a.lse_out = g.lse_out;
    a.splits = splits;
    a.ws_acc = static_cast<float *>(workspace);
    a.ws_ml = a.ws_acc + static_cast<int64_t>(g.num_reqs) * a.splits * g.num_q_heads * kHeadDim;
    // the list follows the partials: an 8-byte aligned offset (two floats per entry above)
    a.units = plan ? reinterpret_cast<int2 *>(a.ws_ml + units * g.num_q_heads * 2) : nullptr;
    a.unit_count = plan ? reinterpret_cast<int32_t *>(a.units + units) : nullptr;
    a.err_flag = g.err_flag;
    a.cache_rows = g.num_blocks * g.block_size;
    a.num_reqs = g.num_reqs;
    a.max_context = g.max_context;
    a.block_size = g.block_size;
    a.table_stride = g.block_table_stride;
    a.range_stride = g.range_stride;
    a.num_q_heads = g.num_q_heads;
    a.num_kv_heads = g.num_kv_heads;
    a.scale_log2 = g.scale * kLog2e;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (a.splits > 0) {
        if (plan) hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
        // G = 8: 156 VGPRs leave room for 3 waves per SIMD, so a compute unit holds one
        // 8-wave workgroup with 4 wave slots idle; the heads of a chunk are split over two
        // workgroups instead (each stages the chunk's slots), and three fit per unit
        const unsigned zsplit = (group == 8 && g.num_kv_heads > 4) ? 2u : 1u;
        const unsigned waves = (static_cast<unsigned>(g.num_kv_heads) + zsplit - 1) / zsplit;
        const dim3 grid = plan ? dim3(static_cast<unsigned>(units), 1u, zsplit)
                               : dim3(static_cast<unsigned>(a.splits), static_cast<unsigned>(g.num_reqs),
                                      zsplit);
        const dim3 block(waves * kWave);
        const size_t lds = 0;
        if (g.mode == KVW_SLOTS_PAGED) launch_partial<KVW_SLOTS_PAGED>(group, grid, block, lds, s, a);
        else launch_partial<KVW_SLOTS_RANGES>(group, grid, block, lds, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    if (a.splits <= kSmallChunks) {
        constexpr int kHeadsPerGroup = kCombineThreads / kWave;
        const dim3 cgrid(static_cast<unsigned>((g.num_q_heads + kHeadsPerGroup - 1) / kHeadsPerGroup),
                         static_cast<unsigned>(g.num_reqs));
        hipLaunchKernelGGL(decode_combine_small_kernel, cgrid, dim3(kCombineThreads), 0, s, a);
    } else {
        const dim3 cgrid(static_cast<unsigned>(g.num_q_heads), static_cast<unsigned>(g.num_reqs));
        hipLaunchKernelGGL(decode_combine_kernel, cgrid, dim3(kCombineThreads), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVW_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KVW_OK;
}

kvw_status kvw_decode_attention(const kvw_decode_args *args, void *stream)
{
    return decode_attention_run(args, stream, "kvw_decode_attention", false);
}

kvw_status kvw_decode_attention_noalloc(const kvw_decode_args *args, void *stream)
{
    return decode_attention_run(args, stream, "kvw_decode_attention_noalloc", true);
}

}  // extern "C"
