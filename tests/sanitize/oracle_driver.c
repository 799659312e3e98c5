/* Calls every function of oracle/oracle.c on seeded small inputs, edge sizes included.
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py.
 * Return codes are not checked against expectations here (the pins do that); the point is
 * that no call reads or writes out of bounds or hits undefined arithmetic. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_slot_mapping_paged(const int32_t *, int32_t, const int64_t *, int64_t, const int32_t *,
                           int32_t, const int32_t *, int32_t, int64_t *, uint32_t *);
int orc_slot_mapping_ranges(const int32_t *, int32_t, const int64_t *, int64_t, const int32_t *,
                            const int32_t *, const int32_t *, const int32_t *, int32_t, int32_t,
                            int64_t *, uint32_t *);
int orc_slot_mapping_paged_cp(const int32_t *, int32_t, const int64_t *, int64_t, const int32_t *,
                              int32_t, const int32_t *, int32_t, int32_t, int32_t, int32_t,
                              int64_t *, uint32_t *);
int orc_slot_mapping_ranges_cp(const int32_t *, int32_t, const int64_t *, int64_t,
                               const int32_t *, const int32_t *, const int32_t *, const int32_t *,
                               int32_t, int32_t, int32_t, int32_t, int32_t, int64_t *, uint32_t *);
int orc_map_to_kernel_blocks(const int32_t *, const int32_t *, int32_t, int32_t, int32_t, int32_t,
                             int32_t *, int32_t, int32_t *, uint32_t *);
int orc_map_ranges_to_kernel_blocks(const int32_t *, const int32_t *, const int32_t *,
                                    const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t *,
                                    int32_t *, int32_t *, int32_t *, uint32_t *);
int orc_ranges_to_block_table(const int32_t *, const int32_t *, const int32_t *, const int32_t *,
                              int32_t, int32_t, int32_t, int32_t, int32_t *, int32_t, int32_t *,
                              uint32_t *);
int64_t orc_coord_offset(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t);
int orc_decode_attention(const uint16_t *, const uint16_t *, const uint16_t *, int64_t,
                         const int64_t *, const int64_t *, const int32_t *, int32_t, int32_t,
                         int32_t, int32_t, double, double *, double *);
int orc_kv_write(const int64_t *, int64_t, int32_t, const uint8_t *, const uint8_t *, int64_t,
                 int64_t, int64_t, int32_t, int64_t, uint8_t *, uint8_t *, int64_t, int64_t,
                 uint32_t *);

static uint64_t g = 88172645463325252ull;
static uint64_t rnd(void) { g ^= g << 13; g ^= g >> 7; g ^= g << 17; return g; }
static int64_t below(int64_t n) { return (int64_t)(rnd() % (uint64_t)n); }

int main(void)
{
    enum { R = 5, STRIDE = 6, RS = 4, M = 64, ROW = 16, BS = 4, NB = 48 };
    long calls = 0, ok = 0;
#define CALL(e) do { ++calls; ok += (e) == 0; } while (0)
    for (int trial = 0; trial < 3000; ++trial) {
        int32_t qsl[R + 1], table[R * STRIDE], nb[R], st[R * RS], ln[R * RS], cm[R * RS], nr[R];
        int64_t pos[M], slots[M];
        uint32_t flags = 0;
        int32_t n_req = (int32_t)below(R + 1), m = (int32_t)below(M + 1);
        qsl[0] = 0;
        for (int r = 0; r < R; ++r) qsl[r + 1] = qsl[r] + (int32_t)below(m / R + 2);
        if (qsl[n_req] > m) qsl[n_req] = m;
        for (int r = 0; r <= n_req; ++r) if (qsl[r] > qsl[n_req]) qsl[r] = qsl[n_req];
        for (int t = 0; t < M; ++t) pos[t] = below(40) - 3;
        for (int i = 0; i < R * STRIDE; ++i) table[i] = (int32_t)below(NB + 2) - 1;
        for (int r = 0; r < R; ++r) {
            nb[r] = (int32_t)below(STRIDE + 3) - 1;
            nr[r] = (int32_t)below(RS + 2) - (below(10) == 0 ? 1 : 0);
            int32_t c = 0;
            for (int i = 0; i < RS; ++i) {
                st[r * RS + i] = (int32_t)below(NB);
                ln[r * RS + i] = 1 + (int32_t)below(3);
                cm[r * RS + i] = c;
                c += ln[r * RS + i];
            }
        }
        CALL(orc_slot_mapping_paged(qsl, n_req, pos, m, table, STRIDE, below(2) ? nb : NULL, BS, slots,
                               &flags));
        CALL(orc_slot_mapping_ranges(qsl, n_req, pos, m, st, ln, cm, nr, RS, BS, slots, &flags));
        int32_t w = 1 + (int32_t)below(3), il = below(2) ? 1 : 2;
        CALL(orc_slot_mapping_paged_cp(qsl, n_req, pos, m, table, STRIDE, nb, BS, w, (int32_t)below(w),
                                  il, slots, &flags));
        CALL(orc_slot_mapping_ranges_cp(qsl, n_req, pos, m, st, ln, cm, nr, RS, BS, w,
                                   (int32_t)below(w), il, slots, &flags));
        int32_t out[R * STRIDE * 4], counts[R], os[R * RS], ol[R * RS], oc[R * RS], on[R];
        CALL(orc_map_to_kernel_blocks(table, nb, R, STRIDE, 8, 4, out, STRIDE * 2 + (int32_t)below(3),
                                 counts, &flags));
        CALL(orc_map_ranges_to_kernel_blocks(st, ln, cm, nr, R, RS, 8, 4, os, ol, oc, on, &flags));
        CALL(orc_ranges_to_block_table(st, ln, cm, nr, R, RS, 8, 2, out, (int32_t)below(STRIDE * 4),
                                  counts, &flags));
        /* two layers of rows of ROW bytes; the window covers every cache row */
        static uint8_t key[2 * M * ROW], val[2 * M * ROW], kc[2 * NB * BS * ROW],
            vc[2 * NB * BS * ROW];
        int64_t ws[M];
        for (int t = 0; t < M; ++t) ws[t] = (t < m && below(3)) ? t * 3 % (NB * BS + 5) : -1;
        CALL(orc_kv_write(ws, m, 2, key, val, (int64_t)M * ROW, ROW, NB, BS, ROW, kc, vc, 0,
                     2 * NB * BS, &flags));
        (void)orc_coord_offset(below(4), below(NB), below(BS), NB, BS, 2048);
        /* decode attention: 4 q heads over 2 kv heads of 8 dims; cache rows reinterpret kc */
        {
            static uint16_t qa[R * 4 * 8];
            static double oa[R * 4 * 8], lse[R * 4];
            int64_t aslots[M], begin[R + 1];
            int32_t sel[R];
            for (int i = 0; i < R * 4 * 8; ++i) qa[i] = (uint16_t)(0x3C00 + below(0x800));
            begin[0] = 0;
            for (int r = 0; r < R; ++r) {
                sel[r] = r;
                begin[r + 1] = begin[r] + below(M / R);
                for (int64_t j = begin[r]; j < begin[r + 1]; ++j) aslots[j] = below(100) - 2;
            }
            CALL(orc_decode_attention(qa, (const uint16_t *)kc, (const uint16_t *)vc, 100, aslots,
                                      begin, sel, R, 4, 2, 8, 0.35, oa, (trial & 1) ? lse : NULL));
        }
    }
    if (ok * 10 < calls * 9) {  /* nearly every call must get past its argument checks */
        fprintf(stderr, "only %ld of %ld calls succeeded\n", ok, calls);
        return 1;
    }
    printf("OK %ld of %ld calls\n", ok, calls);
    return 0;
}
