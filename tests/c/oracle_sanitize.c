/* Drives every exported function of oracle/pkv_oracle.c on small seeded inputs -- ragged and empty sequences,
 * partial last blocks, unit lists, splits and their combine, the append with skipped slots, varlen and windowed
 * attention, the QKV step in both norm modes, and the error returns -- so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees every code path touch memory.  It also checks a few values that hold exactly
 * (a one-row sequence returns its V row, weights sum to one, split then combine equals the dense result) and prints
 * one "ok" line per check; any sanitizer report or failed check ends the run with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
void oracle_f16_array_to_f64(const uint16_t *src, int64_t n, double *dst);
int64_t oracle_k_index(int32_t Hkv, int32_t BS, int32_t D, int64_t b, int h, int o, int d);
int64_t oracle_v_index(int32_t Hkv, int32_t BS, int32_t D, int64_t b, int h, int o, int d);
int oracle_decode_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t BS, int32_t N, int32_t M, double scale,
                            const int32_t *units, int64_t n_units, double *out, int32_t n_threads);
int oracle_attention_weights(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *block_tables, const int32_t *context_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t BS, int32_t N, int32_t M, double scale, int32_t s,
                             int32_t hq, double *out, double *weights);
int oracle_split_count(int32_t L, int32_t BS, int32_t S, int32_t chunk_blocks);
int oracle_split_partials(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                          const int32_t *block_tables, const int32_t *context_lens, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t D, int32_t BS, int32_t N, int32_t M, double scale, int32_t S,
                          int32_t chunk_blocks, double *O, double *m_out, double *l_out);
int oracle_split_combine(const double *O, const double *m_in, const double *l_in, const int32_t *context_lens,
                         int32_t B, int32_t Hq, int32_t D, int32_t BS, int32_t S, int32_t chunk_blocks, double *out);
int64_t oracle_paged_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping, int32_t T,
                               int32_t Hkv, int32_t D, int32_t BS, int32_t N, uint16_t *k_pool, uint16_t *v_pool);
int oracle_varlen_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                            const int32_t *block_tables, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                            int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t N,
                            int32_t M, double scale, const int32_t *units, int64_t n_units, double *out,
                            int32_t n_threads);
int oracle_decode_attention_window(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                   const int32_t *block_tables, const int32_t *context_lens, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t BS, int32_t N, int32_t M, double scale,
                                   int32_t window, const int32_t *units, int64_t n_units, double *out,
                                   int32_t n_threads);
int oracle_qkv_norm_rope_paged(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                               const float *cos_t, const float *sin_t, int32_t P_rows, const int32_t *cu_seqlens_q,
                               const int32_t *rope_pos, const int32_t *cache_pos, const int32_t *block_tables,
                               int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t N,
                               int32_t M, double eps, int32_t qk_mode, double *q_out, double *k_out, int64_t *slots,
                               uint16_t *v_pool);

static int failures = 0;
static void check(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok)
        failures++;
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {  /* xorshift64* */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (uint32_t)((rng * 2685821657736338717ull) >> 32);
}
/* an fp16 bit pattern of magnitude in [0.25, 2) and random sign */
static uint16_t rand_f16(void) {
    const uint32_t r = next_u32();
    const uint16_t exp = (uint16_t)(13 + (r % 3));
    return (uint16_t)(((r >> 8) & 1u) << 15 | exp << 10 | ((r >> 9) & 0x3FFu));
}
static void fill(uint16_t *p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        p[i] = rand_f16();
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

enum { B = 3, HQ = 4, HKV = 2, D = 64, BS = 16, N = 16, M = 4, T = 4, TV = 5, P = 80 };

int main(void) {
    const int64_t pool_elems = (int64_t)N * HKV * BS * D;
    uint16_t *kp = xmalloc(sizeof(uint16_t) * pool_elems), *vp = xmalloc(sizeof(uint16_t) * pool_elems);
    uint16_t *q = xmalloc(sizeof(uint16_t) * B * HQ * D);
    fill(kp, pool_elems);
    fill(vp, pool_elems);
    fill(q, B * HQ * D);
    /* sequence 0: 37 rows (partial last block), 1: empty, 2: a full table of 64 rows; distinct blocks */
    int32_t lens[B] = {37, 0, 64};
    int32_t bt[B * M] = {5, 2, 9, -1, -1, -1, -1, -1, 0, 7, 3, 12};
    const double scale = 0.125;
    double *out = xmalloc(sizeof(double) * B * HQ * D);

    check(oracle_f16_to_f64(0x3C00) == 1.0 && oracle_f16_to_f64(0x0001) == ldexp(1.0, -24), "f16 decode");
    double dec[8];
    oracle_f16_array_to_f64(q, 8, dec);
    check(dec[3] == oracle_f16_to_f64(q[3]), "f16 array decode");
    check(oracle_k_index(HKV, BS, D, 3, 1, 17 % 16, 9) >= 0 && oracle_v_index(HKV, BS, D, N - 1, HKV - 1, BS - 1, D - 1) ==
              pool_elems - 1, "index functions stay inside the pool");

    int rc = oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, NULL, 0, out, 2);
    int finite = 1, zeros = 1;
    for (int i = 0; i < B * HQ * D; ++i)
        finite &= isfinite(out[i]) ? 1 : 0;
    for (int i = 0; i < HQ * D; ++i)
        zeros &= out[1 * HQ * D + i] == 0.0;
    check(rc == 0 && finite && zeros, "decode attention: all units, empty sequence gives zeros");

    int32_t units[4] = {2, 3, 0, 1};
    double two[2 * D];
    rc = oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, units, 2, two, 1);
    check(rc == 0 && memcmp(two, out + (2 * HQ + 3) * D, sizeof(double) * D) == 0 &&
              memcmp(two + D, out + 1 * D, sizeof(double) * D) == 0, "decode attention: unit list");

    double w[M * BS], o1[D];
    rc = oracle_attention_weights(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, 0, 2, o1, w);
    double sw = 0.0;
    for (int t = 0; t < lens[0]; ++t)
        sw += w[t];
    check(rc == 0 && fabs(sw - 1.0) < 1e-12, "attention weights sum to one");

    int32_t one[B] = {1, 0, 1};
    rc = oracle_decode_attention(q, kp, vp, bt, one, B, HQ, HKV, D, BS, N, M, scale, NULL, 0, out, 3);
    int same = rc == 0;
    for (int d = 0; d < D; ++d)  /* sequence 0, query head 3 -> kv head 1; row 0 of block 5 */
        same &= out[3 * D + d] == oracle_f16_to_f64(vp[oracle_v_index(HKV, BS, D, 5, 1, 0, d)]);
    check(same, "a one-row sequence returns its V row");

    enum { S = 3 };
    double *O = xmalloc(sizeof(double) * B * HQ * S * D), *mo = xmalloc(sizeof(double) * B * HQ * S),
           *lo = xmalloc(sizeof(double) * B * HQ * S), *comb = xmalloc(sizeof(double) * B * HQ * D),
           *dense = xmalloc(sizeof(double) * B * HQ * D);
    rc = oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, NULL, 0, dense, 1);
    int rc2 = oracle_split_partials(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, S, 0, O, mo, lo);
    int rc3 = oracle_split_combine(O, mo, lo, lens, B, HQ, D, BS, S, 0, comb);
    double worst = 0.0;
    for (int i = 0; i < B * HQ * D; ++i)
        worst = fmax(worst, fabs(comb[i] - dense[i]));
    check(rc == 0 && rc2 == 0 && rc3 == 0 && worst < 1e-12, "split partials then combine equal the dense result");
    check(oracle_split_count(37, BS, 3, 0) == 3 && oracle_split_count(37, BS, 8, 0) == 3 &&
              oracle_split_count(0, BS, 4, 0) == 0 && oracle_split_count(64, BS, 2, 1) >= 1, "split counts");
    rc2 = oracle_split_partials(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, S, 2, O, mo, lo);
    rc3 = oracle_split_combine(O, mo, lo, lens, B, HQ, D, BS, S, 2, comb);
    worst = 0.0;
    for (int i = 0; i < B * HQ * D; ++i)
        worst = fmax(worst, fabs(comb[i] - dense[i]));
    check(rc2 == 0 && rc3 == 0 && worst < 1e-12, "split partials with fixed two-block chunks");

    /* append: tokens to slots 5*16+4, skipped (-1), out of the pool, 12*16+15 */
    uint16_t *kn = xmalloc(sizeof(uint16_t) * T * HKV * D), *vn = xmalloc(sizeof(uint16_t) * T * HKV * D);
    fill(kn, T * HKV * D);
    fill(vn, T * HKV * D);
    int32_t slots[T] = {5 * BS + 4, -1, N * BS, 12 * BS + 15};
    int64_t written = oracle_paged_kv_append(kn, vn, slots, T, HKV, D, BS, N, kp, vp);
    check(written == 2 && kp[oracle_k_index(HKV, BS, D, 12, 1, 15, 7)] == kn[(3 * HKV + 1) * D + 7] &&
              vp[oracle_v_index(HKV, BS, D, 5, 0, 4, 63)] == vn[63], "append writes the valid slots only");

    /* varlen: sequence 0 appends 3 rows from row 34, sequence 1 none, sequence 2 two rows from row 62 */
    int32_t cu[B + 1] = {0, 3, 3, 5}, pos[B] = {34, 5, 62};
    uint16_t *qv = xmalloc(sizeof(uint16_t) * TV * HQ * D);
    fill(qv, TV * HQ * D);
    double *ov = xmalloc(sizeof(double) * TV * HQ * D);
    rc = oracle_varlen_attention(qv, kp, vp, bt, cu, pos, B, TV, HQ, HKV, D, BS, N, M, scale, NULL, 0, ov, 2);
    finite = 1;
    for (int i = 0; i < TV * HQ * D; ++i)
        finite &= isfinite(ov[i]) ? 1 : 0;
    check(rc == 0 && finite, "varlen attention");
    int32_t vunits[2] = {4, 0};
    rc = oracle_varlen_attention(qv, kp, vp, bt, cu, pos, B, TV, HQ, HKV, D, BS, N, M, scale, vunits, 1, two, 1);
    check(rc == 0 && memcmp(two, ov + 4 * HQ * D, sizeof(double) * D) == 0, "varlen unit list");

    /* the pools changed with the append: the full attention again, then the windows */
    rc3 = oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, NULL, 0, dense, 2);
    rc = oracle_decode_attention_window(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, 20, NULL, 0, out, 2);
    rc2 = oracle_decode_attention_window(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, 1000, NULL, 0, comb, 1);
    worst = 0.0;
    for (int i = 0; i < B * HQ * D; ++i)
        worst = fmax(worst, fabs(comb[i] - dense[i]));
    check(rc == 0 && rc2 == 0 && rc3 == 0 && worst < 1e-12, "windowed attention; a window past the length is the full one");

    /* QKV step, both norm modes, positions inside a 80-row table */
    const int W = HQ + 2 * HKV;
    uint16_t *qkv = xmalloc(sizeof(uint16_t) * TV * W * D), qw[D], kw[D];
    fill(qkv, TV * W * D);
    fill(qw, D);
    fill(kw, D);
    float *ct = xmalloc(sizeof(float) * P * D / 2), *st = xmalloc(sizeof(float) * P * D / 2);
    for (int i = 0; i < P * D / 2; ++i) {
        ct[i] = (float)cos(0.01 * i);
        st[i] = (float)sin(0.01 * i);
    }
    double *qo = xmalloc(sizeof(double) * TV * HQ * D), *ko = xmalloc(sizeof(double) * TV * HKV * D);
    int64_t qslots[TV];
    for (int mode = 0; mode < 2; ++mode) {
        rc = oracle_qkv_norm_rope_paged(qkv, qw, kw, ct, st, P, cu, pos, pos, bt, B, TV, HQ, HKV, D, BS, N, M, 1e-6,
                                        mode, qo, ko, qslots, vp);
        check(rc == 0 && qslots[0] == 9 * BS + 2 && qslots[4] == 12 * BS + 15, mode ? "qkv step, rms norm" :
                                                                                      "qkv step, no norm");
    }

    /* error returns */
    int32_t bad_bt[B * M];
    memcpy(bad_bt, bt, sizeof bad_bt);
    bad_bt[1] = N + 3;
    check(oracle_decode_attention(q, kp, vp, bad_bt, lens, B, HQ, HKV, D, BS, N, M, scale, NULL, 0, out, 2) != 0,
          "a table entry outside the pool is an error");
    check(oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, 3, D, BS, N, M, scale, NULL, 0, out, 1) != 0,
          "Hq not a multiple of Hkv is an error");
    int32_t bad_units[2] = {B, 0};
    check(oracle_decode_attention(q, kp, vp, bt, lens, B, HQ, HKV, D, BS, N, M, scale, bad_units, 1, out, 1) != 0,
          "a unit outside the batch is an error");
    int32_t bad_cu[B + 1] = {0, 4, 3, 5};
    check(oracle_varlen_attention(qv, kp, vp, bt, bad_cu, pos, B, TV, HQ, HKV, D, BS, N, M, scale, NULL, 0, ov, 1) !=
              0, "decreasing prefix sums are an error");
    int32_t far[B] = {34, 5, P};
    check(oracle_qkv_norm_rope_paged(qkv, qw, kw, ct, st, P, cu, far, pos, bt, B, TV, HQ, HKV, D, BS, N, M, 1e-6, 1,
                                     qo, ko, qslots, vp) != 0, "a RoPE position past the table is an error");

    free(kp); free(vp); free(q); free(out); free(O); free(mo); free(lo); free(comb); free(dense);
    free(kn); free(vn); free(qv); free(ov); free(qkv); free(ct); free(st); free(qo); free(ko);
    return failures == 0 ? 0 : 1;
}
