/*
 * pkv_oracle.c -- plain, slow, f64 CPU oracle for paged-KV decode attention and
 * the paged KV append.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library under paged_kv_decode_04_amd/) never links, loads or calls it, and
 * this file includes no header of the product path: the two share no code.
 *
 * What is computed, and where the pages define it:
 *
 *  - Paged KV append.  A new token's K and V rows go to the pool position named
 *    by its slot; slot = physical_block * block_size + position_in_block.
 *    [kapsl-backends 0.1.1, src/gguf_native.rs: one_token_compute (the
 *    launch_kv_write call with physical_block / pos_in_block) and
 *    forward_batch_decode_greedy (launch_batch_kv_write with per-token
 *    physical_blocks / pos_in_blocks)]
 *
 *  - Paged decode attention.  For sequence s and query head hq:
 *      out = softmax(scale * q . K^T) . V
 *    over the context_lens[s] rows of the sequence, row t living in physical
 *    block block_tables[s][t / block_size] at offset t % block_size.
 *    [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *    BackendPagedKv::paged_decode_attention and paged_batched_decode_attention;
 *    kapsl-backends 0.1.1, src/gguf_native.rs: forward_batch_decode_greedy,
 *    where context_lens counts the rows after the new token was appended]
 *    Query head hq reads kv head hq / G with G = num_q_heads / num_kv_heads.
 *    [cortiq-engine 0.8.80, src/gpu_cuda.rs: the heads-per-kv-head grouping]
 *
 *  - Split QKV, q/k RMSNorm, RoPE and the paged-cache write: the step that
 *    produces the rows the attention reads (see oracle_qkv_norm_rope_paged).
 *
 *  - Paged varlen attention: several new query rows per sequence, each
 *    attending the rows up to and including its own position (see
 *    oracle_varlen_attention for the passages).
 *
 *  - Split-K ("flash decoding") partials and their log-sum-exp combine.  The
 *    pages give only the buffer names partial_out / partial_m / partial_l and
 *    the two launches [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *    SplitKScratch and paged_batched_flash_dispatch]; the formulas below are
 *    the plain reading: per split j, m_j = max z, l_j = sum exp(z - m_j),
 *    O_j = sum exp(z - m_j) v; then out = sum_j e^(m_j - M) O_j /
 *    sum_j e^(m_j - M) l_j with M = max_j m_j.
 *
 * Pool layouts (the pages do not fix one; this library and the HIP library
 * both document the same two).  Each block of block_size rows is stored as
 * block_size/16 panels of 16 rows:
 *    k_pool[num_blocks][num_kv_heads][block_size/16][head_dim/32][16][32]
 *           (a panel holds each row's dims in 32-wide pieces: dims 0..31
 *           of the 16 rows, then dims 32..63, ...)
 *    v_pool[num_blocks][num_kv_heads][block_size/16][4][head_dim][4]
 *           (a panel holds V in four quads of 4 rows; in a quad each
 *           dim's 4 rows are adjacent: dim 0 of rows 4i..4i+3, then dim 1,
 *           ...)
 * head_dim must be a multiple of 32 and block_size a multiple of 16.
 *
 * All arithmetic is IEEE binary64; fp16 inputs are decoded exactly.  No
 * blocking, fusion or reordering beyond the definitions above.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE 754 binary16 -> binary64, exact.
 * sign s, 5-bit exponent e, 10-bit fraction f:
 *   e == 0      : (-1)^s * f * 2^-24            (zero and subnormals)
 *   0 < e < 31  : (-1)^s * (1024 + f) * 2^(e-25)
 *   e == 31     : (-1)^s * inf if f == 0, else NaN                         */
double oracle_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

void oracle_f16_array_to_f64(const uint16_t *src, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_f16_to_f64(src[i]);
}

/* ------------------------------------------------------------------ */
/* Problem description and the two pool index functions.                */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint16_t *q;            /* [B][Hq][D] fp16 bits */
    const uint16_t *k_pool;       /* [N][Hkv][BS/16][D/32][16][32] fp16 bits */
    const uint16_t *v_pool;       /* [N][Hkv][BS/16][4][D][4] fp16 bits */
    const int32_t *block_tables;  /* [B][M] */
    const int32_t *context_lens;  /* [B] */
    int32_t B, Hq, Hkv, D, BS, N, M;
    double scale;
    int32_t window;               /* sliding window: > 0 attends only the last `window` rows; 0 = all rows */
} oracle_problem;

/* k_pool element (block b, kv head h, row offset o, dim d): panel o / 16, piece d / 32, row o % 16, dim d % 32 */
static int64_t k_index(const oracle_problem *P, int64_t b, int h, int o, int d)
{
    int64_t panel = (b * P->Hkv + h) * (P->BS / 16) + o / 16;
    return ((panel * (P->D / 32) + d / 32) * 16 + o % 16) * 32 + d % 32;
}

/* v_pool element (block b, kv head h, row offset o, dim d): panel o / 16, quad (o % 16) / 4, dim d, row o % 4 */
static int64_t v_index(const oracle_problem *P, int64_t b, int h, int o, int d)
{
    int64_t panel = (b * P->Hkv + h) * (P->BS / 16) + o / 16;
    return ((panel * 4 + (o % 16) / 4) * P->D + d) * 4 + o % 4;
}

int64_t oracle_k_index(int32_t Hkv, int32_t BS, int32_t D, int64_t b, int h, int o, int d)
{
    oracle_problem P;
    memset(&P, 0, sizeof P);
    P.Hkv = Hkv; P.BS = BS; P.D = D;
    return k_index(&P, b, h, o, d);
}

int64_t oracle_v_index(int32_t Hkv, int32_t BS, int32_t D, int64_t b, int h, int o, int d)
{
    oracle_problem P;
    memset(&P, 0, sizeof P);
    P.Hkv = Hkv; P.BS = BS; P.D = D;
    return v_index(&P, b, h, o, d);
}

/* Physical block of row t of sequence s, or -1 when the table does not name
 * a valid block for it. */
static int64_t row_block(const oracle_problem *P, int s, int t)
{
    int j = t / P->BS;
    if (j >= P->M)
        return -1;
    int32_t p = P->block_tables[(int64_t)s * P->M + j];
    if (p < 0 || p >= P->N)
        return -1;
    return p;
}

/* z_t = scale * sum_d q[d] * k_t[d] for rows t in [t0, t1) of sequence s,
 * kv head hk, with q the D-vector of one query head.  Returns 0, or -2 when a
 * row's block is not a valid pool block. */
static int scores_for(const oracle_problem *P, int s, const uint16_t *q, int hk, int t0, int t1, double *z)
{
    for (int t = t0; t < t1; ++t) {
        int64_t p = row_block(P, s, t);
        if (p < 0)
            return -2;
        int o = t % P->BS;
        double acc = 0.0;
        for (int d = 0; d < P->D; ++d)
            acc += oracle_f16_to_f64(q[d]) * oracle_f16_to_f64(P->k_pool[k_index(P, p, hk, o, d)]);
        z[t - t0] = P->scale * acc;
    }
    return 0;
}

/* z for decode query (s, hq). */
static int scores(const oracle_problem *P, int s, int hq, int t0, int t1, double *z)
{
    int G = P->Hq / P->Hkv;
    return scores_for(P, s, P->q + ((int64_t)s * P->Hq + hq) * P->D, hq / G, t0, t1, z);
}

/* softmax(z) . V over rows lo..L-1 of sequence s, kv head hk, for one query
 * vector q: out[0..D); weights[0..L-lo) (optional) receives the normalised
 * softmax weights.  An empty range gives out = 0. */
static int attend_range(const oracle_problem *P, int s, const uint16_t *q, int hk, int lo, int L, double *out,
                        double *weights)
{
    for (int d = 0; d < P->D; ++d)
        out[d] = 0.0;
    if (lo < 0)
        lo = 0;
    if (L <= lo)
        return 0;
    int n = L - lo;
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    if (!z)
        return -3;
    int rc = scores_for(P, s, q, hk, lo, L, z);
    if (rc) {
        free(z);
        return rc;
    }
    double m = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (z[i] > m)
            m = z[i];
    double l = 0.0;
    for (int i = 0; i < n; ++i)
        l += exp(z[i] - m);
    for (int i = 0; i < n; ++i) {
        double w = exp(z[i] - m);
        int t = lo + i;
        int64_t p = row_block(P, s, t);
        int o = t % P->BS;
        for (int d = 0; d < P->D; ++d)
            out[d] += w * oracle_f16_to_f64(P->v_pool[v_index(P, p, hk, o, d)]);
        if (weights)
            weights[i] = w / l;
    }
    for (int d = 0; d < P->D; ++d)
        out[d] /= l;
    free(z);
    return 0;
}

/* softmax(z) . V over rows 0..L-1 (see attend_range). */
static int attend(const oracle_problem *P, int s, const uint16_t *q, int hk, int L, double *out, double *weights)
{
    return attend_range(P, s, q, hk, 0, L, out, weights);
}

/* One decode output row: (s, hq) over the context_lens[s] rows of sequence s,
 * or with a sliding window W > 0 over its last W rows only: rows
 * max(0, L - W) .. L - 1 [cortiq-engine 0.8.80, src/gpu_cuda.rs: the decode
 * attend, first = stored - window (saturating), the KvMirror window]. */
static int attention_unit(const oracle_problem *P, int s, int hq, double *out, double *weights)
{
    int G = P->Hq / P->Hkv;
    int L = P->context_lens[s];
    int lo = (P->window > 0 && L > P->window) ? L - P->window : 0;
    return attend_range(P, s, P->q + ((int64_t)s * P->Hq + hq) * P->D, hq / G, lo, L, out, weights);
}

/* ------------------------------------------------------------------ */
/* Threaded driver over (sequence, query head) units.                   */
/* ------------------------------------------------------------------ */

typedef struct {
    const oracle_problem *P;
    const int32_t *units;   /* pairs (s, hq); NULL = every unit in order */
    int64_t n_units;
    double *out;            /* [n_units][D] */
    int64_t next;           /* shared work counter */
    int rc;
    pthread_mutex_t lock;
} unit_pool;

static void *unit_worker(void *arg)
{
    unit_pool *W = (unit_pool *)arg;
    for (;;) {
        pthread_mutex_lock(&W->lock);
        int64_t u = W->next++;
        pthread_mutex_unlock(&W->lock);
        if (u >= W->n_units)
            break;
        int s, hq;
        if (W->units) {
            s = W->units[2 * u];
            hq = W->units[2 * u + 1];
        } else {
            s = (int)(u / W->P->Hq);
            hq = (int)(u % W->P->Hq);
        }
        int rc = attention_unit(W->P, s, hq, W->out + u * W->P->D, NULL);
        if (rc) {
            pthread_mutex_lock(&W->lock);
            W->rc = rc;
            pthread_mutex_unlock(&W->lock);
        }
    }
    return NULL;
}

static int check_geometry(const oracle_problem *P)
{
    if (P->B < 0 || P->Hq <= 0 || P->Hkv <= 0 || P->D <= 0 || P->BS <= 0 || P->N < 0 || P->M < 0)
        return -1;
    if (P->Hq % P->Hkv || P->D % 32 || P->BS % 16)
        return -1;
    return 0;
}

/* Decode attention for the listed (s, hq) units (or all B*Hq of them when
 * units is NULL), each row of out[n_units][D] in f64. */
int oracle_decode_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                            int32_t N, int32_t M, double scale,
                            const int32_t *units, int64_t n_units, double *out, int32_t n_threads)
{
    oracle_problem P = {q, k_pool, v_pool, block_tables, context_lens, B, Hq, Hkv, D, BS, N, M, scale, 0};
    if (check_geometry(&P))
        return -1;
    if (!units)
        n_units = (int64_t)B * Hq;
    for (int64_t u = 0; units && u < n_units; ++u)
        if (units[2 * u] < 0 || units[2 * u] >= B || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hq)
            return -1;
    if (n_threads < 1)
        n_threads = 1;
    unit_pool W;
    W.P = &P; W.units = units; W.n_units = n_units; W.out = out; W.next = 0; W.rc = 0;
    pthread_mutex_init(&W.lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    int started = 0;
    for (int i = 0; i < n_threads; ++i)
        if (pthread_create(&th[i], NULL, unit_worker, &W) == 0)
            ++started;
    if (started == 0)
        unit_worker(&W);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&W.lock);
    return W.rc;
}

/* Softmax weights of one unit: weights[0..context_lens[s]) sum to 1. */
int oracle_attention_weights(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                             const int32_t *block_tables, const int32_t *context_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                             int32_t N, int32_t M, double scale, int32_t s, int32_t hq,
                             double *out, double *weights)
{
    oracle_problem P = {q, k_pool, v_pool, block_tables, context_lens, B, Hq, Hkv, D, BS, N, M, scale, 0};
    if (check_geometry(&P) || s < 0 || s >= B || hq < 0 || hq >= Hq)
        return -1;
    return attention_unit(&P, s, hq, out, weights);
}

/* ------------------------------------------------------------------ */
/* Split-K partials and combine.                                        */
/* ------------------------------------------------------------------ */

/* The block range of split j of a sequence with L rows.  Blocks are whole:
 * nb = ceil(L / BS) blocks, chunk = chunk_blocks if > 0 else ceil(nb / S),
 * split j covers blocks [j*chunk, min(nb, (j+1)*chunk)).  Returns the number
 * of non-empty splits, ceil(nb / chunk) (0 when L <= 0). */
static int split_range(int L, int BS, int S, int chunk_blocks, int j, int *b0, int *b1)
{
    if (L <= 0) {
        *b0 = *b1 = 0;
        return 0;
    }
    int nb = (L + BS - 1) / BS;
    int chunk = chunk_blocks > 0 ? chunk_blocks : (nb + S - 1) / S;
    int nvalid = (nb + chunk - 1) / chunk;
    int lo = j * chunk;
    int hi = (j + 1) * chunk;
    if (lo > nb) lo = nb;
    if (hi > nb) hi = nb;
    *b0 = lo;
    *b1 = hi;
    return nvalid;
}

int oracle_split_count(int32_t L, int32_t BS, int32_t S, int32_t chunk_blocks)
{
    int b0, b1;
    return split_range(L, BS, S, chunk_blocks, 0, &b0, &b1);
}

/* Partials for every (s, hq, j): O[B][Hq][S][D], m[B][Hq][S], l[B][Hq][S].
 * An empty split gives m = -inf, l = 0, O = 0.  m is in the units of z
 * (natural log domain). */
int oracle_split_partials(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                          const int32_t *block_tables, const int32_t *context_lens,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                          int32_t N, int32_t M, double scale, int32_t S, int32_t chunk_blocks,
                          double *O, double *m_out, double *l_out)
{
    oracle_problem P = {q, k_pool, v_pool, block_tables, context_lens, B, Hq, Hkv, D, BS, N, M, scale, 0};
    if (check_geometry(&P) || S < 1 || chunk_blocks < 0)
        return -1;
    int G = Hq / Hkv;
    for (int s = 0; s < B; ++s) {
        int L = context_lens[s];
        for (int hq = 0; hq < Hq; ++hq) {
            int hk = hq / G;
            for (int j = 0; j < S; ++j) {
                int64_t base = ((int64_t)s * Hq + hq) * S + j;
                double *Oj = O + base * D;
                int b0, b1;
                split_range(L, BS, S, chunk_blocks, j, &b0, &b1);
                int t0 = b0 * BS;
                int t1 = b1 * BS < L ? b1 * BS : L;
                for (int d = 0; d < D; ++d)
                    Oj[d] = 0.0;
                if (t1 <= t0) {
                    m_out[base] = -INFINITY;
                    l_out[base] = 0.0;
                    continue;
                }
                double *z = (double *)malloc(sizeof(double) * (size_t)(t1 - t0));
                if (!z)
                    return -3;
                int rc = scores(&P, s, hq, t0, t1, z);
                if (rc) {
                    free(z);
                    return rc;
                }
                double m = -INFINITY;
                for (int t = t0; t < t1; ++t)
                    if (z[t - t0] > m)
                        m = z[t - t0];
                double l = 0.0;
                for (int t = t0; t < t1; ++t) {
                    double w = exp(z[t - t0] - m);
                    int64_t p = row_block(&P, s, t);
                    int o = t % BS;
                    l += w;
                    for (int d = 0; d < D; ++d)
                        Oj[d] += w * oracle_f16_to_f64(v_pool[v_index(&P, p, hk, o, d)]);
                }
                m_out[base] = m;
                l_out[base] = l;
                free(z);
            }
        }
    }
    return 0;
}

/* Log-sum-exp combine of the non-empty splits of each (s, hq):
 *   M = max_j m_j,  out = sum_j e^(m_j - M) O_j / sum_j e^(m_j - M) l_j
 * over j < ceil(nb / chunk); entries of later splits are never read.  A
 * sequence with no rows gives out = 0. */
int oracle_split_combine(const double *O, const double *m_in, const double *l_in,
                         const int32_t *context_lens, int32_t B, int32_t Hq, int32_t D,
                         int32_t BS, int32_t S, int32_t chunk_blocks, double *out)
{
    if (B < 0 || Hq <= 0 || D <= 0 || BS <= 0 || S < 1 || chunk_blocks < 0)
        return -1;
    for (int s = 0; s < B; ++s) {
        int nvalid = oracle_split_count(context_lens[s], BS, S, chunk_blocks);
        if (nvalid > S)
            return -4; /* the grid has fewer splits than the sequence needs */
        for (int hq = 0; hq < Hq; ++hq) {
            int64_t row = (int64_t)s * Hq + hq;
            double *o = out + row * D;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            if (nvalid == 0)
                continue;
            double M = -INFINITY;
            for (int j = 0; j < nvalid; ++j)
                if (m_in[row * S + j] > M)
                    M = m_in[row * S + j];
            double den = 0.0;
            for (int j = 0; j < nvalid; ++j) {
                double a = exp(m_in[row * S + j] - M);
                den += a * l_in[row * S + j];
                for (int d = 0; d < D; ++d)
                    o[d] += a * O[(row * S + j) * D + d];
            }
            for (int d = 0; d < D; ++d)
                o[d] /= den;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Paged KV append.                                                      */
/* ------------------------------------------------------------------ */

/* Copies k[i][h][:] and v[i][h][:] (fp16 bits, [T][Hkv][D]) to the pool
 * position of slot_mapping[i]: block slot / BS, row offset slot % BS.  Slots
 * outside [0, N*BS) are skipped (a negative slot marks padding).  Returns the
 * number of skipped tokens, or -1 on a bad geometry. */
int64_t oracle_paged_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
                               int32_t T, int32_t Hkv, int32_t D, int32_t BS, int32_t N,
                               uint16_t *k_pool, uint16_t *v_pool)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || D % 32 || BS <= 0 || BS % 16 || N < 0)
        return -1;
    oracle_problem P;
    memset(&P, 0, sizeof P);
    P.Hkv = Hkv; P.BS = BS; P.D = D; P.N = N;
    int64_t skipped = 0;
    for (int i = 0; i < T; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= (int64_t)N * BS) {
            ++skipped;
            continue;
        }
        int64_t b = slot / BS;
        int o = (int)(slot % BS);
        for (int h = 0; h < Hkv; ++h)
            for (int d = 0; d < D; ++d) {
                int64_t src = ((int64_t)i * Hkv + h) * D + d;
                k_pool[k_index(&P, b, h, o, d)] = k[src];
                v_pool[v_index(&P, b, h, o, d)] = v[src];
            }
    }
    return skipped;
}

/* ------------------------------------------------------------------ */
/* Paged varlen attention (several new query rows per sequence).        */
/* ------------------------------------------------------------------ */

/* Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of the
 * token-major q[T][Hq][D] (and of out); its i-th new row sits at absolute
 * position pos_offsets[s] + i of the sequence and attends rows
 * 0 .. pos_offsets[s] + i (itself included, nothing after it).  The pool must
 * already hold the new rows' K/V.
 * [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_varlen_attention
 * (q token-major [M_total][heads][dim]) and the q_len > 1 branch of
 * paged_decode_attention, which passes cu_seqlens_q = [0, q_len] and
 * pos_offsets = [final_kv_len - q_len]]
 *
 * units: NULL = every (token, head) in order, else n_units pairs
 * (token, hq).  Returns 0; -1 for bad geometry, prefix sums that do not run
 * 0 = cu[0] <= cu[1] <= ... <= cu[B] = T, a negative position, or a row past
 * the table capacity M*BS; -2 for a table entry outside the pool. */
typedef struct {
    const oracle_problem *P;
    const int32_t *cu, *pos;
    int32_t T;
    const int32_t *units;
    int64_t n_units;
    double *out;
    int64_t next;
    int rc;
    pthread_mutex_t lock;
} varlen_pool;

static int varlen_row(const varlen_pool *W, int32_t tok, int32_t hq, double *out)
{
    const oracle_problem *P = W->P;
    int s = 0;
    while (s < P->B && W->cu[s + 1] <= tok)
        ++s;
    int i = tok - W->cu[s];
    int G = P->Hq / P->Hkv;
    return attend(P, s, P->q + ((int64_t)tok * P->Hq + hq) * P->D, hq / G, W->pos[s] + i + 1, out, NULL);
}

static void *varlen_worker(void *arg)
{
    varlen_pool *W = (varlen_pool *)arg;
    for (;;) {
        pthread_mutex_lock(&W->lock);
        int64_t u = W->next++;
        pthread_mutex_unlock(&W->lock);
        if (u >= W->n_units)
            break;
        int32_t tok, hq;
        if (W->units) {
            tok = W->units[2 * u];
            hq = W->units[2 * u + 1];
        } else {
            tok = (int32_t)(u / W->P->Hq);
            hq = (int32_t)(u % W->P->Hq);
        }
        int rc = varlen_row(W, tok, hq, W->out + u * W->P->D);
        if (rc) {
            pthread_mutex_lock(&W->lock);
            W->rc = rc;
            pthread_mutex_unlock(&W->lock);
        }
    }
    return NULL;
}

int oracle_varlen_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                            const int32_t *block_tables, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                            int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                            int32_t N, int32_t M, double scale,
                            const int32_t *units, int64_t n_units, double *out, int32_t n_threads)
{
    oracle_problem P = {q, k_pool, v_pool, block_tables, NULL, B, Hq, Hkv, D, BS, N, M, scale, 0};
    if (check_geometry(&P) || T < 0)
        return -1;
    if (B > 0 && (cu_seqlens_q[0] != 0 || cu_seqlens_q[B] != T))
        return -1;
    if (B == 0 && T != 0)
        return -1;
    for (int s = 0; s < B; ++s) {
        if (cu_seqlens_q[s + 1] < cu_seqlens_q[s] || pos_offsets[s] < 0)
            return -1;
        if ((int64_t)pos_offsets[s] + (cu_seqlens_q[s + 1] - cu_seqlens_q[s]) > (int64_t)M * BS)
            return -1;
    }
    if (!units)
        n_units = (int64_t)T * Hq;
    for (int64_t u = 0; units && u < n_units; ++u)
        if (units[2 * u] < 0 || units[2 * u] >= T || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hq)
            return -1;
    if (n_threads < 1)
        n_threads = 1;
    varlen_pool W;
    W.P = &P; W.cu = cu_seqlens_q; W.pos = pos_offsets; W.T = T; W.units = units; W.n_units = n_units;
    W.out = out; W.next = 0; W.rc = 0;
    pthread_mutex_init(&W.lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    int started = 0;
    for (int i = 0; i < n_threads; ++i)
        if (pthread_create(&th[i], NULL, varlen_worker, &W) == 0)
            ++started;
    if (started == 0)
        varlen_worker(&W);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&W.lock);
    return W.rc;
}


/* ------------------------------------------------------------------ */
/* Sliding-window decode attention.                                     */
/* ------------------------------------------------------------------ */

/* Decode attention where sequence s's new row attends only its last `window`
 * rows (window > 0), rows max(0, L - window) .. L - 1; window = 0 is plain
 * decode attention.  Same arguments and output as oracle_decode_attention. */
int oracle_decode_attention_window(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                                   int32_t N, int32_t M, double scale, int32_t window,
                                   const int32_t *units, int64_t n_units, double *out, int32_t n_threads)
{
    oracle_problem P = {q, k_pool, v_pool, block_tables, context_lens, B, Hq, Hkv, D, BS, N, M, scale, window};
    if (check_geometry(&P) || window < 0)
        return -1;
    if (!units)
        n_units = (int64_t)B * Hq;
    for (int64_t u = 0; units && u < n_units; ++u)
        if (units[2 * u] < 0 || units[2 * u] >= B || units[2 * u + 1] < 0 || units[2 * u + 1] >= Hq)
            return -1;
    if (n_threads < 1)
        n_threads = 1;
    unit_pool W;
    W.P = &P; W.units = units; W.n_units = n_units; W.out = out; W.next = 0; W.rc = 0;
    pthread_mutex_init(&W.lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    int started = 0;
    for (int i = 0; i < n_threads; ++i)
        if (pthread_create(&th[i], NULL, unit_worker, &W) == 0)
            ++started;
    if (started == 0)
        unit_worker(&W);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&W.lock);
    return W.rc;
}


/* ------------------------------------------------------------------ */
/* Split QKV, q/k RMSNorm, RoPE and the paged-cache write.              */
/* ------------------------------------------------------------------ */

/* The step before attention in a decode or prefill layer: one call takes the
 * fused QKV projection rows and leaves the rotated queries in q_out and the
 * new K and V rows in the paged cache.
 * [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 * split_qkv_norm_rope_into_paged_cache (one sequence: tokens, pos_offset,
 * cache_len, block_table) and split_qkv_norm_rope_into_paged_cache_varlen
 * (cu_seqlens_q, pos_offsets, block_tables); one launch covers
 * q_heads + 2 * kv_heads heads per token.  ferrum-kernels 0.7.1, cuda.rs:
 * qk_norm_rope (norm weight, cos, sin, pos_offset, eps, mode)]
 *
 * The pages give the arguments, not the arithmetic; the readings here:
 *  - qkv[T][(Hq + 2*Hkv) * D] fp16, token-major; a row holds the Hq query
 *    heads, then the Hkv key heads, then the Hkv value heads, D dims each;
 *  - token i of sequence s (tokens cu[s] .. cu[s+1]-1) takes RoPE position
 *    rope_pos[s] + (i - cu[s]) and goes to row cache_pos[s] + (i - cu[s]) of
 *    the sequence, i.e. block block_tables[s][row / BS], offset row % BS
 *    (the varlen form passes pos_offsets for both; the one-sequence form
 *    passes pos_offset and cache_len);
 *  - qk_mode 1: each query and key head is RMS-normalised over its D dims and
 *    scaled by the norm weight, x_d <- x_d / sqrt(mean_e(x_e^2) + eps) * w_d
 *    (q_norm_w for query heads, k_norm_w for key heads); qk_mode 0: no norm;
 *  - RoPE rotates dim j with dim j + D/2 (j < D/2) by the angle whose cosine
 *    and sine are cos_t[p][j], sin_t[p][j] (tables of D/2 floats per
 *    position p):  (a, b) -> (a*c - b*s, b*c + a*s);
 *  - value heads are copied unchanged.
 *
 * Outputs: q_out[T][Hq][D] and k_out[T][Hkv][D] in f64 (the rotated query
 * rows and key rows, unrounded), slots[T] = block * BS + offset of the row
 * each token went to, and v_pool with each token's value rows stored (fp16
 * bits, exact copies) at its slot.  k_pool is not written: the key rows are
 * real-valued here and are compared against the pool by the caller.
 *
 * Returns 0; -1 for a bad geometry or mode, prefix sums that do not run
 * 0 = cu[0] <= ... <= cu[B] = T, a position outside [0, P) or a cache row
 * outside [0, M*BS); -2 for a table entry outside the pool. */
int oracle_qkv_norm_rope_paged(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                               const float *cos_t, const float *sin_t, int32_t P_rows,
                               const int32_t *cu_seqlens_q, const int32_t *rope_pos, const int32_t *cache_pos,
                               const int32_t *block_tables, int32_t B, int32_t T, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t BS, int32_t N, int32_t M, double eps, int32_t qk_mode,
                               double *q_out, double *k_out, int64_t *slots, uint16_t *v_pool)
{
    if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D % 8 || BS <= 0 || BS % 16 || N < 0 || M < 0)
        return -1;
    if ((qk_mode != 0 && qk_mode != 1) || (B == 0 && T != 0) || eps < 0.0)
        return -1;
    if (B > 0 && (cu_seqlens_q[0] != 0 || cu_seqlens_q[B] != T))
        return -1;
    oracle_problem P;
    memset(&P, 0, sizeof P);
    P.Hkv = Hkv; P.BS = BS; P.D = D; P.N = N;
    const int width = (Hq + 2 * Hkv) * D;
    const int half = D / 2;
    double *x = (double *)malloc(sizeof(double) * (size_t)D);
    if (!x)
        return -3;
    int rc = 0;
    for (int s = 0; s < B && rc == 0; ++s) {
        if (cu_seqlens_q[s + 1] < cu_seqlens_q[s]) {
            rc = -1;
            break;
        }
        for (int i = cu_seqlens_q[s]; i < cu_seqlens_q[s + 1]; ++i) {
            int64_t p = (int64_t)rope_pos[s] + (i - cu_seqlens_q[s]);
            int64_t row = (int64_t)cache_pos[s] + (i - cu_seqlens_q[s]);
            if (p < 0 || p >= P_rows || row < 0 || row >= (int64_t)M * BS) {
                rc = -1;
                break;
            }
            int32_t blk = block_tables[(int64_t)s * M + row / BS];
            if (blk < 0 || blk >= N) {
                rc = -2;
                break;
            }
            int off = (int)(row % BS);
            slots[i] = (int64_t)blk * BS + off;
            /* query heads 0..Hq-1, then key heads Hq..Hq+Hkv-1: norm (mode 1), then rotate */
            for (int h = 0; h < Hq + Hkv; ++h) {
                const uint16_t *src = qkv + (int64_t)i * width + (int64_t)h * D;
                for (int d = 0; d < D; ++d)
                    x[d] = oracle_f16_to_f64(src[d]);
                if (qk_mode == 1) {
                    const uint16_t *w = h < Hq ? q_norm_w : k_norm_w;
                    double ss = 0.0;
                    for (int d = 0; d < D; ++d)
                        ss += x[d] * x[d];
                    double r = sqrt(ss / D + eps);
                    for (int d = 0; d < D; ++d)
                        x[d] = x[d] / r * oracle_f16_to_f64(w[d]);
                }
                double *dst = h < Hq ? q_out + ((int64_t)i * Hq + h) * D : k_out + ((int64_t)i * Hkv + (h - Hq)) * D;
                for (int j = 0; j < half; ++j) {
                    double c = (double)cos_t[p * half + j], sn = (double)sin_t[p * half + j];
                    double a = x[j], b = x[j + half];
                    dst[j] = a * c - b * sn;
                    dst[j + half] = b * c + a * sn;
                }
            }
            /* value heads: copied into the pool row */
            for (int h = 0; h < Hkv; ++h) {
                const uint16_t *src = qkv + (int64_t)i * width + (int64_t)(Hq + Hkv + h) * D;
                for (int d = 0; d < D; ++d)
                    v_pool[v_index(&P, blk, h, off, d)] = src[d];
            }
        }
    }
    free(x);
    return rc;
}
