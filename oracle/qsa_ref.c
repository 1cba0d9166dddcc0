/*
 * qsa_ref.c -- plain, slow, obviously correct CPU oracle of the QSA hot path.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg use it. It shares no code with the
 * HIP library. Arithmetic is double precision throughout; the steps follow the
 * order in which the pages describe the layer: compress key blocks, score them
 * with the indexer, keep the best blocks, attend over the kept tokens.
 *
 * Readings taken where the pages are silent (each is restated at its step; the
 * numbers are the ones the design notes use for the same readings):
 *   R1  compression of a micro-block = sum of its indexer keys, stored as bf16;
 *   R3  score = sum_h w[t,h] * relu(q_idx[t,h] . K^[b]) with relu(x) = x>0 ? x : +0;
 *   R4  order = score descending, ties to the lower block index;
 *   R5  the budget counts compressed blocks only: the raw tail is attended on top;
 *   R6  a block is a candidate once all of its tokens are at or before the query;
 *       the tokens after the last complete block (0..bs-1 of them) are attended raw;
 *   R8  query head h uses key/value head h / (Hq/Hkv) (contiguous groups);
 *   R9  softmax scale 1/sqrt(D) unless given;
 *   R10 output and log-sum-exp per head;
 *   R11 a query with no more visible blocks than the budget keeps all of them;
 *   R14 one selection per query token, shared by every head;
 *   R18 FP8 cache: E4M3 bytes with one fp32 scale per (token, KV head) row;
 *   R19 the backward differentiates the attention over fixed selections.
 */
#include "qsa_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round x to the nearest bf16 value, ties to even. bf16 keeps 8 significant bits
 * and the fp32 exponent range, so the rounding quantum is 2^(e-8) for
 * x = m * 2^e with 0.5 <= |m| < 1, never finer than the subnormal step 2^-133. */
uint16_t qsa_ref_bf16_round(double x)
{
    if (x == 0.0)
        return signbit(x) ? 0x8000u : 0x0000u;
    int e;
    (void)frexp(x, &e);
    int qe = (e < -125 ? -125 : e) - 8;
    double r = ldexp(nearbyint(ldexp(x, -qe)), qe); /* default mode: ties to even */
    if (fabs(r) >= 0x1p128)
        return x > 0 ? 0x7f80u : 0xff80u;
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------- fp8 */

/* OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities, S.1111.111 is NaN, largest finite magnitude 448, subnormals m/8 * 2^-6. */
static double e4m3_value(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

double qsa_ref_e4m3_value(uint8_t b) { return e4m3_value(b); }

/* Round x to the nearest E4M3 value, ties to even; magnitudes beyond 448 (infinities
 * included) saturate to 448 and NaN gives the format's NaN pattern (quantization only
 * ever rounds finite quotients). The rounding quantum is 2^(e-4) for |x| = m * 2^e
 * with 0.5 <= m < 1, never finer than the subnormal step 2^-9. */
uint8_t qsa_ref_e4m3_round(double x)
{
    uint8_t sign = signbit(x) ? 0x80u : 0x00u;
    double a = fabs(x);
    if (isnan(x))
        return (uint8_t)(sign | 0x7Fu);
    if (a == 0.0)
        return sign;
    if (a > 448.0)
        a = 448.0;
    int e;
    (void)frexp(a, &e);
    int qe = (e < -5 ? -5 : e) - 4;
    double r = ldexp(nearbyint(ldexp(a, -qe)), qe); /* default mode: ties to even */
    if (r > 448.0)
        r = 448.0;
    /* encode r exactly */
    if (r < 0x1p-6)
        return (uint8_t)(sign | (uint8_t)nearbyint(ldexp(r, 9)));
    int re;
    double mr = frexp(r, &re);              /* r = mr * 2^re, 0.5 <= mr < 1 */
    int m = (int)nearbyint(ldexp(mr, 4)) - 8;  /* 3 mantissa bits */
    int eb = re - 1 + 7;                    /* biased exponent */
    return (uint8_t)(sign | (uint8_t)(eb << 3) | (uint8_t)m);
}

/* ------------------------------------------------------------ bookkeeping */

static int dims_ok(const qsa_ref_dims *d)
{
    return d && d->n_q_heads > 0 && d->n_kv_heads > 0 && d->head_dim > 0 &&
           d->n_q_heads % d->n_kv_heads == 0 && d->n_idx_heads > 0 && d->idx_dim > 0 &&
           d->block_size > 0 && d->topk_blocks > 0;
}

static int seqs_ok(int32_t batch, const int32_t *cu_q, const int32_t *cu_k)
{
    if (batch < 0 || !cu_k)
        return 0;
    if (cu_k[0] != 0 || (cu_q && cu_q[0] != 0))
        return 0;
    for (int32_t b = 0; b < batch; ++b) {
        int32_t L = cu_k[b + 1] - cu_k[b];
        if (L < 0)
            return 0;
        if (cu_q) {
            int32_t nq = cu_q[b + 1] - cu_q[b];
            if (nq < 0 || nq > L)
                return 0;
        }
    }
    return 1;
}

/* Where query row r lives: its sequence, its absolute position t, the
 * sequence's first key row and first compressed block. */
typedef struct {
    int32_t seq;
    int64_t t;
    int64_t key0;
    int64_t blk0;
} row_pos;

static row_pos locate_row(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                          const int32_t *cu_k, int64_t r)
{
    row_pos p = {-1, 0, 0, 0};
    int64_t blk0 = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = cu_k[b + 1] - cu_k[b];
        if (r >= cu_q[b] && r < cu_q[b + 1]) {
            int64_t nq = cu_q[b + 1] - cu_q[b];
            p.seq = b;
            p.t = L - nq + (r - cu_q[b]);
            p.key0 = cu_k[b];
            p.blk0 = blk0;
            return p;
        }
        blk0 += L / d->block_size;
    }
    return p;
}

/* Reading R6: blocks whose every token is at or before t. */
static int64_t visible_blocks(const qsa_ref_dims *d, int64_t t)
{
    return (t + 1) / d->block_size;
}

/* ------------------------------------------------------------- step 1 */

/* Compressed key blocks. The pages have the indexer score compressed key blocks of
 * 4-token micro-blocks but do not give the operator (elzobrito.github.io,
 * "Linear attention carries the stream; sparse attention retrieves detail").
 * Reading R1: the block key is the sum of the block's indexer keys, taken in token
 * order and stored as bf16. Only complete blocks are compressed; the trailing
 * L mod bs tokens stay raw. */
int qsa_ref_compress(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_k,
                     const uint16_t *k_idx, uint16_t *k_blk)
{
    if (!dims_ok(d) || !seqs_ok(batch, NULL, cu_k) ||
        ((!k_idx || !k_blk) && cu_k[batch] > 0))
        return -1;
    const int64_t Di = d->idx_dim, bs = d->block_size;
    int64_t out_b = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = cu_k[b + 1] - cu_k[b];
        for (int64_t blk = 0; blk < L / bs; ++blk, ++out_b) {
            for (int64_t j = 0; j < Di; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < bs; ++i)
                    s += bf16_value(k_idx[(cu_k[b] + blk * bs + i) * Di + j]);
                k_blk[out_b * Di + j] = qsa_ref_bf16_round(s);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------- step 2 */

static double relu(double x) { return x > 0.0 ? x : 0.0; }

/* Indexer score of block `blk` for one query row. The pages describe a small
 * indexer whose query heads share one key ("MQA indexer", aiany.app, "Key
 * Capabilities") scoring compressed blocks. Reading R3:
 *     s = sum_h w[h] * relu(q_idx[h] . K^[blk]). */
static double block_score(const qsa_ref_dims *d, const double *qi_row, const float *w_row,
                          const uint16_t *kb, double *kd)
{
    const int64_t Hi = d->n_idx_heads, Di = d->idx_dim;
    for (int64_t j = 0; j < Di; ++j)
        kd[j] = bf16_value(kb[j]);
    double s = 0.0;
    for (int64_t h = 0; h < Hi; ++h) {
        double dot = 0.0;
        for (int64_t j = 0; j < Di; ++j)
            dot += qi_row[h * Di + j] * kd[j];
        s += (double)w_row[h] * relu(dot);
    }
    return s;
}

/* The indexer query of one row as doubles (exact), [Hi * Di]. NULL if out of memory. */
static double *widen_row(const qsa_ref_dims *d, const uint16_t *qi_row)
{
    const int64_t n = (int64_t)d->n_idx_heads * d->idx_dim;
    double *qd = (double *)malloc((size_t)(n + d->idx_dim) * sizeof *qd);
    if (qd)
        for (int64_t i = 0; i < n; ++i)
            qd[i] = bf16_value(qi_row[i]);
    return qd;
}

int qsa_ref_row_scores(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q_idx, const float *w,
                       const uint16_t *k_blk, int64_t row, double *scores,
                       int64_t *n_out)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || row < 0 ||
        row >= cu_q[batch] || !n_out)
        return -1;
    row_pos p = locate_row(d, batch, cu_q, cu_k, row);
    int64_t nv = visible_blocks(d, p.t);
    const int64_t Hi = d->n_idx_heads, Di = d->idx_dim;
    double *qd = widen_row(d, q_idx + row * Hi * Di);
    if (!qd)
        return -1;
    for (int64_t blk = 0; blk < nv; ++blk)
        scores[blk] = block_score(d, qd, w + row * Hi, k_blk + (p.blk0 + blk) * Di,
                                  qd + Hi * Di);
    free(qd);
    *n_out = nv;
    return 0;
}

/* ------------------------------------------------------------- step 3 */

typedef struct {
    double s;
    int32_t blk;
} scored_block;

/* Reading R4: higher score first; equal scores go to the lower block index. */
static int by_score_then_index(const void *a, const void *b)
{
    const scored_block *x = (const scored_block *)a, *y = (const scored_block *)b;
    if (x->s != y->s)
        return x->s > y->s ? -1 : 1;
    return (x->blk > y->blk) - (x->blk < y->blk);
}

static int by_index(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Keep the budget of best blocks: the pages give the budget as 512 blocks, i.e.
 * 2,048 tokens per query (elzobrito.github.io, "Linear attention carries the stream;
 * sparse attention retrieves detail"). Reading R11: a query with no more visible
 * blocks than the budget keeps all of them. The kept ids are written in ascending
 * order and the row is padded with -1. */
static void select_row(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q_idx, const float *w,
                       const uint16_t *k_blk, int64_t row, int32_t *sel_row)
{
    const int64_t k = d->topk_blocks, Hi = d->n_idx_heads, Di = d->idx_dim;
    row_pos p = locate_row(d, batch, cu_q, cu_k, row);
    int64_t nv = visible_blocks(d, p.t);
    int64_t kept = nv < k ? nv : k;
    if (nv <= k) {
        for (int64_t i = 0; i < nv; ++i)
            sel_row[i] = (int32_t)i;
    } else {
        scored_block *c = (scored_block *)malloc((size_t)nv * sizeof *c);
        double *qd = widen_row(d, q_idx + row * Hi * Di);
        for (int64_t blk = 0; blk < nv; ++blk) {
            c[blk].s = block_score(d, qd, w + row * Hi, k_blk + (p.blk0 + blk) * Di,
                                   qd + Hi * Di);
            c[blk].blk = (int32_t)blk;
        }
        free(qd);
        qsort(c, (size_t)nv, sizeof *c, by_score_then_index);
        for (int64_t i = 0; i < k; ++i)
            sel_row[i] = c[i].blk;
        free(c);
        qsort(sel_row, (size_t)k, sizeof *sel_row, by_index);
    }
    for (int64_t i = kept; i < k; ++i)
        sel_row[i] = -1;
}

/* ------------------------------------------------------------- step 4 */

/* Attention of one query row. Keys: the tokens of the kept blocks, in ascending
 * order, then the raw tokens after the last complete block (readings R5 and R6: the
 * last, incomplete block is attended without compression, elzobrito.github.io). A
 * row's selection is read up to its first negative entry; entries naming a block that
 * is not visible at t (b >= nvis(t): reading R6, only complete blocks at or before t
 * are candidates) are not attended, so a selection supplied from outside can never
 * reach past the row's position. Query head
 * h reads key/value head h / (Hq/Hkv): the 24 query heads share 2 key/value heads
 * (axbrief.com, "Shifting from Tokens to Micro-Blocks"), twelve per KV head
 * (blog.compendialabs.org, "Qwen Sparse Attention -- Full Attention When It
 * Counts"). Softmax with a max shift, then normalisation; lse = m + ln(l) of the
 * scaled logits. */
/* One element of K or V: bf16, or (FP8 KV cache) an E4M3 byte times the fp32 scale
 * of its (token, KV head) row. */
typedef struct {
    const uint16_t *bf;
    const uint8_t *f8;
    const float *scale;
} kv_src;

static double kv_value(const kv_src *s, int64_t token, int64_t g, int64_t Hkv, int64_t D,
                       int64_t c)
{
    int64_t r = token * Hkv + g;
    if (s->f8)
        return e4m3_value(s->f8[r * D + c]) * (double)s->scale[r];
    return bf16_value(s->bf[r * D + c]);
}

static void attend_row(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q, const kv_src *k,
                       const kv_src *v, const int32_t *sel_row, int64_t row,
                       double *out_row, double *lse_row)
{
    const int64_t Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
    const int64_t bs = d->block_size, kb = d->topk_blocks;
    const double scale = d->softmax_scale > 0 ? d->softmax_scale : 1.0 / sqrt((double)D);
    row_pos p = locate_row(d, batch, cu_q, cu_k, row);
    int64_t nv = visible_blocks(d, p.t);

    /* the attended positions J(t), ascending */
    int64_t n_sel = 0, n_vis = 0;
    while (n_sel < kb && sel_row[n_sel] >= 0)
        n_vis += sel_row[n_sel++] < nv;
    int64_t n_tail = p.t + 1 - nv * bs;
    int64_t nj = n_vis * bs + n_tail;
    int64_t *J = (int64_t *)malloc((size_t)nj * sizeof *J);
    int64_t n = 0;
    for (int64_t i = 0; i < n_sel; ++i)
        if (sel_row[i] < nv)
            for (int64_t j = 0; j < bs; ++j)
                J[n++] = (int64_t)sel_row[i] * bs + j;
    for (int64_t j = nv * bs; j <= p.t; ++j)
        J[n++] = j;

    /* the attended K and V rows of a key/value head, widened once for the query heads
     * that read it */
    double *z = (double *)malloc((size_t)nj * sizeof *z);
    double *kd = (double *)malloc((size_t)(nj * D + 1) * sizeof *kd);
    double *vd = (double *)malloc((size_t)(nj * D + 1) * sizeof *vd);
    int64_t g_wide = -1;
    for (int64_t h = 0; h < Hq; ++h) {
        int64_t g = h / (Hq / Hkv);
        if (g != g_wide) {
            for (int64_t i = 0; i < nj; ++i)
                for (int64_t c = 0; c < D; ++c) {
                    kd[i * D + c] = kv_value(k, p.key0 + J[i], g, Hkv, D, c);
                    vd[i * D + c] = kv_value(v, p.key0 + J[i], g, Hkv, D, c);
                }
            g_wide = g;
        }
        const uint16_t *qh = q + (row * Hq + h) * D;
        double m = -INFINITY;
        for (int64_t i = 0; i < nj; ++i) {
            double dot = 0.0;
            for (int64_t c = 0; c < D; ++c)
                dot += bf16_value(qh[c]) * kd[i * D + c];
            z[i] = dot * scale;
            if (z[i] > m)
                m = z[i];
        }
        double l = 0.0;
        for (int64_t i = 0; i < nj; ++i) {
            z[i] = exp(z[i] - m);
            l += z[i];
        }
        double *o = out_row + h * D;
        for (int64_t c = 0; c < D; ++c)
            o[c] = 0.0;
        for (int64_t i = 0; i < nj; ++i)
            for (int64_t c = 0; c < D; ++c)
                o[c] += z[i] * vd[i * D + c];
        for (int64_t c = 0; c < D; ++c)
            o[c] /= l;
        if (lse_row)
            lse_row[h] = m + log(l);
    }
    free(vd);
    free(kd);
    free(z);
    free(J);
}

/* ------------------------------------------------------- row-parallel loop */

typedef struct {
    int op; /* 0 select, 1 attend */
    const qsa_ref_dims *d;
    int32_t batch;
    const int32_t *cu_q, *cu_k;
    const uint16_t *q, *q_idx, *k_blk;
    kv_src k, v;
    const float *w;
    int32_t *sel_w;
    const int32_t *sel_r;
    double *out, *lse;
    const int64_t *rows;
    int64_t lo, hi, step;
} row_job;

static void *run_rows(void *arg)
{
    row_job *j = (row_job *)arg;
    const int64_t kb = j->d->topk_blocks, Hq = j->d->n_q_heads, D = j->d->head_dim;
    for (int64_t i = j->lo; i < j->hi; i += j->step) {
        int64_t r = j->rows ? j->rows[i] : i;
        if (j->op == 0)
            select_row(j->d, j->batch, j->cu_q, j->cu_k, j->q_idx, j->w, j->k_blk, r,
                       j->sel_w + r * kb);
        else
            attend_row(j->d, j->batch, j->cu_q, j->cu_k, j->q, &j->k, &j->v,
                       j->sel_r + r * kb, r, j->out + r * Hq * D,
                       j->lse ? j->lse + r * Hq : NULL);
    }
    return NULL;
}

static void for_rows(row_job proto, int64_t n_rows, int32_t n_threads)
{
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if (n_rows < n_threads)
        n_threads = n_rows > 0 ? (int32_t)n_rows : 1;
    pthread_t tid[256];
    row_job jobs[256];
    for (int32_t i = 0; i < n_threads; ++i) {
        jobs[i] = proto;
        jobs[i].lo = i;             /* rows i, i + n_threads, ...: costs grow with t */
        jobs[i].hi = n_rows;
        jobs[i].step = n_threads;
    }
    for (int32_t i = 1; i < n_threads; ++i)
        pthread_create(&tid[i], NULL, run_rows, &jobs[i]);
    run_rows(&jobs[0]);
    for (int32_t i = 1; i < n_threads; ++i)
        pthread_join(tid[i], NULL);
}

static int rows_ok(const int32_t *cu_q, int32_t batch, const int64_t *rows, int64_t n_rows)
{
    if (!rows)
        return 1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= cu_q[batch])
            return 0;
    return 1;
}

int qsa_ref_select(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                   const int32_t *cu_k, const uint16_t *q_idx, const float *w,
                   const uint16_t *k_blk, int32_t *sel, const int64_t *rows,
                   int64_t n_rows, int32_t n_threads)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || !sel ||
        !rows_ok(cu_q, batch, rows, n_rows))
        return -1;
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = 0;
    j.d = d;
    j.batch = batch;
    j.cu_q = cu_q;
    j.cu_k = cu_k;
    j.q_idx = q_idx;
    j.w = w;
    j.k_blk = k_blk;
    j.sel_w = sel;
    j.rows = rows;
    for_rows(j, rows ? n_rows : cu_q[batch], n_threads);
    return 0;
}

int qsa_ref_attend(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                   const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, const int32_t *sel, double *out, double *lse,
                   const int64_t *rows, int64_t n_rows, int32_t n_threads)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || !sel || !out ||
        !rows_ok(cu_q, batch, rows, n_rows))
        return -1;
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = 1;
    j.d = d;
    j.batch = batch;
    j.cu_q = cu_q;
    j.cu_k = cu_k;
    j.q = q;
    j.k.bf = k;
    j.v.bf = v;
    j.sel_r = sel;
    j.out = out;
    j.lse = lse;
    j.rows = rows;
    for_rows(j, rows ? n_rows : cu_q[batch], n_threads);
    return 0;
}

/* FP8 KV cache (a variant of the attention's K/V storage; the attention is defined on
 * the dequantized values): each (token, KV head) row x of K or V gets the fp32 scale
 * s = amax|x| / 448 (1 for an all-zero row) and the bytes e4m3_round(fp32(x / s)),
 * both divisions in fp32 (computed here in double and rounded once to fp32, which
 * gives the correctly rounded fp32 quotient). */
int qsa_ref_quantize_kv(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_k,
                        const uint16_t *k, const uint16_t *v, uint8_t *k8, uint8_t *v8,
                        float *k_scale, float *v_scale)
{
    if (!dims_ok(d) || !seqs_ok(batch, NULL, cu_k) || !k || !v || !k8 || !v8 ||
        !k_scale || !v_scale)
        return -1;
    const int64_t rows = (int64_t)cu_k[batch] * d->n_kv_heads, D = d->head_dim;
    for (int which = 0; which < 2; ++which) {
        const uint16_t *x = which ? v : k;
        uint8_t *q8 = which ? v8 : k8;
        float *sc = which ? v_scale : k_scale;
        for (int64_t r = 0; r < rows; ++r) {
            double amax = 0.0;
            for (int64_t c = 0; c < D; ++c)
                amax = fmax(amax, fabs(bf16_value(x[r * D + c])));
            float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
            sc[r] = s;
            for (int64_t c = 0; c < D; ++c) {
                float y = (float)(bf16_value(x[r * D + c]) / (double)s);
                q8[r * D + c] = qsa_ref_e4m3_round((double)y);
            }
        }
    }
    return 0;
}

int qsa_ref_attend_fp8(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q, const uint8_t *k8,
                       const uint8_t *v8, const float *k_scale, const float *v_scale,
                       const int32_t *sel, double *out, double *lse, const int64_t *rows,
                       int64_t n_rows, int32_t n_threads)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || !sel || !out || !k8 || !v8 ||
        !k_scale || !v_scale || !rows_ok(cu_q, batch, rows, n_rows))
        return -1;
    row_job j;
    memset(&j, 0, sizeof j);
    j.op = 1;
    j.d = d;
    j.batch = batch;
    j.cu_q = cu_q;
    j.cu_k = cu_k;
    j.q = q;
    j.k.f8 = k8;
    j.k.scale = k_scale;
    j.v.f8 = v8;
    j.v.scale = v_scale;
    j.sel_r = sel;
    j.out = out;
    j.lse = lse;
    j.rows = rows;
    for_rows(j, rows ? n_rows : cu_q[batch], n_threads);
    return 0;
}

/* ------------------------------------------------------------- backward */

/* Gradients of the attention over fixed selections: for the scalar
 * sum_{t,h,c} dout[t,h,c] * out[t,h,c], with out as in qsa_ref_attend, the partial
 * derivatives with respect to q, k and v. The selection is a fixed input (it is not
 * differentiable; the pages give no training objective for the indexer). Per row and
 * head, with z_j = scale * q.k_j and p = softmax(z) over the attended tokens J(t):
 *   dP_j = dout . v_j,  dS_j = p_j * (dP_j - sum_i p_i dP_i),
 *   dq += scale * sum_j dS_j k_j,  dk_j += scale * dS_j q,  dv_j += p_j dout,
 * with dk, dv summed over every (row, head) that attends the token (row order). */
int qsa_ref_attend_backward(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                            const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const int32_t *sel, const double *dout,
                            double *dq, double *dk, double *dv, const int64_t *rows,
                            int64_t n_rows)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || !q || !k || !v || !sel ||
        !dout || !dq || !dk || !dv || !rows_ok(cu_q, batch, rows, n_rows))
        return -1;
    const int64_t Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
    const int64_t bs = d->block_size, kb = d->topk_blocks;
    const double scale = d->softmax_scale > 0 ? d->softmax_scale : 1.0 / sqrt((double)D);
    const int64_t tq = cu_q[batch], tk = cu_k[batch];
    memset(dq, 0, (size_t)(tq * Hq * D) * sizeof *dq);
    memset(dk, 0, (size_t)(tk * Hkv * D) * sizeof *dk);
    memset(dv, 0, (size_t)(tk * Hkv * D) * sizeof *dv);
    int64_t *J = (int64_t *)malloc((size_t)(kb * bs + bs) * sizeof *J);
    double *z = (double *)malloc((size_t)(kb * bs + bs) * sizeof *z);
    double *dp = (double *)malloc((size_t)(kb * bs + bs) * sizeof *dp);
    if (!J || !z || !dp) {
        free(J), free(z), free(dp);
        return -1;
    }
    const int64_t n_loop = rows ? n_rows : tq;
    for (int64_t ri = 0; ri < n_loop; ++ri) {
        const int64_t row = rows ? rows[ri] : ri;
        row_pos p = locate_row(d, batch, cu_q, cu_k, row);
        const int64_t nv = visible_blocks(d, p.t);
        const int32_t *sel_row = sel + row * kb;
        int64_t n_sel = 0;
        while (n_sel < kb && sel_row[n_sel] >= 0)
            ++n_sel;
        int64_t nj = 0;
        for (int64_t i = 0; i < n_sel; ++i)
            if (sel_row[i] < nv)   /* as in the forward: invisible blocks are not attended */
                for (int64_t j = 0; j < bs; ++j)
                    J[nj++] = p.key0 + (int64_t)sel_row[i] * bs + j;
        for (int64_t j = nv * bs; j <= p.t; ++j)
            J[nj++] = p.key0 + j;
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / (Hq / Hkv);
            const uint16_t *qh = q + (row * Hq + h) * D;
            const double *go = dout + (row * Hq + h) * D;
            double m = -INFINITY;
            for (int64_t i = 0; i < nj; ++i) {
                double dot = 0.0;
                for (int64_t c = 0; c < D; ++c)
                    dot += bf16_value(qh[c]) * bf16_value(k[(J[i] * Hkv + g) * D + c]);
                z[i] = dot * scale;
                if (z[i] > m)
                    m = z[i];
            }
            double l = 0.0;
            for (int64_t i = 0; i < nj; ++i) {
                z[i] = exp(z[i] - m);
                l += z[i];
            }
            double pdp = 0.0;
            for (int64_t i = 0; i < nj; ++i) {
                z[i] /= l; /* p_i */
                double s = 0.0;
                for (int64_t c = 0; c < D; ++c)
                    s += go[c] * bf16_value(v[(J[i] * Hkv + g) * D + c]);
                dp[i] = s;
                pdp += z[i] * s;
            }
            double *gq = dq + (row * Hq + h) * D;
            for (int64_t i = 0; i < nj; ++i) {
                const double ds = z[i] * (dp[i] - pdp);
                const int64_t r = J[i] * Hkv + g;
                for (int64_t c = 0; c < D; ++c) {
                    gq[c] += scale * ds * bf16_value(k[r * D + c]);
                    dk[r * D + c] += scale * ds * bf16_value(qh[c]);
                    dv[r * D + c] += z[i] * go[c];
                }
            }
        }
    }
    free(J);
    free(z);
    free(dp);
    return 0;
}

int qsa_ref_forward(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                    const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const uint16_t *q_idx, const float *w,
                    const uint16_t *k_idx, uint16_t *k_blk, int32_t *sel,
                    double *out, double *lse, const int64_t *rows, int64_t n_rows,
                    int32_t n_threads)
{
    if (!dims_ok(d) || !cu_q || !seqs_ok(batch, cu_q, cu_k) || !k_blk || !out ||
        !rows_ok(cu_q, batch, rows, n_rows))
        return -1;
    if (qsa_ref_compress(d, batch, cu_k, k_idx, k_blk) != 0)
        return -1;
    int32_t *s = sel;
    if (!s) {
        s = (int32_t *)malloc((size_t)cu_q[batch] * (size_t)d->topk_blocks * sizeof *s + 1);
        if (!s)
            return -1;
    }
    int rc = qsa_ref_select(d, batch, cu_q, cu_k, q_idx, w, k_blk, s, rows, n_rows, n_threads);
    if (rc == 0)
        rc = qsa_ref_attend(d, batch, cu_q, cu_k, q, k, v, s, out, lse, rows, n_rows,
                            n_threads);
    if (!sel)
        free(s);
    return rc;
}
