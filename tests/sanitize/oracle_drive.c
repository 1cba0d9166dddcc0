/* oracle_drive.c -- runs every entry point of the CPU oracle on small ragged batches
 * (empty sequences, partial blocks, rows within and beyond the budget, several
 * threads) and on invalid arguments, for a build under AddressSanitizer +
 * UndefinedBehaviorSanitizer and one under ThreadSanitizer (the threaded select and
 * attention). It also checks what holds whatever the values: forward equals compress
 * -> select -> attend, results do not depend on the thread count or on the rows asked
 * for, selections are ascending visible block ids padded with -1.
 *
 * Built by tests/test_sanitizers.py. Exit status 0 and no sanitizer report mean clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qsa_ref.h"

static int g_fail = 0;
#define EXPECT(c)                                                                     \
    do {                                                                              \
        if (!(c)) {                                                                   \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                                 \
        }                                                                             \
    } while (0)

static uint64_t g_rng = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64(void) { /* xorshift64* */
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return g_rng * 2685821657736338717ull;
}
/* a bf16 pattern of a value in [-2, 2) on a 1/64 grid (exactly representable) */
static uint16_t rnd_bf16(void) {
    const float x = (float)((int)(next_u64() % 256) - 128) / 64.0f;
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static void *xcalloc(size_t n, size_t sz) {
    void *p = calloc(n ? n : 1, sz);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

typedef struct {
    int32_t batch;
    int32_t cu_q[16], cu_k[16];
    int64_t tq, tk, nblk;
    uint16_t *q, *k, *v, *q_idx, *k_idx, *k_blk;
    float *w;
} Case;

static void make_case(Case *c, int32_t batch, const int32_t *lens, const int32_t *q_lens,
                      const qsa_ref_dims *d) {
    c->batch = batch;
    c->cu_q[0] = c->cu_k[0] = 0;
    c->nblk = 0;
    for (int b = 0; b < batch; ++b) {
        c->cu_k[b + 1] = c->cu_k[b] + lens[b];
        c->cu_q[b + 1] = c->cu_q[b] + q_lens[b];
        c->nblk += lens[b] / d->block_size;
    }
    c->tq = c->cu_q[batch];
    c->tk = c->cu_k[batch];
    const size_t nq = (size_t)c->tq * d->n_q_heads * d->head_dim;
    const size_t nk = (size_t)c->tk * d->n_kv_heads * d->head_dim;
    c->q = xcalloc(nq, 2);
    c->k = xcalloc(nk, 2);
    c->v = xcalloc(nk, 2);
    c->q_idx = xcalloc((size_t)c->tq * d->n_idx_heads * d->idx_dim, 2);
    c->k_idx = xcalloc((size_t)c->tk * d->idx_dim, 2);
    c->k_blk = xcalloc((size_t)c->nblk * d->idx_dim, 2);
    c->w = xcalloc((size_t)c->tq * d->n_idx_heads, 4);
    for (size_t i = 0; i < nq; ++i) c->q[i] = rnd_bf16();
    for (size_t i = 0; i < nk; ++i) { c->k[i] = rnd_bf16(); c->v[i] = rnd_bf16(); }
    for (int64_t i = 0; i < c->tq * d->n_idx_heads * d->idx_dim; ++i) c->q_idx[i] = rnd_bf16();
    for (int64_t i = 0; i < c->tk * d->idx_dim; ++i) c->k_idx[i] = rnd_bf16();
    for (int64_t i = 0; i < c->tq * d->n_idx_heads; ++i) c->w[i] = 1.0f + (float)(next_u64() % 2);
}

static void free_case(Case *c) {
    free(c->q); free(c->k); free(c->v); free(c->q_idx); free(c->k_idx); free(c->k_blk);
    free(c->w);
}

static void run_case(const qsa_ref_dims *d, int32_t batch, const int32_t *lens,
                     const int32_t *q_lens) {
    Case c;
    make_case(&c, batch, lens, q_lens, d);
    const int K = d->topk_blocks, H = d->n_q_heads, D = d->head_dim;
    const size_t no = (size_t)c.tq * H * D, nl = (size_t)c.tq * H;
    int32_t *sel1 = xcalloc((size_t)c.tq * K, 4), *sel3 = xcalloc((size_t)c.tq * K, 4);
    int32_t *self = xcalloc((size_t)c.tq * K, 4);
    double *o1 = xcalloc(no, 8), *o3 = xcalloc(no, 8), *of = xcalloc(no, 8);
    double *l1 = xcalloc(nl, 8), *l3 = xcalloc(nl, 8), *lf = xcalloc(nl, 8);
    uint16_t *kb2 = xcalloc((size_t)c.nblk * d->idx_dim, 2);

    EXPECT(qsa_ref_compress(d, batch, c.cu_k, c.k_idx, c.k_blk) == 0);
    EXPECT(qsa_ref_select(d, batch, c.cu_q, c.cu_k, c.q_idx, c.w, c.k_blk, sel1, NULL, 0, 1) == 0);
    EXPECT(qsa_ref_select(d, batch, c.cu_q, c.cu_k, c.q_idx, c.w, c.k_blk, sel3, NULL, 0, 3) == 0);
    EXPECT(memcmp(sel1, sel3, (size_t)c.tq * K * 4) == 0);
    /* selections: ascending visible ids, then -1 */
    for (int b = 0; b < batch; ++b) {
        const int64_t L = c.cu_k[b + 1] - c.cu_k[b], nq = c.cu_q[b + 1] - c.cu_q[b];
        for (int64_t r = c.cu_q[b]; r < c.cu_q[b + 1]; ++r) {
            const int64_t t = L - nq + (r - c.cu_q[b]), nv = (t + 1) / d->block_size;
            int seen_pad = 0;
            for (int j = 0; j < K; ++j) {
                const int32_t s = sel1[r * K + j];
                if (s < 0) { EXPECT(s == -1); seen_pad = 1; continue; }
                EXPECT(!seen_pad && s < nv && (j == 0 || s > sel1[r * K + j - 1]));
            }
            int64_t n = 0;
            double *sc = xcalloc((size_t)(nv > 0 ? nv : 1), 8);
            EXPECT(qsa_ref_row_scores(d, batch, c.cu_q, c.cu_k, c.q_idx, c.w, c.k_blk, r, sc,
                                      &n) == 0);
            EXPECT(n == nv);
            free(sc);
        }
    }
    EXPECT(qsa_ref_attend(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, sel1, o1, l1, NULL, 0, 1) == 0);
    EXPECT(qsa_ref_attend(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, sel1, o3, l3, NULL, 0, 4) == 0);
    EXPECT(memcmp(o1, o3, no * 8) == 0 && memcmp(l1, l3, nl * 8) == 0);
    EXPECT(qsa_ref_forward(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, c.q_idx, c.w, c.k_idx, kb2,
                           self, of, lf, NULL, 0, 2) == 0);
    EXPECT(memcmp(self, sel1, (size_t)c.tq * K * 4) == 0);
    EXPECT(memcmp(of, o1, no * 8) == 0 && memcmp(lf, l1, nl * 8) == 0);
    EXPECT(c.nblk == 0 || memcmp(kb2, c.k_blk, (size_t)c.nblk * d->idx_dim * 2) == 0);
    for (size_t i = 0; i < no; ++i) EXPECT(isfinite(o1[i]));

    /* a subset of rows (last, first, a middle one) gives the same rows */
    if (c.tq > 0) {
        const int64_t rows[3] = {c.tq - 1, 0, c.tq / 2};
        int32_t *ss = xcalloc((size_t)c.tq * K, 4);
        double *os = xcalloc(no, 8), *ls = xcalloc(nl, 8);
        EXPECT(qsa_ref_select(d, batch, c.cu_q, c.cu_k, c.q_idx, c.w, c.k_blk, ss, rows, 3, 2) == 0);
        EXPECT(qsa_ref_attend(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, sel1, os, ls, rows, 3, 2) == 0);
        for (int i = 0; i < 3; ++i) {
            const int64_t r = rows[i];
            EXPECT(memcmp(ss + r * K, sel1 + r * K, (size_t)K * 4) == 0);
            EXPECT(memcmp(os + r * H * D, o1 + r * H * D, (size_t)H * D * 8) == 0);
        }
        free(ss); free(os); free(ls);
    }

    /* FP8 cache and its attention */
    {
        const size_t nk = (size_t)c.tk * d->n_kv_heads * D;
        uint8_t *k8 = xcalloc(nk, 1), *v8 = xcalloc(nk, 1);
        float *ks = xcalloc((size_t)c.tk * d->n_kv_heads, 4);
        float *vs = xcalloc((size_t)c.tk * d->n_kv_heads, 4);
        double *o8 = xcalloc(no, 8), *l8 = xcalloc(nl, 8);
        EXPECT(qsa_ref_quantize_kv(d, batch, c.cu_k, c.k, c.v, k8, v8, ks, vs) == 0);
        EXPECT(qsa_ref_attend_fp8(d, batch, c.cu_q, c.cu_k, c.q, k8, v8, ks, vs, sel1, o8, l8,
                                  NULL, 0, 3) == 0);
        for (size_t i = 0; i < no; ++i) EXPECT(isfinite(o8[i]));
        free(k8); free(v8); free(ks); free(vs); free(o8); free(l8);
    }

    /* backward, all rows and a subset */
    {
        const size_t nk = (size_t)c.tk * d->n_kv_heads * D;
        double *dout = xcalloc(no, 8), *dq = xcalloc(no, 8);
        double *dk = xcalloc(nk, 8), *dv = xcalloc(nk, 8);
        for (size_t i = 0; i < no; ++i) dout[i] = (double)((int)(next_u64() % 64) - 32) / 16.0;
        EXPECT(qsa_ref_attend_backward(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, sel1, dout, dq,
                                       dk, dv, NULL, 0) == 0);
        if (c.tq > 0) {
            const int64_t rows[2] = {c.tq - 1, 0};
            EXPECT(qsa_ref_attend_backward(d, batch, c.cu_q, c.cu_k, c.q, c.k, c.v, sel1, dout,
                                           dq, dk, dv, rows, 2) == 0);
        }
        free(dout); free(dq); free(dk); free(dv);
    }

    free(sel1); free(sel3); free(self); free(o1); free(o3); free(of); free(l1); free(l3);
    free(lf); free(kb2);
    free_case(&c);
}

int main(void) {
    qsa_ref_dims d = {24, 2, 128, 4, 64, 4, 4, 0.0};

    /* tiny, empty and ragged sequences, partial blocks, decode rows */
    {
        const int32_t lens[] = {7, 1, 2, 3, 0, 64, 45};
        const int32_t ql[] = {7, 1, 2, 3, 0, 64, 9};
        run_case(&d, 7, lens, ql);
    }
    d.topk_blocks = 1;
    {
        const int32_t lens[] = {1, 13}, ql[] = {1, 13};
        run_case(&d, 2, lens, ql);
    }
    d.topk_blocks = 16;
    {
        const int32_t lens[] = {300, 133, 5}, ql[] = {3, 133, 0};
        run_case(&d, 3, lens, ql);
    }
    d.topk_blocks = 512; /* the model's budget: these rows keep every block */
    {
        const int32_t lens[] = {70, 9}, ql[] = {70, 1};
        run_case(&d, 2, lens, ql);
    }
    /* a batch of nothing */
    run_case(&d, 0, NULL, NULL);

    /* the roundings at their edges */
    {
        const double xs[] = {0.0, -0.0, 1.0, -1.0, 3.0e38, -3.5e38, 1e-45, 1e-40, 448.0, 449.0,
                             464.0, 1e6, 0.0009765625, 1.0 / 0.0, -1.0 / 0.0, 0.0 / 0.0};
        for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
            (void)qsa_ref_bf16_round(xs[i]);
            (void)qsa_ref_e4m3_round(xs[i]);
        }
        for (int b = 0; b < 256; ++b) (void)qsa_ref_e4m3_value((uint8_t)b);
        EXPECT(qsa_ref_bf16_round(1.0) == 0x3F80);
    }

    /* invalid arguments: rejected with -1, nothing written */
    {
        int32_t cq[2] = {0, 8}, ck[2] = {0, 4}; /* more queries than keys */
        uint16_t kb[64];
        int32_t sel[8 * 4];
        double out[8], lse[8];
        float w[8 * 4] = {0};
        memset(sel, 0x7f, sizeof sel);
        EXPECT(qsa_ref_compress(NULL, 1, ck, kb, kb) == -1);
        EXPECT(qsa_ref_select(&d, 1, cq, ck, kb, w, kb, sel, NULL, 0, 1) == -1);
        EXPECT(sel[0] == 0x7f7f7f7f);
        EXPECT(qsa_ref_attend(&d, -1, cq, ck, kb, kb, kb, sel, out, lse, NULL, 0, 1) == -1);
        qsa_ref_dims bad = d;
        bad.topk_blocks = 0;
        int32_t cq2[2] = {0, 1}, ck2[2] = {0, 4};
        EXPECT(qsa_ref_select(&bad, 1, cq2, ck2, kb, w, kb, sel, NULL, 0, 1) == -1);
        const int64_t bad_row = 5;
        int64_t n = 0;
        double sc[4];
        EXPECT(qsa_ref_row_scores(&d, 1, cq2, ck2, kb, w, kb, bad_row, sc, &n) == -1);
    }

    if (g_fail) {
        fprintf(stderr, "%d expectation(s) failed\n", g_fail);
        return 1;
    }
    printf("oracle_drive: ok\n");
    return 0;
}
