/*
 * qsa_ref.h -- CPU oracle of the Qwen Sparse Attention (QSA) hot path.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library. It shares no
 * code, header, table or helper with the HIP library; both sides only receive the
 * same seeded inputs.
 *
 * What it computes (sources are the web pages on Qwen3.8-Flash-Next):
 *   - keys are grouped into 4-token micro-blocks ("Shifting from Tokens to
 *     Micro-Blocks", axbrief.com; FAQ of hellomarvisaitoday.com);
 *   - a small multi-query indexer scores compressed key blocks and the best
 *     blocks, 512 blocks = 2,048 tokens, are kept, while the last incomplete block
 *     stays uncompressed ("Linear attention carries the stream; sparse attention
 *     retrieves detail", elzobrito.github.io; "Key Capabilities", aiany.app);
 *   - attention is grouped-query with 24 query heads sharing 2 key/value heads
 *     ("Shifting from Tokens to Micro-Blocks"; "Qwen Sparse Attention -- Full
 *     Attention When It Counts", blog.compendialabs.org).
 * Steps the pages leave open are fixed by explicit readings, stated at each
 * function below.
 *
 * Everything is computed in double precision from the bf16 / fp32 inputs, which
 * are widened exactly. The only roundings are the ones the definition contains:
 * the compressed block key is stored as bf16 (round to nearest, ties to even).
 *
 * Layouts (row-major, tokens packed across the batch):
 *   sequence b owns key rows [cu_k[b], cu_k[b+1]) (length L_b) and query rows
 *   [cu_q[b], cu_q[b+1]) (q_b of them); its queries are its LAST q_b tokens, so
 *   query row r sits at absolute position t = L_b - q_b + (r - cu_q[b]).
 *   q      bf16 [Tq, Hq, D]        k, v   bf16 [Tk, Hkv, D]
 *   q_idx  bf16 [Tq, Hi, Di]       w      fp32 [Tq, Hi]
 *   k_idx  bf16 [Tk, Di]           k_blk  bf16 [sum_b floor(L_b/bs), Di]
 *   sel    int32 [Tq, topk]  ascending block ids local to the sequence, -1 padded
 *   out    double [Tq, Hq, D]      lse    double [Tq, Hq]
 * bf16 values are passed as their raw 16-bit patterns.
 *
 * Return value: 0 on success, -1 on invalid arguments (nothing written).
 */
#ifndef QSA_REF_H
#define QSA_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t n_q_heads;    /* Hq, 24 in the model                         */
    int32_t n_kv_heads;   /* Hkv, 2 in the model                         */
    int32_t head_dim;     /* D                                           */
    int32_t n_idx_heads;  /* Hi, indexer query heads                     */
    int32_t idx_dim;      /* Di, indexer width                           */
    int32_t block_size;   /* tokens per micro-block, 4 in the model      */
    int32_t topk_blocks;  /* block budget, 512 in the model              */
    double  softmax_scale;/* <= 0 selects 1/sqrt(head_dim)               */
} qsa_ref_dims;

/* Compress every complete block of every sequence. */
int qsa_ref_compress(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_k,
                     const uint16_t *k_idx, uint16_t *k_blk);

/* Scores of one query row against each of its visible blocks (n = visible
 * blocks is written to *n_out; scores must hold at least that many). */
int qsa_ref_row_scores(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q_idx, const float *w,
                       const uint16_t *k_blk, int64_t row, double *scores,
                       int64_t *n_out);

/* Block selection for the listed rows (rows == NULL: every row). */
int qsa_ref_select(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                   const int32_t *cu_k, const uint16_t *q_idx, const float *w,
                   const uint16_t *k_blk, int32_t *sel, const int64_t *rows,
                   int64_t n_rows, int32_t n_threads);

/* Sparse GQA attention over the selected blocks plus the raw tail. */
int qsa_ref_attend(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                   const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, const int32_t *sel, double *out, double *lse,
                   const int64_t *rows, int64_t n_rows, int32_t n_threads);

/* compress (all complete blocks) -> select -> attend. sel may be NULL. */
int qsa_ref_forward(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                    const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const uint16_t *q_idx, const float *w,
                    const uint16_t *k_idx, uint16_t *k_blk, int32_t *sel,
                    double *out, double *lse, const int64_t *rows, int64_t n_rows,
                    int32_t n_threads);

/* FP8 KV cache: K and V as OCP FP8 E4M3 bytes [Tk, Hkv, D] with one fp32 scale per
 * (token, KV head) [Tk, Hkv]; a stored element means byte value * scale. The scale
 * of a row is amax / 448 (1 for an all-zero row) and each byte is the E4M3 rounding
 * (nearest, ties to even) of the fp32 quotient x / scale. This changes how K and V
 * are stored, not what the attention computes: qsa_ref_attend_fp8 is qsa_ref_attend
 * on the dequantized values. */
int qsa_ref_quantize_kv(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_k,
                        const uint16_t *k, const uint16_t *v, uint8_t *k8, uint8_t *v8,
                        float *k_scale, float *v_scale);
int qsa_ref_attend_fp8(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                       const int32_t *cu_k, const uint16_t *q, const uint8_t *k8,
                       const uint8_t *v8, const float *k_scale, const float *v_scale,
                       const int32_t *sel, double *out, double *lse, const int64_t *rows,
                       int64_t n_rows, int32_t n_threads);

/* Backward of qsa_ref_attend over fixed selections: given dout [Tq, Hq, D], the
 * gradients dq [Tq, Hq, D], dk and dv [Tk, Hkv, D] of sum(dout * out). Single-threaded
 * (dk and dv accumulate across rows in the given row order). With rows != NULL only
 * those query rows contribute: their dq, and their shares of dk and dv (every other
 * entry is 0), so a key attended only by those rows gets its full gradient. */
int qsa_ref_attend_backward(const qsa_ref_dims *d, int32_t batch, const int32_t *cu_q,
                            const int32_t *cu_k, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const int32_t *sel, const double *dout,
                            double *dq, double *dk, double *dv, const int64_t *rows,
                            int64_t n_rows);

/* The bf16 and E4M3 roundings the oracle uses and the E4M3 decoding (exposed so tests
 * can pin them). E4M3 rounding saturates magnitudes beyond 448 (infinities too) to 448
 * and maps NaN to the NaN pattern 0x7F (with the sign bit of x). */
uint16_t qsa_ref_bf16_round(double x);
uint8_t qsa_ref_e4m3_round(double x);
double qsa_ref_e4m3_value(uint8_t b);

#ifdef __cplusplus
}
#endif
#endif
