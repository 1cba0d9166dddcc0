/*
 * qsa.h -- C ABI of the Qwen Sparse Attention (QSA) hot path on MI355X (gfx950).
 *
 * QSA is the attention layer the Qwen3.8-Flash-Next pages describe: keys are grouped
 * into 4-token micro-blocks, a small multi-query indexer scores compressed key
 * blocks, a budget of 512 blocks (2,048 tokens) is kept per query while the final
 * incomplete block stays uncompressed, and grouped-query attention with 24 query
 * heads over 2 key/value heads runs over the kept tokens only.
 * Sources: elzobrito.github.io "Long context became an architecture problem",
 * section "Linear attention carries the stream; sparse attention retrieves detail";
 * axbrief.com, section "Shifting from Tokens to Micro-Blocks"; aiany.app, section
 * "Key Capabilities"; hellomarvisaitoday.com, FAQ; blog.compendialabs.org,
 * section "Qwen Sparse Attention -- Full Attention When It Counts".
 *
 * Readings where the pages are silent (the same ones the CPU oracle takes):
 *   - block key K^[b] = bf16(sum of the 4 indexer keys of block b), summed exactly;
 *   - score s[t,b] = sum_h w[t,h] * relu(q_idx[t,h] . K^[b]);
 *   - the kept blocks are the first `topk_blocks` in the order (score descending,
 *     block index ascending); all visible blocks when there are no more than that;
 *   - block b is visible to the query at position t once 4b+3 <= t, i.e. there are
 *     nvis(t) = floor((t+1)/4) visible blocks; tokens 4*nvis(t)..t (0 to 3 of them)
 *     are attended raw, on top of the budget;
 *   - query head h reads key/value head h / 12; one selection per query token;
 *   - softmax scale 1/sqrt(128) unless given; O and lse are fp32.
 *
 * CONVENTIONS
 *   Pointers named *_dev and every tensor pointer are DEVICE pointers owned by the
 *   caller; the library never frees or retains them and allocates no device memory.
 *   Tokens are packed ("varlen"): sequence b owns key rows [cu_k[b], cu_k[b+1]) of
 *   length L_b and query rows [cu_q[b], cu_q[b+1]); its queries are its LAST
 *   q_b = cu_q[b+1]-cu_q[b] tokens (prefill: q_b = L_b; decode: q_b = 1), so query
 *   row r is at position t = L_b - q_b + (r - cu_q[b]). The query's own key/value
 *   and indexer key are already in k, v, k_idx. Compressed blocks are packed by
 *   sequence: sequence b owns block rows [B_b, B_b + floor(L_b/4)) with
 *   B_b = sum_{i<b} floor(L_i/4). Block ids in `sel` are local to the sequence.
 *   Layouts (row-major, bf16 passed as raw 16-bit patterns):
 *     q      [Tq, 24, 128] bf16       k, v   [Tk, 2, 128] bf16
 *     q_idx  [Tq, 4, 64]   bf16       w      [Tq, 4] fp32
 *     k_idx  [Tk, 64]      bf16       k_blk  [sum_b floor(L_b/4), 64] bf16
 *     sel    [Tq, topk]    int32, ascending, padded with -1
 *     out    [Tq, 24, 128] fp32       lse    [Tq, 24] fp32 (natural log)
 *   with Tq = cu_q[batch], Tk = cu_k[batch].
 *
 *   Every call validates its arguments on the host first; on error it returns a
 *   status, enqueues nothing and leaves every output untouched. On success it
 *   enqueues its kernels on `stream` (a hipStream_t of the current device; NULL = the
 *   null stream) and
 *   returns; results are valid once the stream has reached that point. Outputs must
 *   not alias inputs. The workspace starts with a 4 KiB control block (counters
 *   through which the workgroups of one kernel hand work to each other): it must be
 *   zero-filled before the workspace is first used (e.g. one hipMemset at
 *   allocation), and every call leaves it zero when its kernels complete. The rest of
 *   the workspace is undefined before and after a call. Calls on different streams
 *   must not share a workspace, and calls that overlap in time must not either. The
 *   only mutable state is the optional, thread-local kernel trace (diagnostics below),
 *   the thread-local second stream of multi-pass prefills (qsa_forward) and the
 *   scratch array of qsa_forward_noalloc; the library is thread-safe. No exceptions
 *   cross this interface.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 1

typedef uint16_t qsa_bf16; /* raw bf16 bits */

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL                         */
    QSA_ERR_SHAPE = 2,       /* cu_* not starting at 0, decreasing, q_b > L_b,
                                totals beyond int32, topk outside [1, 512]          */
    QSA_ERR_UNSUPPORTED = 3, /* dims other than 24 / 2 / 128 / 4 / 64 / block 4;
                                attention calls: a sequence over 4,194,304 tokens  */
    QSA_ERR_WORKSPACE = 4,   /* ws_bytes smaller than qsa_workspace_size()          */
    QSA_ERR_DEVICE = 5       /* a launch failed (hipGetLastError)                   */
} qsa_status;

typedef struct {
    int32_t n_q_heads;   /* 24                                    */
    int32_t n_kv_heads;  /* 2                                     */
    int32_t head_dim;    /* 128                                   */
    int32_t n_idx_heads; /* 4                                     */
    int32_t idx_dim;     /* 64                                    */
    int32_t block_size;  /* 4                                     */
    int32_t topk_blocks; /* 1..512 (the model: 512)               */
    float softmax_scale; /* <= 0 selects 1/sqrt(head_dim)        */
} qsa_dims;

typedef struct {
    int32_t batch;             /* number of sequences, >= 0                      */
    const int32_t *cu_q_host;  /* [batch+1] host: validation and grid sizing     */
    const int32_t *cu_k_host;  /* [batch+1] host                                 */
    const int32_t *cu_q_dev;   /* [batch+1] device copy of the same values       */
    const int32_t *cu_k_dev;   /* [batch+1] device copy of the same values       */
} qsa_seqs;

/* QSA_ABI_VERSION of the built library. */
int32_t qsa_abi_version(void);

/* Static, human-readable name of a status value (a qsa_status; the parameter is a plain
 * int so that any value a C caller passes is well defined: others name no status and
 * give "unknown qsa_status"). */
const char *qsa_status_string(int32_t status);

/* Bytes of device workspace that qsa_select, qsa_attend and qsa_forward need for
 * these dims and sequences (one size serves all three). Host-only, no device call. */
qsa_status qsa_workspace_size(const qsa_dims *dims, const qsa_seqs *seqs, size_t *bytes);

/* Compress every complete micro-block of every sequence: the pages' "compressed key
 * blocks" (elzobrito.github.io, "Linear attention carries the stream; sparse
 * attention retrieves detail"). k_blk[B_b + i][j] = bf16 round-to-nearest-even of the
 * exact sum k_idx[4i][j] + k_idx[4i+1][j] + k_idx[4i+2][j] + k_idx[4i+3][j] of
 * sequence b. The L_b mod 4 trailing tokens are not compressed. cu_q is not read
 * (seqs->cu_q_* may be NULL). No workspace. */
qsa_status qsa_compress(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *k_idx,
                        qsa_bf16 *k_blk, void *stream);

/* Indexer scoring and top-k block selection for every query row: the small MQA
 * indexer scores compressed blocks and the best `topk_blocks` are kept (aiany.app,
 * "Key Capabilities"; elzobrito.github.io, same section as above). Rows with at most
 * topk_blocks visible blocks keep all of them without scoring. Writes sel [Tq, topk]
 * (ascending local block ids, -1 padded). k_blk must hold every block visible to some
 * query. Needs the workspace. */
qsa_status qsa_select(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q_idx,
                      const float *w, const qsa_bf16 *k_blk, int32_t *sel, void *ws,
                      size_t ws_bytes, void *stream);

/* The indexer scores alone, for the listed query rows: the scoring half of
 * qsa_select (the small MQA indexer of aiany.app, "Key Capabilities", scoring the
 * compressed key blocks of elzobrito.github.io, "Linear attention carries the stream;
 * sparse attention retrieves detail"), computed by the same MFMA code (bf16 products,
 * fp32 sums; exact when the indexer data are small integers).
 *   rows    DEVICE int64 [n_rows]: query rows, each in [0, Tq)
 *   scores  DEVICE fp32 [n_rows, ld], row-major: scores[i][b] = s[t,b] =
 *           sum_h w[t,h] * relu(q_idx[t,h] . K^[b]) for the visible blocks b < nvis(t)
 *           of row rows[i] (a score of -0 is written as +0), -INFINITY for
 *           nvis(t) <= b < ld; a row id outside [0, Tq) gets NaN in every column.
 * ld must be at least the largest floor(L_b/4) (QSA_ERR_SHAPE otherwise); n_rows in
 * [0, INT32_MAX]. k_blk must hold the listed rows' visible blocks. No workspace. */
qsa_status qsa_score(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q_idx,
                     const float *w, const qsa_bf16 *k_blk, const int64_t *rows, int64_t n_rows,
                     float *scores, int64_t ld, void *stream);

/* Grouped-query attention of every query row over the tokens of its selected blocks
 * plus its raw tail (24 query heads paired with 2 KV heads, axbrief.com "Shifting
 * from Tokens to Micro-Blocks"; blog.compendialabs.org "Qwen Sparse Attention --
 * Full Attention When It Counts"). sel entries are read up to the first -1; entries
 * outside [0, nvis(t)) are ignored. Writes out [Tq, 24, 128] fp32 and, if lse is not
 * NULL, lse [Tq, 24] fp32 = log of the softmax denominator of the scaled logits.
 * Needs the workspace. */
qsa_status qsa_attend(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                      const qsa_bf16 *k, const qsa_bf16 *v, const int32_t *sel, float *out,
                      float *lse, void *ws, size_t ws_bytes, void *stream);

/* The whole layer step of the pages' sparse attention, compress -> select -> attend
 * on one stream: compressed key blocks scored by the MQA indexer, the best 512 blocks
 * (2,048 tokens) kept while the final incomplete block stays raw (elzobrito.github.io,
 * "Linear attention carries the stream; sparse attention retrieves detail"; aiany.app,
 * "Key Capabilities"), then attention of the 24 query heads over 2 KV heads on the kept
 * tokens (axbrief.com, "Shifting from Tokens to Micro-Blocks"; blog.compendialabs.org,
 * "Qwen Sparse Attention -- Full Attention When It Counts").
 * If k_idx is not NULL, the blocks that contain at least one query token
 * (blocks floor((L_b - q_b)/4) .. floor(L_b/4)-1 of each sequence) are (re)compressed
 * from k_idx into k_blk first; earlier blocks must already be valid in k_blk (a cache
 * built by qsa_compress or by earlier steps). A prefill therefore compresses every
 * block, a decode step only the block its token completes. If k_idx is NULL, k_blk
 * must already be complete. If sel is NULL the selection is kept in the workspace.
 * lse may be NULL.
 * Streams: the work is ordered on `stream`: it starts after the work enqueued there
 * before the call, and work enqueued there after the call starts after it. A prefill
 * whose selection runs in several passes may attend each pass's rows on a second
 * stream of the library's (one per host thread and device, default priority, created
 * by the first such call and kept until the process ends), forked from and joined back
 * into `stream` by events; both are recorded into a graph that `stream` captures, so
 * capture such a call after one eager call on the same thread has created that
 * stream. */
qsa_status qsa_forward(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                       const qsa_bf16 *k, const qsa_bf16 *v, const qsa_bf16 *q_idx,
                       const float *w, const qsa_bf16 *k_idx, qsa_bf16 *k_blk, int32_t *sel,
                       float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qsa_forward without a workspace
 * argument. Its workspace is a scratch array of QSA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library, one per GPU, held until the process ends; the call allocates
 * nothing. Calls whose qsa_workspace_size exceeds that return QSA_ERR_WORKSPACE before
 * any device call (a decode batch of 16 x 262,144 tokens needs under 8 MiB; a prefill
 * needs its selection when sel is NULL plus its score keys). Every call on a GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams, other
 * host threads) race and must be serialised by the caller. The array's control block
 * is zero before the first call and every call leaves it zero. All of its work runs on
 * `stream` (no second stream). Other arguments and results as qsa_forward. */
#define QSA_NOALLOC_SCRATCH_BYTES (64u << 20)
qsa_status qsa_forward_noalloc(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                               const qsa_bf16 *k, const qsa_bf16 *v, const qsa_bf16 *q_idx,
                               const float *w, const qsa_bf16 *k_idx, qsa_bf16 *k_blk,
                               int32_t *sel, float *out, float *lse, void *stream);

/* ---------------------------------------------------------------- FP8 KV cache
 * A storage variant of the attention's K and V (the pages' FP8 builds are of the
 * model, blog.compendialabs.org, "What This Means"; here FP8 halves the bytes the
 * attention gathers): K and V as OCP FP8 E4M3 bytes, layout k8 / v8 [Tk, 2, 128], with
 * one fp32 scale per (token, KV head), k_scale / v_scale [Tk, 2]. A stored element
 * stands for byte value * scale; the attention is the same computation on those
 * values. Selection does not read K or V and is unchanged. */

/* Builds the FP8 cache of bf16 K and V: for each (token, KV head) row x of 128 values,
 * scale = fp32(amax|x| / 448) (1 for an all-zero row) and byte i = E4M3 rounding
 * (nearest, ties to even; magnitudes beyond 448 saturate) of the fp32 quotient
 * x[i] / scale. cu_q is not read. No workspace. */
qsa_status qsa_quantize_kv(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *k,
                           const qsa_bf16 *v, uint8_t *k8, uint8_t *v8, float *k_scale,
                           float *v_scale, void *stream);

/* qsa_attend over the FP8 cache. All pointers 16-byte aligned. */
qsa_status qsa_attend_fp8(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                          const uint8_t *k8, const uint8_t *v8, const float *k_scale,
                          const float *v_scale, const int32_t *sel, float *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream);

/* qsa_forward over the FP8 cache (compress, selection and streams as in qsa_forward). */
qsa_status qsa_forward_fp8(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                           const uint8_t *k8, const uint8_t *v8, const float *k_scale,
                           const float *v_scale, const qsa_bf16 *q_idx, const float *w,
                           const qsa_bf16 *k_idx, qsa_bf16 *k_blk, int32_t *sel, float *out,
                           float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- backward
 * Gradients of the attention over FIXED selections: the pages speak of how the model
 * was trained (axbrief.com, "Shifting from Tokens to Micro-Blocks", its optimizers) but
 * give no training objective for the indexer,
 * so only the attention is differentiated; selection and compression have no
 * gradient. For a loss whose gradient with respect to out is dout, with P the softmax
 * of the scaled logits of a (row, head) over its attended keys (its selected blocks'
 * tokens and its raw tail, as in qsa_attend) and D = sum_d dout * out of that
 * (row, head):
 *   dP = dout . v_j,   dS = P * (dP - D),
 *   dq = scale * sum_j dS_j k_j,   dk_j = scale * sum dS_j q,   dv_j = sum P_j dout,
 * the last two summed over every (row, head of the key's KV group) that attends key j.
 * Layouts: q, sel, out, lse as in qsa_attend (out and lse as qsa_attend wrote them);
 * dout [Tq, 24, 128] bf16; dq [Tq, 24, 128] fp32; dk, dv [Tk, 2, 128] fp32, written for
 * every key (0 where no row attends it). Results are deterministic: no gradient is
 * accumulated with atomics. The workspace (its own size, below) starts with the same
 * 4 KiB control block as the forward's, which this call does not touch, so one
 * allocation of the larger size serves both. All pointers 16-byte aligned.
 * Streams: ordered on `stream` as qsa_forward; dq is computed on the library's second
 * stream of this host thread and device (see qsa_forward), forked from and joined back
 * into `stream` by events, while dk and dv are computed on `stream`. */

/* Bytes of workspace qsa_attend_backward needs (about 4 * Tq * (topk + 1) for the
 * block -> rows lists plus small tables). Host-only. QSA_ERR_UNSUPPORTED when
 * Tq * (topk + 1) exceeds INT32_MAX. */
qsa_status qsa_backward_workspace_size(const qsa_dims *dims, const qsa_seqs *seqs,
                                       size_t *bytes);

qsa_status qsa_attend_backward(const qsa_dims *dims, const qsa_seqs *seqs, const qsa_bf16 *q,
                               const qsa_bf16 *k, const qsa_bf16 *v, const int32_t *sel,
                               const float *out, const float *lse, const qsa_bf16 *dout,
                               float *dq, float *dk, float *dv, void *ws, size_t ws_bytes,
                               void *stream);

/* ---------------------------------------------------------------- diagnostics
 * Per-kernel timing with HIP events, for benchmarks and profiling. Between
 * qsa_trace_begin and qsa_trace_end on one host thread, each kernel the library
 * launches from that thread (up to max_kernels of them) is bracketed by two HIP events
 * recorded on the kernel's own stream. qsa_trace_end waits for those events, writes
 * each traced kernel's kind (QSA_KERNEL_*) and duration in milliseconds, in launch
 * order, into the caller's host arrays (at most max_out entries) and returns how many
 * kernels were traced (or -1 if no trace was open or an event call failed). The
 * events are created and destroyed by the library; tracing adds a small gap between
 * kernels, so timed runs should not trace. The trace is thread-local state. */
enum {
    QSA_KERNEL_PREP = 0,
    QSA_KERNEL_COMPRESS = 1,
    QSA_KERNEL_SCORE = 2,
    QSA_KERNEL_SELECT = 3,
    QSA_KERNEL_ATTEND = 4,
    QSA_KERNEL_COMBINE = 5,
    QSA_KERNEL_BWD_PREP = 6,
    QSA_KERNEL_BWD_ROWS = 7,
    QSA_KERNEL_BWD_COUNT = 8,
    QSA_KERNEL_BWD_COLSCAN = 9,
    QSA_KERNEL_BWD_SCAN = 10,
    QSA_KERNEL_BWD_FILL = 11,
    QSA_KERNEL_BWD_DQ = 12,
    QSA_KERNEL_BWD_DKV = 13,
    QSA_KERNEL_SCORE_SELECT = 14,  /* prefill: one pass's selection + the next pass's scoring */
    QSA_KERNEL_ATTEND_DENSE = 15   /* prefill rows that keep every visible block (causal) */
};
qsa_status qsa_trace_begin(int32_t max_kernels);
int32_t qsa_trace_end(int32_t max_out, int32_t *kind_out, float *ms_out);
/* Static name of a QSA_KERNEL_* kind ("score", ...). */
const char *qsa_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H */
