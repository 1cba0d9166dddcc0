// qsa_launch.h -- host-side launchers of the QSA kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

struct SeqInfo;
struct DecodeTables;

// FP8 KV cache operands: E4M3 bytes [Tk, 2, 128] and fp32 scales [Tk, 2].
struct Fp8Kv {
    const uint8_t *k8, *v8;
    const float *k_scale, *v_scale;
};

// Chunk lists one decode merge takes with 8 candidates per thread; rows of up to
// MERGE_CHUNKS_WIDE chunks are merged after scoring with 32 per thread.
constexpr int MERGE_CHUNKS = 64;
constexpr int MERGE_CHUNKS_WIDE = 256;

// Prefill score + select launches whose rows see more blocks than this take the variant
// for long rows (score tiles grouped 4 at a time, selections that list the first radix
// digit's crossing bin in LDS); the others keep the leaner kernel, at more waves per SIMD.
constexpr int64_t SEL_LONG_KEYS = 16384;

// Optional per-kernel event trace (thread-local; see qsa_trace_begin).
void trace_before(int kind, hipStream_t st);
hipError_t trace_after(hipStream_t st, hipError_t launch_status);

hipError_t launch_prep(const int32_t *cu_q, const int32_t *cu_k, int batch, int topk,
                       SeqInfo *tab, hipStream_t st);
hipError_t launch_compress(const int32_t *cu_q, const int32_t *cu_k, int batch,
                           int64_t max_blocks, const uint16_t *k_idx, uint16_t *k_blk,
                           int incremental, SeqInfo *tab, int topk, hipStream_t st);
// One prefill launch: selection of rows [row_base, row_base + n_rows) from sel_keys
// (slot s at sel_keys[s - sel_slot_base]) and, at the same time, scoring of tiles
// [tile_base, tile_base + n_tiles) into score_keys (slot s at score_keys[s -
// score_slot_base]); either part may be empty.
hipError_t launch_score_select(const SeqInfo *tab, int batch, int topk, const uint16_t *q_idx,
                               const float *w, const uint16_t *k_blk, uint32_t *score_keys,
                               int64_t tile_base, int64_t n_tiles, int64_t score_slot_base,
                               int64_t max_blocks, int64_t chunk_blocks,
                               const uint32_t *sel_keys, int64_t sel_slot_base, int32_t *sel,
                               int64_t row_base, int64_t n_rows, bool long_rows,
                               hipStream_t st);
// Scores of the listed rows (fp32, -inf past the row's visible blocks), [n_rows, ld].
hipError_t launch_score_rows(const int32_t *cu_q, const int32_t *cu_k, int batch,
                             const int64_t *rows, int64_t n_rows, const uint16_t *q_idx,
                             const float *w, const uint16_t *k_blk, float *scores, int64_t ld,
                             hipStream_t st);
hipError_t launch_score_local(const DecodeTables &d, int64_t n_tiles, int topk,
                              const uint16_t *q_idx, const float *w, const uint16_t *k_idx,
                              uint16_t *k_blk, uint32_t *keys, uint32_t *cand_key,
                              int32_t *cand_idx, int ch, int max_chunks, int32_t *sel,
                              uint32_t *ctl, hipStream_t st);
// Selection of the decode rows whose tile's chunks fit one merge (the scoring kernel
// leaves them to this launch: one workgroup per row).
hipError_t launch_merge_dec(const DecodeTables &d, int64_t n_rows, int topk,
                            const uint16_t *q_idx, const float *w, uint16_t *k_blk,
                            uint32_t *keys, uint32_t *cand_key, int32_t *cand_idx, int ch,
                            int max_chunks, int32_t *sel, hipStream_t st);
// Selection of rows [row_base, row_base + n_rows) (decode tables: rows 0..n_rows-1)
// from their score keys (slot s at keys[s - slot_base]).
hipError_t launch_select(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         const uint32_t *keys, int64_t slot_base, const uint32_t *cand_key,
                         const int32_t *cand_idx, int ch, int max_chunks, int32_t *sel,
                         int64_t row_base, int64_t n_rows, int dense_only, hipStream_t st);
// Decode rows whose tile's chunks fit one merge, merged by the attention workgroups
// themselves (each workgroup of a row merges its candidates into LDS first).
struct AttnMerge {
    const uint16_t *q_idx;
    const float *w;
    uint16_t *k_blk;
    uint32_t *keys, *cand_key;
    int32_t *cand_idx;
    int ch, max_chunks;
    int32_t *sel;   // where the merged selections are written out (the one attend reads)
};
// skip_dense (prefill, nsplit 1): rows with at most topk visible blocks are left to
// launch_attend_dense. row0: the launch attends rows row0 .. row0 + n_rows - 1 (nonzero
// only for prefill launches with one split per row).
hipError_t launch_attend(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         float scale, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const Fp8Kv *fp8, const int32_t *sel, float *out, float *lse,
                         float *part, int nsplit, int64_t n_rows, const AttnMerge *merge,
                         bool skip_dense, hipStream_t st, int64_t row0 = 0);
// Causal attention of the rows in the dense regime (every visible block kept), in tiles
// of DN_ROWS rows sharing their keys through LDS (qsa_dense.hip). sel not null: the
// kernel also writes these rows' selections (calls without scored rows).
hipError_t launch_attend_dense(const SeqInfo *tab, int batch, int topk, float scale,
                               const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               float *out, float *lse, int32_t *sel, int64_t n_tiles,
                               hipStream_t st);
// Attention backward over fixed selections (qsa_backward.hip).
struct BwdSeq;
struct BwdBuffers {
    BwdSeq *seq;      // [batch]
    float *delta;     // [Tq, 24]
    int32_t *nsel;    // [Tq]
    int32_t *off;     // [nkb_total + 1]
    int32_t *tot;     // [nkb_total]
    int32_t *mat;     // count matrices of all sequences
    int32_t *list;    // block -> rows lists
};
// side (not null): dQ runs on it, forked from st after the block -> rows index is built and
// joined back into st by the two events, while st runs the dK/dV launches.
hipError_t launch_backward(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_q_host,
                           const int32_t *cu_k_host, int batch, int topk,
                           float scale, int64_t n_rows, int64_t n_chunks, int64_t nkb_total,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *sel, const float *out, const float *lse,
                           const uint16_t *dout, float *dq, float *dk, float *dv,
                           const BwdBuffers &b, hipStream_t st,
                           hipStream_t side = nullptr, hipEvent_t fork = nullptr,
                           hipEvent_t join = nullptr);
// Clears n 32-bit words with a kernel.
hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t st);
hipError_t launch_quantize_kv(const uint16_t *k, const uint16_t *v, uint8_t *k8, uint8_t *v8,
                              float *k_scale, float *v_scale, int64_t rows, hipStream_t st);

}  // namespace qsa
