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

// Chunk lists one decode merge takes (longer rows merge groups of chunks first).
constexpr int MERGE_CHUNKS = 64;

// Optional per-kernel event trace (thread-local; see qsa_trace_begin).
void trace_before(int kind, hipStream_t st);
hipError_t trace_after(hipStream_t st, hipError_t launch_status);

hipError_t launch_prep(const int32_t *cu_q, const int32_t *cu_k, int batch, int topk,
                       SeqInfo *tab, hipStream_t st);
hipError_t launch_compress(const int32_t *cu_q, const int32_t *cu_k, int batch,
                           int64_t max_blocks, const uint16_t *k_idx, uint16_t *k_blk,
                           int incremental, SeqInfo *tab, int topk, hipStream_t st);
hipError_t launch_score(const SeqInfo *tab, int batch, int topk, const uint16_t *q_idx,
                        const float *w, const uint16_t *k_blk, uint32_t *keys,
                        int64_t n_tiles, int64_t max_blocks, int64_t chunk_blocks,
                        hipStream_t st);
hipError_t launch_score_local(const DecodeTables &d, int64_t n_tiles, int topk,
                              const uint16_t *q_idx, const float *w, const uint16_t *k_idx,
                              uint16_t *k_blk, uint32_t *keys, uint32_t *cand_key,
                              int32_t *cand_idx, int ch, int max_chunks, int32_t *sel,
                              uint32_t *glist_key, int32_t *glist_idx, uint32_t *ctl,
                              hipStream_t st);
// Selection of the decode rows whose tile's chunks fit one merge (the scoring kernel
// leaves them to this launch: one workgroup per row).
hipError_t launch_merge_dec(const DecodeTables &d, int64_t n_rows, int topk,
                            const uint16_t *q_idx, const float *w, uint16_t *k_blk,
                            uint32_t *keys, uint32_t *cand_key, int32_t *cand_idx, int ch,
                            int max_chunks, int32_t *sel, hipStream_t st);
hipError_t launch_select(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         const uint32_t *keys, const uint32_t *cand_key, const int32_t *cand_idx,
                         int ch, int max_chunks, int32_t *sel, int64_t n_rows, int64_t max_nvis,
                         int dense_only, hipStream_t st);
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
hipError_t launch_attend(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         float scale, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const Fp8Kv *fp8, const int32_t *sel, float *out, float *lse,
                         float *part, int nsplit, int64_t n_rows, const AttnMerge *merge,
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
hipError_t launch_backward(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_q_host,
                           const int32_t *cu_k_host, int batch, int topk,
                           float scale, int64_t n_rows, int64_t n_chunks, int64_t nkb_total,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *sel, const float *out, const float *lse,
                           const uint16_t *dout, float *dq, float *dk, float *dv,
                           const BwdBuffers &b, hipStream_t st);
hipError_t launch_quantize_kv(const uint16_t *k, const uint16_t *v, uint8_t *k8, uint8_t *v8,
                              float *k_scale, float *v_scale, int64_t rows, hipStream_t st);

}  // namespace qsa
