// qsa_kernels.hip -- gfx950 kernels of the QSA hot path:
//   prep / compress   per-sequence bookkeeping; micro-block key compression (HBM stream)
//   score             indexer scores of whole rows, 4 query rows per tile (prefill)
//   score_local       indexer scores of one block chunk + the chunk's exact local
//                     top-KP candidates (decode: few rows, long contexts)
//   select            exact top-k per row: from a chunk-candidate union when valid,
//                     else from the full row (radix select, LDS histograms)
//   attend            sparse GQA attention over gathered micro-blocks (MFMA, online
//                     softmax), split over keys when rows are few
//   combine           log-sum-exp merge of the key splits
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// =============================================================== prep
// Per-sequence table: first compressed block, first score tile and first score slot.
// Score rows are the positions t >= max(L-nq, 4*topk+3) (more visible blocks than the
// budget); they are tiled 4 rows at a time.
template <int NT>
__device__ void prep_body(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                          int batch, int topk, SeqInfo *__restrict__ tab, int64_t *sh) {
    int64_t carry_blk = 0, carry_tile = 0, carry_slot = 0;
    for (int base = 0; base < batch; base += NT) {
        const int b = base + threadIdx.x;
        int32_t q0 = 0, nq = 0, k0 = 0, L = 0;
        int64_t nblk = 0, ntile = 0, nslot = 0;
        if (b < batch) {
            q0 = cu_q[b]; nq = cu_q[b + 1] - q0;
            k0 = cu_k[b]; L = cu_k[b + 1] - k0;
            nblk = L / BS;
            const int64_t ts = first_scored_pos(L, nq, topk);
            if (ts < L) {
                ntile = (L - ts + 3) / 4;
                nslot = slots_before(L) - slots_before(ts);
            }
        }
        int64_t tot_b, tot_t, tot_s;
        const int64_t eb = block_excl_scan<int64_t, NT>(nblk, sh, &tot_b);
        const int64_t et = block_excl_scan<int64_t, NT>(ntile, sh, &tot_t);
        const int64_t es = block_excl_scan<int64_t, NT>(nslot, sh, &tot_s);
        if (b < batch) {
            SeqInfo s;
            s.q0 = q0; s.nq = nq; s.k0 = k0; s.L = L;
            s.blk0 = (int32_t)(carry_blk + eb);
            s.tile0 = (int32_t)(carry_tile + et);
            s.s0 = carry_slot + es;
            tab[b] = s;
        }
        carry_blk += tot_b; carry_tile += tot_t; carry_slot += tot_s;
    }
}

constexpr int PREP_NT = 256;

__global__ void __launch_bounds__(PREP_NT)
prep_kernel(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int batch,
            int topk, SeqInfo *__restrict__ tab) {
    __shared__ int64_t sh[PREP_NT / WAVE + 1];
    prep_body<PREP_NT>(cu_q, cu_k, batch, topk, tab, sh);
}

// =============================================================== compress
// Sum of the 4 indexer keys of each micro-block, exactly (double), rounded once to
// bf16. Thread = (block, 8 consecutive dims): 4 x 16-byte reads, one 16-byte write,
// so a wave streams 8 whole blocks (4 KiB in, 1 KiB out) with full coalescing.
// Grid: x = block group, y = sequence. When `tab` is given, the workgroup at
// (gridDim.x - 1, 0) also builds the per-sequence table (fused prep).
constexpr int CMP_NT = 256;
constexpr int CMP_BLOCKS_PER_WG = CMP_NT / 8;

// Dims 8c .. 8c+7 of block `blk` of the sequence starting at key row k0 and block row
// blk0: exact (double) sum of the 4 token keys, rounded once to bf16.
__device__ __forceinline__ void compress_one(const uint16_t *__restrict__ k_idx,
                                             uint16_t *__restrict__ k_blk, int64_t k0,
                                             int64_t blk0, int64_t blk, int c) {
    const uint16_t *src = k_idx + (k0 + blk * BS) * DI + c * 8;
    const u32x4 r0 = load16(src), r1 = load16(src + DI), r2 = load16(src + 2 * DI),
                r3 = load16(src + 3 * DI);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const double s_lo = (((double)bf16_lo(r0[q]) + (double)bf16_lo(r1[q])) +
                             (double)bf16_lo(r2[q])) + (double)bf16_lo(r3[q]);
        const double s_hi = (((double)bf16_hi(r0[q]) + (double)bf16_hi(r1[q])) +
                             (double)bf16_hi(r2[q])) + (double)bf16_hi(r3[q]);
        out[q] = f64_to_bf16_rne(s_lo) | (f64_to_bf16_rne(s_hi) << 16);
    }
    *reinterpret_cast<u32x4 *>(k_blk + (blk0 + blk) * DI + c * 8) = out;
}

__global__ void __launch_bounds__(CMP_NT)
compress_kernel(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                const uint16_t *__restrict__ k_idx, uint16_t *__restrict__ k_blk,
                int incremental, SeqInfo *__restrict__ tab, int batch, int topk) {
    __shared__ int64_t red[CMP_NT / WAVE + 1];
    if (tab && blockIdx.x == gridDim.x - 1) {
        if (blockIdx.y == 0) prep_body<CMP_NT>(cu_q, cu_k, batch, topk, tab, red);
        return;
    }
    const int b = blockIdx.y;
    const int32_t k0 = cu_k[b], L = cu_k[b + 1] - k0;
    const int64_t nblk = L / BS;
    int64_t lo = 0;
    if (incremental) {
        const int32_t nq = cu_q[b + 1] - cu_q[b];
        lo = (int64_t)(L - nq) / BS;
    }
    const int64_t first = lo + (int64_t)blockIdx.x * CMP_BLOCKS_PER_WG;
    if (first >= nblk) return;  // whole workgroup idle

    // first block row of this sequence: sum of floor(L_i/4) over earlier sequences
    int64_t part = 0;
    for (int i = threadIdx.x; i < b; i += CMP_NT) part += (cu_k[i + 1] - cu_k[i]) / BS;
    int64_t blk0;
    (void)block_excl_scan<int64_t, CMP_NT>(part, red, &blk0);

    const int64_t blk = first + threadIdx.x / 8;
    if (blk >= nblk) return;
    compress_one(k_idx, k_blk, k0, blk0, blk, threadIdx.x % 8);
}

// =============================================================== scoring core
// Tile = up to 4 consecutive query rows of one sequence. MFMA rows = (row, indexer
// head) pairs (16 = 4 x 4), columns = 16 blocks, K = 64 indexer dims in two
// 16x16x32 bf16 steps. The contraction order of the dims is permuted so each lane
// reads 16 contiguous bytes of a block key per step (A and B share the permutation):
// step m, lane group g holds dims 32m + 8g .. 32m + 8g + 7. Output lane (g, c) holds
// the 4 head dot products of row g and block c; the score sum_h w_h relu(dot_h) is
// formed in-lane and turned into an order key.
struct TileInfo {
    SeqInfo s;
    int64_t ts, t0, row0, nv_max;
    int nrows;
};

__device__ __forceinline__ TileInfo tile_info(const SeqInfo *tab, int batch, int topk,
                                              int64_t tile) {
    TileInfo ti;
    const int sb = find_seq(batch, tile, [&](int i) { return (int64_t)tab[i].tile0; });
    ti.s = tab[sb];
    ti.ts = first_scored_pos(ti.s.L, ti.s.nq, topk);
    ti.t0 = ti.ts + 4 * (tile - ti.s.tile0);
    ti.nrows = (int)min<int64_t>(4, ti.s.L - ti.t0);
    ti.row0 = ti.s.q0 + (ti.t0 - (ti.s.L - ti.s.nq));
    ti.nv_max = nvis_of(ti.t0 + ti.nrows - 1);
    return ti;
}

// RowView of query row r from the per-sequence table.
__device__ __forceinline__ RowView tab_row(const SeqInfo *tab, int batch, int topk, int64_t r) {
    const int sb = find_seq(batch, r, [&](int i) { return (int64_t)tab[i].q0; });
    const SeqInfo s = tab[sb];
    RowView v;
    v.k0 = s.k0;
    v.t = (int64_t)s.L - s.nq + (r - s.q0);
    v.blk0 = s.blk0;
    v.slot = s.s0 + slots_before(v.t) - slots_before(first_scored_pos(s.L, s.nq, topk));
    return v;
}

struct ScoreLane {
    u32x4 qa[2];
    float wr[HI];
    int64_t slot, nv_row;
};

// Operands of a tile of nrows query rows starting at row0 (position t0); slot_g is
// the first score slot of this lane's output row (row0 + lane/16), if it exists.
__device__ __forceinline__ ScoreLane score_lane_setup(const uint16_t *__restrict__ q_idx,
                                                      const float *__restrict__ w,
                                                      int64_t row0, int nrows, int64_t t0,
                                                      int64_t slot_g) {
    ScoreLane sl;
    const int l = lane_id(), g = l >> 4, c = l & 15;
    const int rr = c >> 2, hh = c & 3;
#pragma unroll
    for (int m = 0; m < 2; ++m)
        sl.qa[m] = load16(q_idx + ((row0 + min(rr, nrows - 1)) * HI + hh) * DI + 32 * m + 8 * g);
    if (rr >= nrows) sl.qa[0] = sl.qa[1] = u32x4{0u, 0u, 0u, 0u};
    const int gg = min(g, nrows - 1);
#pragma unroll
    for (int h = 0; h < HI; ++h) sl.wr[h] = g < nrows ? w[(row0 + gg) * HI + h] : 0.f;
    sl.slot = g < nrows ? slot_g : 0;
    sl.nv_row = g < nrows ? nvis_of(t0 + g) : 0;
    return sl;
}

// Keys of NB groups of 16 consecutive blocks starting at b0, b0 + step, ...; all
// loads are issued before the first MFMA (loads past hi are clamped to block hi-1).
template <int NB>
__device__ __forceinline__ void score_groups(const ScoreLane &sl, const uint16_t *kb,
                                             int64_t b0, int64_t step, int64_t hi,
                                             uint32_t (&key)[NB]) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    u32x4 b[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int64_t blk = b0 + u * step + c;
        const uint16_t *src = kb + (blk < hi ? blk : hi - 1) * DI + 8 * g;
        b[u][0] = load16(src);
        b[u][1] = load16(src + 32);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the MFMAs
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_bf16_16x16x32(sl.qa[0], b[u][0], acc);
        acc = mfma_bf16_16x16x32(sl.qa[1], b[u][1], acc);
        float sc = sl.wr[0] * fmaxf(acc[0], 0.f);
        sc += sl.wr[1] * fmaxf(acc[1], 0.f);
        sc += sl.wr[2] * fmaxf(acc[2], 0.f);
        sc += sl.wr[3] * fmaxf(acc[3], 0.f);
        key[u] = score_key(sc);
    }
}

constexpr int SCORE_BATCH = 8;  // 16-block groups per wave in flight

// score_groups with whole-block loads: each load instruction reads 8 complete 128-byte
// blocks (lane 8j + q: the 16-byte chunk q of block j), the access the address units
// coalesce, and each group's chunks reach the MFMA operand layout (lane (g, c): chunks
// g and 4 + g of block c) through one of the wave's two LDS tiles (16 blocks, 144-byte
// pitch: the 16 blocks' rows start on distinct 4-bank groups), used in turn.
constexpr int SC_PITCH = 144;
constexpr int SC_TILE = 16 * SC_PITCH;
template <int NB>
__device__ __forceinline__ void score_groups_lds(const ScoreLane &sl, const uint16_t *kb,
                                                 int64_t b0, int64_t step, int64_t hi,
                                                 uint32_t (&key)[NB], uint8_t *tiles) {
    const int l = lane_id(), g = l >> 4, c = l & 15, bj = l >> 3, q = l & 7;
    u32x4 b[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t blk = b0 + u * step + 8 * h + bj;
            b[u][h] = load16(kb + (blk < hi ? blk : hi - 1) * DI + 8 * q);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the batch ahead of the MFMAs
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        uint8_t *t = tiles + (u & 1) * SC_TILE;
        wave_lds_sync();   // this tile's reads of two groups ago are done
        *reinterpret_cast<u32x4 *>(t + bj * SC_PITCH + 16 * q) = b[u][0];
        *reinterpret_cast<u32x4 *>(t + (8 + bj) * SC_PITCH + 16 * q) = b[u][1];
        wave_lds_sync();
        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(t + c * SC_PITCH + 16 * g);
        const u32x4 x1 = *reinterpret_cast<const u32x4 *>(t + c * SC_PITCH + 64 + 16 * g);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_bf16_16x16x32(sl.qa[0], x0, acc);
        acc = mfma_bf16_16x16x32(sl.qa[1], x1, acc);
        float sc = sl.wr[0] * fmaxf(acc[0], 0.f);
        sc += sl.wr[1] * fmaxf(acc[1], 0.f);
        sc += sl.wr[2] * fmaxf(acc[2], 0.f);
        sc += sl.wr[3] * fmaxf(acc[3], 0.f);
        key[u] = score_key(sc);
    }
}

constexpr int SCORE_NT = 256;

// Whole rows: grid x = tile, y = chunk of `chunk_blocks` blocks.
__global__ void __launch_bounds__(SCORE_NT) __attribute__((amdgpu_waves_per_eu(4, 8)))
score_kernel(const SeqInfo *__restrict__ tab, int batch, int topk,
             const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
             const uint16_t *__restrict__ k_blk, uint32_t *__restrict__ keys,
             int64_t chunk_blocks) {
    const TileInfo ti = tile_info(tab, batch, topk, blockIdx.x);
    const int64_t lo = (int64_t)blockIdx.y * chunk_blocks;
    const int64_t hi = min<int64_t>(ti.nv_max, lo + chunk_blocks);
    if (lo >= hi) return;
    const int g = lane_id() >> 4;
    const ScoreLane sl = score_lane_setup(
        q_idx, w, ti.row0, ti.nrows, ti.t0,
        ti.s.s0 + slots_before(ti.t0 + g) - slots_before(ti.ts));
    const uint16_t *kb = k_blk + (int64_t)ti.s.blk0 * DI;
    const int c = lane_id() & 15;
    __shared__ __attribute__((aligned(16))) uint8_t tiles[SCORE_NT / WAVE][2 * SC_TILE];
    constexpr int64_t step = 16 * (SCORE_NT / WAVE);
    for (int64_t b0 = lo + 16 * (threadIdx.x / WAVE); b0 < hi; b0 += step * SCORE_BATCH) {
        uint32_t key[SCORE_BATCH];
        score_groups_lds<SCORE_BATCH>(sl, kb, b0, step, hi, key, tiles[threadIdx.x / WAVE]);
#pragma unroll
        for (int u = 0; u < SCORE_BATCH; ++u) {
            const int64_t blk = b0 + u * step + c;
            if (blk < hi && blk < sl.nv_row) keys[sl.slot + blk] = key[u];
        }
    }
}

// =============================================================== score_local + select
// Decode-shaped launches: grid x = chunk of CH blocks, y = tile, so workgroups are
// dispatched (and their loads largely served) row by row. Each workgroup scores its
// chunk for the tile's rows and, for each row whose selection can come from chunk
// candidates, writes the chunk's KP best (key, block) pairs in ascending block order to
// cand[row][chunk][0..KP), padded with key 0 (below every real key). The local top-KP
// is exact and needs no workgroup-wide histogram: each wave takes the top KP of its 256
// positions with a wave-private radix select, and one wave takes the top KP of those
// 4 x KP (tiles of several rows: one wave per row over the whole chunk). Rows whose
// tile has at most MERGE_CHUNKS chunks are then merged after this kernel: in a forward
// step by the decode attention's workgroups, after a selection alone by merge_dec_kernel
// (one workgroup per row). Longer rows merge groups of chunks inside this kernel: candidates
// are written through to the coherence point, and the workgroup that completes a group
// (then the tile) behind an arrival counter in the control block (reset by that
// workgroup) merges it.
constexpr int LOC_NT = 256;
constexpr int LOC_MAX_CH = 1024;
constexpr int KP = 32;
constexpr int SEL_NT = 256;

// A row may be selected from chunk candidates when its full chunks alone provide at
// least topk candidates (so the union always holds topk real keys).
__device__ __forceinline__ bool cand_eligible(int64_t nv, int topk, int ch) {
    return nv > topk && (nv / ch) * KP >= topk;
}

struct SelectArgs {
    const SeqInfo *tab;
    int batch, topk;
    const uint32_t *keys;
    const uint32_t *cand_key;
    const int32_t *cand_idx;
    int ch, max_chunks;  // ch = 0: no candidates
    int32_t *sel;
    int dense_only;      // only rows with at most topk visible blocks
};

// Top-k of the n keys at `kk` (global memory): their positions, ascending, to out.
// hist: LDS, kHistBins entries (the radix histogram, then the emit pass's counts).
template <int PER, typename KP_T>
__device__ __forceinline__ void select_keys(KP_T kk, int64_t n, int topk, int32_t *out,
                                            uint32_t *hist, int32_t *scan_sh, uint32_t *found) {
    uint32_t theta;
    int64_t need;
    radix_kth<SEL_NT>(kk, n, topk, kWide, hist, scan_sh, found, &theta, &need);
    static_assert(4 * (SEL_NT / WAVE) * PER <= kHistBins, "emit counts fit the histogram");
    emit_kept<SEL_NT, PER>(kk, n, theta, need, out, topk, reinterpret_cast<int32_t *>(hist));
}

// Level-one merges take at most MERGE_CHUNKS chunk lists (KP candidates each; the
// constant is shared with the host, qsa_launch.h); rows with more chunks first merge
// G = ceil(nch / MERGE_CHUNKS) groups of ceil(nch / G) consecutive chunks (balanced,
// so every group holds more than MERGE_CHUNKS / 2 chunk
// lists: at least topk real candidates), then the group lists (topk entries each) of
// at most MAX_GROUPS groups.
constexpr int MAX_GROUPS = 4;

// Top-k of the n <= 2048 candidates (key, id) at ck[0..n) / ci[0..n) (written by other
// workgroups of this kernel: agent-scope loads); key 0 marks padding, which is never
// kept because every caller has at least k real candidates. Kept ids go out in
// position order: to out_idx with plain stores, or (WT_OUT) with their keys through to
// the coherence point, padded with key 0 / id -1 up to k. When nv > 0 the positions are
// the KP-entry lists of chunks c0, c0+1, ... of a row with nv visible blocks: returns
// false if a chunk holding more than KP of the row's blocks had all KP candidates kept
// (only such a chunk can hide a better block, so only then can the result be inexact).
template <bool WT_OUT>
__device__ __forceinline__ bool merge_candidates(const uint32_t *ck, const int32_t *ci, int n,
                                                 int k, int32_t *out_idx, uint32_t *out_key,
                                                 int64_t nv, int ch, int c0, int *viol,
                                                 TopkSmem *tsm) {
    const int tid = threadIdx.x;
    uint32_t x[8];
    int32_t id[8];
    u32x4 kq[2], iq[2];
    const bool have = 8 * tid < n;
#pragma unroll
    for (int v4 = 0; v4 < 2; ++v4) {
        kq[v4] = have ? load16_wt(ck + 8 * tid + 4 * v4) : u32x4{0u, 0u, 0u, 0u};
        iq[v4] = have ? load16_wt(ci + 8 * tid + 4 * v4) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int v4 = 0; v4 < 2; ++v4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[4 * v4 + e] = kq[v4][e];
            id[4 * v4 + e] = (int32_t)iq[v4][e];
        }
    }
    if (tid == 0) *viol = 0;
    uint32_t kept;
    int first;
    const int tot = block_topk_regs<SEL_NT, 8>(x, n, k, *tsm, &kept, &first);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (kept & (1u << e)) {
            if (first < k) {
                if (WT_OUT) {
                    store_wt(out_key + first, x[e]);
                    store_wt(out_idx + first, id[e]);
                } else {
                    out_idx[first] = id[e];
                }
            }
            ++first;
        }
    }
    if (WT_OUT) {
        for (int i = tot + tid; i < k; i += SEL_NT) {
            store_wt(out_key + i, 0u);
            store_wt(out_idx + i, -1);
        }
    }
    if (nv > 0) {
        int kc = __popc(kept);
        kc += __shfl_xor(kc, 1);
        kc += __shfl_xor(kc, 2);
        static_assert(KP == 32, "4 threads hold one chunk list");
        const int c = c0 + tid / 4;
        const int64_t nc = have ? min<int64_t>(ch, nv - (int64_t)c * ch) : 0;
        if (nc > KP && kc >= KP) *viol = 1;
    }
    __syncthreads();
    return !*viol;
}

// One workgroup selects one query row from its full key row: rows within the budget
// keep blocks 0..nvis-1, others get an exact radix select over the keys in global memory
// (each pass re-reads them from L2; staging up to 64 KB of keys per row in LDS held
// occupancy to two workgroups per CU and was a third slower).
__device__ __forceinline__ void select_body(const SelectArgs &a, const RowView rv, int64_t row,
                                            uint32_t *hist, int32_t *scan_sh, uint32_t *found) {
    const int64_t nv = nvis_of(rv.t);
    int32_t *out = a.sel + row * a.topk;
    const int tid = threadIdx.x;
    if (nv <= a.topk) {
        for (int i = tid; i < a.topk; i += SEL_NT) out[i] = i < nv ? i : -1;
        return;
    }
    if (a.dense_only) return;
    select_keys<16>(a.keys + rv.slot, nv, a.topk, out, hist, scan_sh, found);
}

struct LocalArgs {
    int topk;
    const uint16_t *q_idx;
    const float *w;
    const uint16_t *k_idx;   // not null: compress each tile's new blocks first
    uint16_t *k_blk;
    uint32_t *keys;          // full key rows, written only when a row needs the exact path
    uint32_t *cand_key;
    int32_t *cand_idx;
    int ch, max_chunks;
    int32_t *sel;
    uint32_t *glist_key;     // [row][MAX_GROUPS][topk] group merge results
    int32_t *glist_idx;
    uint32_t *ctl;           // arrival counters and flags (zero between calls)
};

// Scores blocks [lo, hi) of a tile; store(row, blk, key) is called for each block
// the lane's row sees.
template <typename Store>
__device__ __forceinline__ void score_range(const ScoreLane &sl, const uint16_t *kb, int64_t lo,
                                            int64_t hi, Store store) {
    const int g = lane_id() >> 4, c = lane_id() & 15;
    constexpr int64_t step = 16 * (LOC_NT / WAVE);
    for (int64_t b0 = lo + 16 * (threadIdx.x / WAVE); b0 < hi; b0 += step * SCORE_BATCH) {
        uint32_t key[SCORE_BATCH];
        score_groups<SCORE_BATCH>(sl, kb, b0, step, hi, key);
#pragma unroll
        for (int u = 0; u < SCORE_BATCH; ++u) {
            const int64_t blk = b0 + u * step + c;
            if (blk < hi && blk < sl.nv_row) store(g, blk, key[u]);
        }
    }
}

// Exact selection of the rows of a tile flagged in exact[] from key rows this
// workgroup recomputes itself (after recompressing the tile's new blocks, so that it
// reads only its own writes).
__device__ __forceinline__ void select_tile_exact(const LocalArgs &a, const DecodeTables &d,
                                                  int tile, const int *exact, uint32_t *hist,
                                                  int32_t *scan_sh, uint32_t *found) {
    const DecTile tl = d.tile[tile];
    const int64_t row0 = tl.row0;
    const int nrows = tl.nrows;
    const int64_t t0 = d.row[row0].t;
    const DecRow r0 = d.row[row0];
    if (a.k_idx && tl.new_hi > tl.new_lo) {
        for (int64_t blk = tl.new_lo + threadIdx.x / 8; blk < tl.new_hi; blk += LOC_NT / 8)
            compress_one(a.k_idx, a.k_blk, r0.k0, r0.blk0, blk, threadIdx.x % 8);
        wait_vmem();
        __syncthreads();
    }
    const int g = lane_id() >> 4;
    const ScoreLane sl = score_lane_setup(a.q_idx, a.w, row0, nrows, t0,
                                          d.row[row0 + min(g, nrows - 1)].slot);
    uint32_t *keys = a.keys;
    const int64_t slot = sl.slot;
    score_range(sl, a.k_blk + (int64_t)r0.blk0 * DI, 0, nvis_of(t0 + nrows - 1),
                [=](int, int64_t blk, uint32_t key) { keys[slot + blk] = key; });
    wait_vmem();
    __syncthreads();
    for (int rr = 0; rr < nrows; ++rr) {
        if (!exact[rr]) continue;   // uniform (LDS)
        const DecRow r = d.row[row0 + rr];
        select_keys<16>((const uint32_t *)(a.keys + r.slot), nvis_of(r.t), a.topk,
                        a.sel + (row0 + rr) * a.topk, hist, scan_sh, found);
    }
}

// LDS of one scoring workgroup.
struct ScoreSmem {
    uint32_t whist[LOC_NT / WAVE][256];   // per-wave histograms (and key transposes)
    uint32_t wl_key[LOC_NT / WAVE][KP];
    int32_t wl_pos[LOC_NT / WAVE][KP];
    uint32_t hist[kHistBins];
    int32_t scan_sh[SEL_NT / WAVE];
    uint32_t found[2];
    int viol, s_last, exact[4];
    TopkSmem tsm;
    __attribute__((aligned(16))) uint8_t tiles[LOC_NT / WAVE][2 * SC_TILE];  // score_groups_lds
};

// One scoring workgroup: chunk `chunk` of tile `tile`. Returns true in the workgroup
// that completed the tile (after it has selected the tile's rows).
__device__ __forceinline__ bool score_chunk(const LocalArgs &a, const DecodeTables &d, int tile,
                                            int chunk, ScoreSmem &sm) {
    const DecTile tl = d.tile[tile];
    const int64_t row0 = tl.row0;
    const int nrows = tl.nrows;
    const int64_t t0 = d.row[row0].t;
    const int64_t nv_max = nvis_of(t0 + nrows - 1);
    const int64_t lo = (int64_t)chunk * a.ch;
    const int64_t hi = min<int64_t>(nv_max, lo + a.ch);
    if (lo >= hi) return false;
    const int l = lane_id(), g = l >> 4, c = l & 15, w = threadIdx.x / WAVE;
    // blocks of this sequence that hold a query token are (re)compressed here first,
    // by every workgroup whose chunk contains them (identical values)
    if (a.k_idx && tl.new_hi > tl.new_lo) {
        const int64_t c_lo = max<int64_t>(lo, tl.new_lo), c_hi = min<int64_t>(hi, tl.new_hi);
        const int64_t blk = c_lo + threadIdx.x / 8;
        if (blk < c_hi)
            compress_one(a.k_idx, a.k_blk, d.row[row0].k0, d.row[row0].blk0, blk,
                         threadIdx.x % 8);
        __threadfence_block();
        __syncthreads();
    }
    const ScoreLane sl = score_lane_setup(a.q_idx, a.w, row0, nrows, t0,
                                          d.row[row0 + min(g, nrows - 1)].slot);
    const uint16_t *kb = a.k_blk + (int64_t)d.row[row0].blk0 * DI;

    // wave w scores the contiguous blocks wlo + 16u + c (u < 16) of its quarter of the
    // chunk; the keys stay in registers (two batches of 8 groups of 16 blocks)
    const int span = a.ch / 4;
    const int64_t wlo = lo + (int64_t)w * span;
    const int64_t whi = min<int64_t>(hi, wlo + span);
    uint32_t key[2 * SCORE_BATCH];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t kk[SCORE_BATCH];
        if (wlo + 16 * SCORE_BATCH * h < whi) {
            score_groups_lds<SCORE_BATCH>(sl, kb, wlo + 16 * SCORE_BATCH * h, 16, whi, kk,
                                          sm.tiles[w]);
        } else {
#pragma unroll
            for (int u = 0; u < SCORE_BATCH; ++u) kk[u] = 0u;
        }
#pragma unroll
        for (int u = 0; u < SCORE_BATCH; ++u) key[SCORE_BATCH * h + u] = kk[u];
    }

    // each tile row whose selection can come from chunk candidates gets this chunk's
    // KP best (key, block) pairs, in ascending block order, padded with key 0. One row:
    // the top KP of each wave's blocks, then the top KP of those 4 x KP. Several rows: the
    // rows' keys go through LDS (the scoring tiles are free by then) and wave w takes the
    // top KP of row w over the whole chunk, all rows at once. (The rows' merges below stay
    // one after another in the whole workgroup: one wave per row was not faster.)
    const bool par_local = nrows > 1;
    if (par_local) {
        uint32_t *rk = reinterpret_cast<uint32_t *>(&sm.tiles[0][0]);   // [row][1024 entries]
        static_assert(sizeof(sm.tiles) >= 4 * 4 * 256 * sizeof(uint32_t), "row keys fit");
        __syncthreads();   // every wave is done with its scoring tiles
#pragma unroll
        for (int u = 0; u < 2 * SCORE_BATCH; ++u) rk[g * 1024 + w * 256 + 16 * u + c] = key[u];
        __syncthreads();
        const int rr = w;
        if (rr < nrows && cand_eligible(nvis_of(t0 + rr), a.topk, a.ch)) {   // uniform per wave
            // lane l: entries 16l .. 16l+15 = wave quarter l/16, blocks 16(l%16) + i of it
            const int64_t vhi = min<int64_t>(hi, nvis_of(t0 + rr));
            const int qw = l >> 4, u0 = 16 * (l & 15);
            uint32_t x[16];
            bool ok[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u32x4 v4 = *reinterpret_cast<const u32x4 *>(rk + rr * 1024 + 16 * l + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * q4 + e] = v4[e];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                ok[i] = u0 + i < span && lo + (int64_t)qw * span + u0 + i < vhi;
            const uint32_t mask = wave_topk_hist<16>(x, ok, KP, sm.whist[w]);
            const int cnt = __popc(mask);
            const int incl = wave_incl_scan_i32(cnt);
            const int tot = __builtin_amdgcn_readlane(incl, WAVE - 1);
            int pos = incl - cnt;
            uint32_t *ck = a.cand_key + ((row0 + rr) * a.max_chunks + chunk) * KP;
            int32_t *ci = a.cand_idx + ((row0 + rr) * a.max_chunks + chunk) * KP;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (mask & (1u << i)) {
                    store_wt(ck + pos, x[i]);
                    store_wt(ci + pos, (int32_t)(lo + (int64_t)qw * span + u0 + i));
                    ++pos;
                }
            }
            if (l >= tot && l < KP) {
                store_wt(ck + l, 0u);
                store_wt(ci + l, -1);
            }
        }
    }
    uint32_t *wk = sm.whist[w];
    for (int rr = 0; !par_local && rr < nrows; ++rr) {
        const int64_t nv = nvis_of(t0 + rr);
        if (!cand_eligible(nv, a.topk, a.ch)) continue;   // uniform over the workgroup
        // the row's keys, position 16u + c, move to lanes as positions 4l .. 4l+3
        if (g == rr) {
#pragma unroll
            for (int u = 0; u < 2 * SCORE_BATCH; ++u) wk[16 * u + c] = key[u];
        }
        wave_lds_sync();
        const u32x4 q4 = *reinterpret_cast<const u32x4 *>(&wk[4 * l]);
        uint32_t x[4];
        bool ok[4];
        const int64_t nvw = min<int64_t>(whi, nv);
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[e] = q4[e]; ok[e] = wlo + 4 * l + e < nvw; }
        wave_lds_sync();   // the histogram below reuses wk
        const uint32_t mask = wave_topk_hist<4>(x, ok, KP, wk);
        const int cnt = __popc(mask);
        int pos = wave_excl_small<4>(cnt);
        const int tot = __builtin_amdgcn_readlane(pos + cnt, WAVE - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (mask & (1u << e)) {
                sm.wl_key[w][pos] = x[e];
                sm.wl_pos[w][pos] = (int32_t)(wlo + 4 * l + e - lo);
                ++pos;
            }
        }
        if (l >= tot && l < KP) sm.wl_key[w][l] = 0u;
        lds_barrier();
        if (w == 0) {
            // entries 2l, 2l+1 of the 4 x KP wave lists (ascending position order)
            uint32_t y[2];
            bool oy[2];
            int py[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * l + e;
                y[e] = sm.wl_key[i / KP][i % KP];
                py[e] = sm.wl_pos[i / KP][i % KP];
                oy[e] = y[e] != 0u;
            }
            const uint32_t m2 = wave_topk_hist<2>(y, oy, KP, sm.whist[0]);
            const int c2 = __popc(m2);
            int o = wave_excl_small<2>(c2);
            const int tot2 = __builtin_amdgcn_readlane(o + c2, WAVE - 1);
            uint32_t *ck = a.cand_key + ((row0 + rr) * a.max_chunks + chunk) * KP;
            int32_t *ci = a.cand_idx + ((row0 + rr) * a.max_chunks + chunk) * KP;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (m2 & (1u << e)) {
                    store_wt(ck + o, y[e]);
                    store_wt(ci + o, (int32_t)(lo + py[e]));
                    ++o;
                }
            }
            if (l >= tot2 && l < KP) {
                store_wt(ck + l, 0u);
                store_wt(ci + l, -1);
            }
        }
        if (rr + 1 < nrows) lds_barrier();   // wave lists are reused by the next row
    }

    // hand over: the workgroup that completes the tile's last chunk merges the rows'
    // candidates; rows with more than MERGE_CHUNKS chunks merge groups of chunks first
    // (the last chunk of each group), then the group lists (the tile's last group)
    wait_vmem();
    __syncthreads();
    const int tid = threadIdx.x;
    const int nch = (int)((nv_max + a.ch - 1) / a.ch);
    const int ngroups = (nch + MERGE_CHUNKS - 1) / MERGE_CHUNKS;
    const int gsize = (nch + ngroups - 1) / ngroups;   // chunks per group (balanced)
    // groups of chunks are merged separately when there are 2 .. MAX_GROUPS of them
    const bool grouped = ngroups > 1 && ngroups <= MAX_GROUPS;
    // rows whose chunks fit one merge are merged by merge_dec_kernel, one workgroup per
    // row: the rows (of all tiles) merge at the same time, and this kernel ends with its
    // last chunk instead of with a merge behind an arrival counter
    if (ngroups == 1) return false;
    if (grouped) {
        const int grp = chunk / gsize;
        const int n_in = min(gsize, nch - grp * gsize);
        if (tid == 0) {
            uint32_t *cnt = &a.ctl[CTL_GROUP + tile * MAX_GROUPS + grp];
            const uint32_t old = atomicAdd(cnt, 1u);
            sm.s_last = old + 1 == (uint32_t)n_in;
            if (sm.s_last) store_wt(cnt, 0u);
        }
        __syncthreads();
        if (!sm.s_last) return false;
        for (int rr = 0; rr < nrows; ++rr) {
            const int64_t nv = nvis_of(t0 + rr), row = row0 + rr;
            if (!cand_eligible(nv, a.topk, a.ch)) continue;   // uniform
            const int64_t cbase = (row * a.max_chunks + grp * gsize) * KP;
            const int64_t gbase = (row * MAX_GROUPS + grp) * a.topk;
            const bool ok = merge_candidates<true>(
                a.cand_key + cbase, a.cand_idx + cbase, n_in * KP, a.topk, a.glist_idx + gbase,
                a.glist_key + gbase, nv, a.ch, grp * gsize, &sm.viol, &sm.tsm);
            if (!ok && tid == 0) store_wt(&a.ctl[CTL_EXACT + row], 1u);
        }
        wait_vmem();
        __syncthreads();
    }
    // the tile counter counts merged groups, or chunks when no grouping is used
    if (tid == 0) {
        const uint32_t old = atomicAdd(&a.ctl[CTL_TILE + tile], 1u);
        sm.s_last = old + 1 == (uint32_t)(grouped ? ngroups : nch);
        if (sm.s_last) store_wt(&a.ctl[CTL_TILE + tile], 0u);
    }
    __syncthreads();
    if (!sm.s_last) return false;

    // this workgroup selects the tile's rows
    int n_exact = 0;
    for (int rr = 0; rr < nrows; ++rr) {
        const int64_t nv = nvis_of(t0 + rr), row = row0 + rr;
        bool done = false;
        if (cand_eligible(nv, a.topk, a.ch) && ngroups <= MAX_GROUPS) {
            if (grouped) {
                if (tid == 0) {
                    sm.exact[rr] = load_wt(&a.ctl[CTL_EXACT + row]) != 0u;
                    store_wt(&a.ctl[CTL_EXACT + row], 0u);
                }
                __syncthreads();
                if (!sm.exact[rr]) {
                    const int64_t gbase = row * MAX_GROUPS * a.topk;
                    done = merge_candidates<false>(a.glist_key + gbase, a.glist_idx + gbase,
                                                   ngroups * a.topk, a.topk, a.sel + row * a.topk,
                                                   nullptr, 0, a.ch, 0, &sm.viol, &sm.tsm);
                }
            } else {
                const int64_t cbase = row * a.max_chunks * KP;
                const int nch_row = (int)((nv + a.ch - 1) / a.ch);
                done = merge_candidates<false>(a.cand_key + cbase, a.cand_idx + cbase,
                                               nch_row * KP, a.topk, a.sel + row * a.topk,
                                               nullptr, nv, a.ch, 0, &sm.viol, &sm.tsm);
            }
        }
        __syncthreads();
        if (tid == 0) sm.exact[rr] = !done;
        n_exact += !done;   // uniform
    }
    __syncthreads();
    if (n_exact > 0) select_tile_exact(a, d, tile, sm.exact, sm.hist, sm.scan_sh, sm.found);
    return true;
}

// Exact selection of one decode row from its full key row, which this workgroup scores
// itself into the row's slots of `keys` (the blocks its tile's tokens complete were
// compressed by the scoring kernel, which has finished).
__device__ __forceinline__ void select_row_exact(const LocalArgs &a, const DecodeTables &d,
                                                 int64_t row, int32_t *out, uint32_t *hist,
                                                 int32_t *scan_sh, uint32_t *found) {
    const DecRow r = d.row[row];
    const ScoreLane sl = score_lane_setup(a.q_idx, a.w, row, 1, r.t, r.slot);
    uint32_t *keys = a.keys;
    const int64_t slot = sl.slot;
    score_range(sl, a.k_blk + (int64_t)r.blk0 * DI, 0, nvis_of(r.t),
                [=](int, int64_t blk, uint32_t key) { keys[slot + blk] = key; });
    wait_vmem();
    __syncthreads();
    select_keys<16>((const uint32_t *)(a.keys + r.slot), nvis_of(r.t), a.topk, out, hist,
                    scan_sh, found);
}

// The rows that are merged from chunk candidates outside the scoring kernel: those whose
// tile has at most MERGE_CHUNKS chunks.
__device__ __forceinline__ bool merged_after_scoring(const DecodeTables &d, const DecRow &r,
                                                     int ch) {
    if (r.tile < 0) return false;
    const DecTile tl = d.tile[r.tile];
    const int64_t nv_max = nvis_of((int64_t)d.row[tl.row0].t + tl.nrows - 1);
    return (nv_max + ch - 1) / ch <= MERGE_CHUNKS;
}

// One workgroup per decode row: rows whose tile's chunks fit one merge get their top-k
// from the chunk candidates the scoring kernel wrote (or exactly, when a chunk may hide
// a better block or the row has too few chunks for candidates).
__global__ void __launch_bounds__(LOC_NT) merge_dec_kernel(LocalArgs a, DecodeTables d) {
    __shared__ ScoreSmem sm;
    const int64_t row = blockIdx.x;
    const DecRow r = d.row[row];
    if (!merged_after_scoring(d, r, a.ch)) return;   // groups of chunks: scoring kernel
    const int64_t nv = nvis_of(r.t);
    bool done = false;
    if (cand_eligible(nv, a.topk, a.ch)) {
        const int64_t cbase = row * a.max_chunks * KP;
        const int nch_row = (int)((nv + a.ch - 1) / a.ch);
        done = merge_candidates<false>(a.cand_key + cbase, a.cand_idx + cbase, nch_row * KP,
                                       a.topk, a.sel + row * a.topk, nullptr, nv, a.ch, 0,
                                       &sm.viol, &sm.tsm);
    }
    if (!done)   // uniform
        select_row_exact(a, d, row, a.sel + row * a.topk, sm.hist, sm.scan_sh, sm.found);
}

// 4 waves per SIMD: the whole decode grid (rows x chunks) is resident at once
__global__ void __launch_bounds__(LOC_NT) __attribute__((amdgpu_waves_per_eu(4, 8)))
score_local_kernel(LocalArgs a, DecodeTables d) {
    __shared__ ScoreSmem sm;
    (void)score_chunk(a, d, blockIdx.y, blockIdx.x, sm);
}

__global__ void __launch_bounds__(SEL_NT)
select_kernel(SelectArgs a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ int32_t scan_sh[SEL_NT / WAVE];
    __shared__ uint32_t found[2];
    const int64_t row = blockIdx.x;
    select_body(a, tab_row(a.tab, a.batch, a.topk, row), row, hist, scan_sh, found);
}

__global__ void __launch_bounds__(SEL_NT)
select_dec_kernel(SelectArgs a, DecodeTables d) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ int32_t scan_sh[SEL_NT / WAVE];
    __shared__ uint32_t found[2];
    const int64_t row = blockIdx.x;
    const DecRow r = d.row[row];
    const RowView rv = {r.k0, r.t, r.blk0, r.slot};
    select_body(a, rv, row, hist, scan_sh, found);
}

// =============================================================== attend
// One wave per (query row, key/value head g, key split). The row's keys are the
// tokens of its kept blocks in ascending order, then its raw tail (one more block
// slot with 0..3 valid tokens). A wave walks them 32 at a time:
//   S^T[32 keys x 16 heads] = K (A operand, 2 x 16 keys) * Q^T (B operand, the 12 live
//   heads of group g): 4 MFMA 16x16x32 steps per 16 keys over the 128 dims, the dims
//   permuted so each lane reads 16 contiguous bytes (step m, group gr holds dims
//   32m + 8gr .. +7).
//   Online softmax per head in base 2; each lane owns one head (its column).
//   O^T[128 dims x 16 heads] += V^T * P^T: P^T is the lane's own 8 probabilities (keys
//   4gr..4gr+3 and 16+4gr..16+4gr+3, the k-slots of its lane group), split into bf16
//   hi + lo parts (2 MFMAs) to keep ~16 bits; V^T rows are permuted so row r of
//   dim-tile mt is dim 8r + mt, which lets each lane load 16 contiguous bytes of V per
//   key.
// K and V are loaded as whole rows (16 lanes per 256-byte row, the access the address
// units coalesce); K then passes through a per-wave LDS tile into the MFMA layout.
// Block ids of the row are held in registers (lane i: slot 64j + i) and broadcast with
// shuffles, and each tile's K/V loads are issued one tile ahead of its MFMAs.
// nsplit = 1: final output. nsplit > 1: unnormalised partial (acc, m, l) per split.
constexpr int ATT_NT = 256;
constexpr int PREC = HD + 4;  // partial record per (row, split, head): acc[128], m, l, pad

struct AttnArgs {
    const SeqInfo *tab;
    int batch;
    int topk;
    float scale_log2;  // softmax scale * log2(e)
    const uint16_t *q, *k, *v;
    const uint8_t *k8, *v8;      // FP8 KV cache (E4M3 bytes) and its per-row scales
    const float *k_scale, *v_scale;
    const int32_t *sel;
    float *out, *lse;
    float *part;
    int nsplit;
    int64_t nrows;
    int merge;        // decode: merge the rows of short tiles here (operands in `loc`)
    LocalArgs loc;
};

__device__ __forceinline__ int64_t part_stride_row(int nsplit) {
    return (int64_t)nsplit * HQ * PREC;
}

// K and V rows of the lane's 8 P keys (keys 4gr..4gr+3 and 16+4gr..16+4gr+3 of the tile),
// dims 8col .. 8col+7: each load instruction reads whole 256-byte rows, one per 16 lanes.
struct KVTile {
    u32x4 kt[8];
    u32x4 vr[8];
    uint32_t valid;  // bit 4u+i: key j0 + 16u + 4gr + i is attended
};
// The same tile from the FP8 KV cache: 8 E4M3 bytes per load, and the K and V scales
// of the lane's 8 P keys (the logit and probability of key e are scaled by them).
struct KVTile8 {
    uint2 kt[8];
    uint2 vr[8];
    float ks[8], vs[8];
    uint32_t valid;
};
// LDS row pitch (bytes) of the per-wave K tile that turns the row-per-16-lanes loads into
// the MFMA operand layout (16 bytes of padding spread the rows over the banks)
template <bool FP8> constexpr int kt_pitch() { return FP8 ? HD + 16 : 2 * HD + 16; }
constexpr int KT_LDS_BYTES = 32 * (2 * HD + 16);   // one wave's tile (the larger, bf16)

template <bool FP8>
__device__ __forceinline__ void attend_body(const AttnArgs &a, const RowView rv, int64_t row,
                                            int g, int sp, uint8_t *klds,
                                            const int32_t *srow) {
    using Tile = typename std::conditional<FP8, KVTile8, KVTile>::type;
    const int64_t t = rv.t;
    const int64_t nv = nvis_of(t);
    const int ntail = (int)(t + 1 - BS * nv);
    const int l = lane_id(), gr = l >> 4, col = l & 15;

    // number of leading selected entries: 8 unconditional loads in flight, then ballots
    int nsel = a.topk;
    int32_t v[KMAX / WAVE];
#pragma unroll
    for (int j = 0; j < KMAX / WAVE; ++j) v[j] = srow[min(64 * j + l, a.topk - 1)];
#pragma unroll
    for (int j = KMAX / WAVE - 1; j >= 0; --j) {
        const unsigned long long bal = __ballot(64 * j + l < a.topk && v[j] < 0);
        if (bal) nsel = 64 * j + __builtin_ctzll(bal);
    }
    const int nslot = nsel + (ntail > 0 ? 1 : 0);
    const int npos = 4 * nslot;
    int chunk = (npos + a.nsplit - 1) / a.nsplit;
    chunk = (chunk + 31) & ~31;
    const int p_lo = sp * chunk;
    const int p_hi = min(npos, p_lo + chunk);

    const int head = g * GQ + col;
    u32x4 qb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        qb[m] = col < GQ ? load16(a.q + (row * HQ + head) * HD + 32 * m + 8 * gr)
                         : u32x4{0u, 0u, 0u, 0u};

    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t kv0 = rv.k0;
    const int64_t safe_tok = kv0 + t;  // always a valid key row
    const uint16_t *kbase = a.k + g * HD;
    const uint16_t *vbase = a.v + g * HD;

    // first token of slot sl (block ids of the current 64-slot group held in `cur`)
    auto slot_token0 = [&](int sl, int32_t cur, bool &ok) -> int64_t {
        const int32_t bid = __shfl(cur, sl & 63);
        if (sl < nsel) {
            ok = bid >= 0 && bid < nv;
            return kv0 + (int64_t)BS * bid;
        }
        ok = sl == nsel && ntail > 0;
        return kv0 + (int64_t)BS * nv;
    };
    auto load_tile = [&](int j0, int32_t cur) -> Tile {
        Tile T;
        T.valid = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int sl = (j0 >> 2) + 4 * h + gr;
            bool okb;
            const int64_t tok0 = slot_token0(sl, cur, okb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 4 * sl + i;
                const bool ok = okb && p < p_hi && (sl < nsel || i < ntail);
                const int64_t tok = ok ? tok0 + i : safe_tok;
                if constexpr (FP8) {
                    T.kt[4 * h + i] = *reinterpret_cast<const uint2 *>(
                        a.k8 + tok * (HKV * HD) + g * HD + 8 * col);
                    T.vr[4 * h + i] = *reinterpret_cast<const uint2 *>(
                        a.v8 + tok * (HKV * HD) + g * HD + 8 * col);
                    T.ks[4 * h + i] = a.k_scale[tok * HKV + g];
                    T.vs[4 * h + i] = a.v_scale[tok * HKV + g];
                } else {
                    T.kt[4 * h + i] = load16(kbase + tok * (HKV * HD) + 8 * col);
                    T.vr[4 * h + i] = load16(vbase + tok * (HKV * HD) + 8 * col);
                }
                if (ok) T.valid |= 1u << (4 * h + i);
            }
        }
        return T;
    };
    // block ids of slots 64*grp .. 64*grp+63 (lane i: slot 64*grp + i), L2-resident
    auto group_ids = [=](int grp) -> int32_t { return srow[min(64 * grp + l, a.topk - 1)]; };

    int cur_grp = p_lo >> 8;  // 64 slots = 256 key positions per group
    int32_t cur = v[0];
#pragma unroll
    for (int j = 1; j < KMAX / WAVE; ++j)
        if (cur_grp == j) cur = v[j];
    Tile nxt;
    if (p_lo < p_hi) nxt = load_tile(p_lo, cur);
    for (int j0 = p_lo; j0 < p_hi; j0 += 32) {
        const Tile T = nxt;
        const int jn = j0 + 32;
        if (jn < p_hi) {
            if ((jn >> 8) != cur_grp) { cur_grp = jn >> 8; cur = group_ids(cur_grp); }
            nxt = load_tile(jn, cur);
        }
        // ---- logits S^T for keys j0 .. j0+31 (lane: keys j0+16u+4gr+i, head col)
        float z[8];
        float mx = -INFINITY;
        // the K rows go through this wave's LDS tile into the MFMA A layout (lane: key
        // 16u + col, dims 32m + 8gr)
        constexpr int KP = kt_pitch<FP8>();
        constexpr int EB = FP8 ? 1 : 2;   // bytes per element
        wave_lds_sync();   // the previous tile's reads are done
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint8_t *dst = klds + (16 * (e >> 2) + 4 * gr + (e & 3)) * KP + 8 * EB * col;
            if constexpr (FP8) *reinterpret_cast<uint2 *>(dst) = T.kt[e];
            else *reinterpret_cast<u32x4 *>(dst) = T.kt[e];
        }
        wave_lds_sync();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint8_t *src = klds + (16 * u + col) * KP + (32 * m + 8 * gr) * EB;
                if constexpr (FP8)
                    c4 = mfma_bf16_16x16x32(e4m3x8_to_bf16x8(*reinterpret_cast<const uint2 *>(src)),
                                            qb[m], c4);
                else c4 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4 *>(src), qb[m], c4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = (T.valid >> (4 * u + i)) & 1u;
                float zz = c4[i] * a.scale_log2;
                if constexpr (FP8) zz *= T.ks[4 * u + i];
                z[4 * u + i] = ok ? zz : -INFINITY;
                mx = fmaxf(mx, z[4 * u + i]);
            }
        }
        mx = wave_max_xor_16_32(mx);
        if (mx == -INFINITY) continue;  // no attended key in the tile (uniform over the wave)
        // the softmax reference m_run (with acc and l_run) moves only when some head's
        // tile maximum exceeds it by more than 2^8, so most tiles skip rescaling the
        // accumulators; every probability exp2(z - m_run) stays at most 2^8
        if (__ballot(mx > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) acc[mt] *= alpha;
            m_run = m_new;
        }
        float p[8], rs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = z[e] == -INFINITY ? 0.f : exp2f(z[e] - m_run);
            rs += p[e];
        }
        l_run += wave_sum_xor_16_32(rs);

        // FP8: the V scale of each key multiplies its probability (the denominator l
        // keeps the unscaled ones)
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (FP8) pv[e] = p[e] * T.vs[e];
            else pv[e] = p[e];
        }
        u32x4 ph, pl;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            const uint32_t h0 = f32_to_bf16_rne(pv[2 * q2]), h1 = f32_to_bf16_rne(pv[2 * q2 + 1]);
            const float r0 = pv[2 * q2] - __uint_as_float(h0 << 16);
            const float r1 = pv[2 * q2 + 1] - __uint_as_float(h1 << 16);
            ph[q2] = h0 | (h1 << 16);
            pl[q2] = f32_to_bf16_rne(r0) | (f32_to_bf16_rne(r1) << 16);
        }
        u32x4 vb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (FP8) vb[e] = e4m3x8_to_bf16x8(T.vr[e]);
            else vb[e] = T.vr[e];
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int q2 = mt >> 1;
            u32x4 va;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t x0 = vb[2 * kk][q2], x1 = vb[2 * kk + 1][q2];
                va[kk] = bf16_pair(x0, x1, mt & 1);
            }
            acc[mt] = mfma_bf16_16x16x32(va, ph, acc[mt]);
            acc[mt] = mfma_bf16_16x16x32(va, pl, acc[mt]);
        }
    }

    // lane (gr, col): acc[mt][i] = O[head col][dim 8*(4gr+i) + mt]
    if (col >= GQ) return;
    if (a.nsplit == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *o = a.out + (row * HQ + head) * HD;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 8 * (4 * gr + i);
            const f32x4 lo4 = {acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv};
            const f32x4 hi4 = {acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv, acc[7][i] * inv};
            *reinterpret_cast<f32x4 *>(o + d0) = lo4;
            *reinterpret_cast<f32x4 *>(o + d0 + 4) = hi4;
        }
        if (a.lse && gr == 0)
            a.lse[row * HQ + head] = l_run > 0.f ? m_run * 0.69314718055994531f + logf(l_run)
                                                 : -INFINITY;
    } else {
        float *pp = a.part + row * part_stride_row(a.nsplit) + ((int64_t)sp * HQ + head) * PREC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 8 * (4 * gr + i);
            const f32x4 lo4 = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
            const f32x4 hi4 = {acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
            *reinterpret_cast<f32x4 *>(pp + d0) = lo4;
            *reinterpret_cast<f32x4 *>(pp + d0 + 4) = hi4;
        }
        if (gr == 0) { pp[HD] = m_run; pp[HD + 1] = l_run; }
    }
}

// wave -> (row, kv head, split)
__device__ __forceinline__ bool attend_item(const AttnArgs &a, int64_t &row, int &g, int &sp) {
    const int64_t item = __builtin_amdgcn_readfirstlane(
        (int)((int64_t)blockIdx.x * (ATT_NT / WAVE) + threadIdx.x / WAVE));
    row = item / (HKV * a.nsplit);
    const int rem = (int)(item % (HKV * a.nsplit));
    g = rem / a.nsplit;
    sp = rem % a.nsplit;
    return row < a.nrows;
}

template <bool FP8>
__global__ void __launch_bounds__(ATT_NT)
attend_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t klds[(ATT_NT / WAVE) * KT_LDS_BYTES];
    int64_t row;
    int g, sp;
    if (!attend_item(a, row, g, sp)) return;
    attend_body<FP8>(a, tab_row(a.tab, a.batch, a.topk, row), row, g, sp,
                     klds + (threadIdx.x / WAVE) * KT_LDS_BYTES, a.sel + row * a.topk);
}

// LDS of a decode attention workgroup that merges its row's candidates.
struct AttnMergeSmem {
    TopkSmem tsm;
    int viol;
    uint32_t hist[kHistBins];   // exact fallback: radix histogram, then the emit counts
    int32_t scan_sh[SEL_NT / WAVE];
    uint32_t found[2];
    int32_t ids[KMAX];          // the row's kept block ids, ascending
};

template <bool FP8>
__global__ void __launch_bounds__(ATT_NT)
attend_dec_kernel(AttnArgs a, DecodeTables d) {
    int64_t row;
    int g, sp;
    if (!attend_item(a, row, g, sp)) return;
    __shared__ __attribute__((aligned(16))) uint8_t klds[(ATT_NT / WAVE) * KT_LDS_BYTES];
    __shared__ AttnMergeSmem ms;
    const DecRow r = d.row[row];
    const RowView rv = {r.k0, r.t, r.blk0, r.slot};
    const int32_t *srow = a.sel + row * a.topk;
    // rows merged from chunk candidates after scoring: every workgroup of the row (its
    // waves are splits of one row) merges them into LDS, the row's first workgroup also
    // writes the selection out
    if (a.merge && merged_after_scoring(d, r, a.loc.ch)) {   // uniform over the workgroup
        const int64_t nv = nvis_of(r.t);
        bool done = false;
        if (cand_eligible(nv, a.topk, a.loc.ch)) {
            const int64_t cbase = row * a.loc.max_chunks * KP;
            const int nch_row = (int)((nv + a.loc.ch - 1) / a.loc.ch);
            done = merge_candidates<false>(a.loc.cand_key + cbase, a.loc.cand_idx + cbase,
                                           nch_row * KP, a.topk, ms.ids, nullptr, nv,
                                           a.loc.ch, 0, &ms.viol, &ms.tsm);
        }
        if (!done)   // uniform
            select_row_exact(a.loc, d, row, ms.ids, ms.hist, ms.scan_sh, ms.found);
        __syncthreads();
        const int64_t item0 = (int64_t)blockIdx.x * (ATT_NT / WAVE);
        if (item0 % (HKV * a.nsplit) == 0)
            for (int i = threadIdx.x; i < a.topk; i += ATT_NT) a.loc.sel[row * a.topk + i] = ms.ids[i];
        srow = ms.ids;
    }
    attend_body<FP8>(a, rv, row, g, sp, klds + (threadIdx.x / WAVE) * KT_LDS_BYTES, srow);
}

// =============================================================== combine
// One wave per (row, head): lane s reads split s's (m, l); the merged output is the
// weighted sum of the split accumulators in split order (deterministic).
constexpr int CMB_NT = 256;

__global__ void __launch_bounds__(CMB_NT)
combine_kernel(const float *__restrict__ part, int nsplit, int64_t nrows,
               float *__restrict__ out, float *__restrict__ lse) {
    const int64_t item = (int64_t)blockIdx.x * (CMB_NT / WAVE) + threadIdx.x / WAVE;
    if (item >= nrows * HQ) return;
    const int64_t row = item / HQ;
    const int head = (int)(item % HQ);
    const int l = lane_id();
    const float *pr = part + row * part_stride_row(nsplit) + (int64_t)head * PREC;
    const int64_t sstride = (int64_t)HQ * PREC;
    const float ms = l < nsplit ? pr[l * sstride + HD] : -INFINITY;
    const float ls = l < nsplit ? pr[l * sstride + HD + 1] : 0.f;
    float M = ms;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) M = fmaxf(M, __shfl_xor(M, d));
    const float f = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
    float Lsum = ls * f;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) Lsum += __shfl_xor(Lsum, d);
    float o0 = 0.f, o1 = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 16) {
        float2 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = s0 + j < nsplit ? *reinterpret_cast<const float2 *>(pr + (s0 + j) * sstride + 2 * l)
                                   : float2{0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float fs = __shfl(f, (s0 + j) & 63);
            o0 += v[j].x * fs;
            o1 += v[j].y * fs;
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float *o = out + (row * HQ + head) * HD;
    o[2 * l] = o0 * inv;
    o[2 * l + 1] = o1 * inv;
    if (lse && l == 0)
        lse[row * HQ + head] = Lsum > 0.f ? M * 0.69314718055994531f + logf(Lsum) : -INFINITY;
}

// =============================================================== FP8 KV cache
// Row = (token, KV head) of K or V, 128 bf16 values: 16 lanes per row (8 values, one
// 16-byte load each), 16 rows per workgroup; grid y = 0 for K, 1 for V. The row's
// scale is amax / 448 (1 for an all-zero row) and each byte the E4M3 rounding of the
// fp32 quotient x / scale (IEEE divisions, as in the definition).
constexpr int QNT_NT = 256;

__global__ void __launch_bounds__(QNT_NT)
quantize_kv_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                   uint8_t *__restrict__ k8, uint8_t *__restrict__ v8,
                   float *__restrict__ k_scale, float *__restrict__ v_scale, int64_t rows) {
    const int64_t r = (int64_t)blockIdx.x * (QNT_NT / 16) + threadIdx.x / 16;
    if (r >= rows) return;   // whole 16-lane groups leave together
    const int c = threadIdx.x % 16;
    const uint16_t *src = blockIdx.y ? v : k;
    uint8_t *dst = blockIdx.y ? v8 : k8;
    float *sc = blockIdx.y ? v_scale : k_scale;
    const u32x4 x4 = load16(src + r * HD + 8 * c);
    float x[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        x[2 * q] = bf16_lo(x4[q]);
        x[2 * q + 1] = bf16_hi(x4[q]);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int dd = 1; dd < 16; dd <<= 1) amax = fmaxf(amax, __shfl_xor(amax, dd));
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) lo |= e4m3_rne(x[e] / s) << (8 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e) hi |= e4m3_rne(x[4 + e] / s) << (8 * e);
    *reinterpret_cast<uint2 *>(dst + r * HD + 8 * c) = uint2{lo, hi};
    if (c == 0) sc[r] = s;
}

hipError_t launch_quantize_kv(const uint16_t *k, const uint16_t *v, uint8_t *k8, uint8_t *v8,
                              float *k_scale, float *v_scale, int64_t rows, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int64_t gx = (rows + QNT_NT / 16 - 1) / (QNT_NT / 16);
    trace_before(1, st);
    hipLaunchKernelGGL(quantize_kv_kernel, dim3((unsigned)gx, 2), dim3(QNT_NT), 0, st, k, v, k8,
                       v8, k_scale, v_scale, rows);
    return trace_after(st, hipGetLastError());
}

// =============================================================== launchers

hipError_t launch_prep(const int32_t *cu_q, const int32_t *cu_k, int batch, int topk,
                       SeqInfo *tab, hipStream_t st) {
    trace_before(0, st);
    hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(PREP_NT), 0, st, cu_q, cu_k, batch, topk, tab);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_compress(const int32_t *cu_q, const int32_t *cu_k, int batch,
                           int64_t max_blocks, const uint16_t *k_idx, uint16_t *k_blk,
                           int incremental, SeqInfo *tab, int topk, hipStream_t st) {
    if (batch <= 0) return hipSuccess;
    int64_t gx = (max_blocks + CMP_BLOCKS_PER_WG - 1) / CMP_BLOCKS_PER_WG;
    if (tab) gx += 1;  // fused prep workgroup
    if (gx <= 0) return hipSuccess;
    trace_before(1, st);
    hipLaunchKernelGGL(compress_kernel, dim3((unsigned)gx, (unsigned)batch), dim3(CMP_NT), 0, st,
                       cu_q, cu_k, k_idx, k_blk, incremental, tab, batch, topk);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_score(const SeqInfo *tab, int batch, int topk, const uint16_t *q_idx,
                        const float *w, const uint16_t *k_blk, uint32_t *keys,
                        int64_t n_tiles, int64_t max_blocks, int64_t chunk_blocks,
                        hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    const int64_t gy = (max_blocks + chunk_blocks - 1) / chunk_blocks;
    trace_before(2, st);
    hipLaunchKernelGGL(score_kernel, dim3((unsigned)n_tiles, (unsigned)gy), dim3(SCORE_NT), 0, st,
                       tab, batch, topk, q_idx, w, k_blk, keys, chunk_blocks);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_score_local(const DecodeTables &d, int64_t n_tiles, int topk,
                              const uint16_t *q_idx, const float *w, const uint16_t *k_idx,
                              uint16_t *k_blk, uint32_t *keys, uint32_t *cand_key,
                              int32_t *cand_idx, int ch, int max_chunks, int32_t *sel,
                              uint32_t *glist_key, int32_t *glist_idx, uint32_t *ctl,
                              hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    LocalArgs a;
    a.topk = topk; a.q_idx = q_idx; a.w = w; a.k_idx = k_idx; a.k_blk = k_blk; a.keys = keys;
    a.cand_key = cand_key; a.cand_idx = cand_idx; a.ch = ch; a.max_chunks = max_chunks;
    a.sel = sel; a.glist_key = glist_key; a.glist_idx = glist_idx; a.ctl = ctl;
    trace_before(2, st);
    hipLaunchKernelGGL(score_local_kernel, dim3((unsigned)max_chunks, (unsigned)n_tiles),
                       dim3(LOC_NT), 0, st, a, d);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_merge_dec(const DecodeTables &d, int64_t n_rows, int topk,
                            const uint16_t *q_idx, const float *w, uint16_t *k_blk,
                            uint32_t *keys, uint32_t *cand_key, int32_t *cand_idx, int ch,
                            int max_chunks, int32_t *sel, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    LocalArgs a = {};
    a.topk = topk; a.q_idx = q_idx; a.w = w; a.k_idx = nullptr; a.k_blk = k_blk; a.keys = keys;
    a.cand_key = cand_key; a.cand_idx = cand_idx; a.ch = ch; a.max_chunks = max_chunks;
    a.sel = sel;
    trace_before(3, st);
    hipLaunchKernelGGL(merge_dec_kernel, dim3((unsigned)n_rows), dim3(LOC_NT), 0, st, a, d);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_select(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         const uint32_t *keys, const uint32_t *cand_key, const int32_t *cand_idx,
                         int ch, int max_chunks, int32_t *sel, int64_t n_rows, int64_t max_nvis,
                         int dense_only, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    SelectArgs a;
    a.tab = tab; a.batch = batch; a.topk = topk; a.keys = keys;
    a.cand_key = cand_key; a.cand_idx = cand_idx; a.ch = ch; a.max_chunks = max_chunks;
    a.sel = sel; a.dense_only = dense_only;
    (void)max_nvis;
    trace_before(3, st);
    if (d)
        hipLaunchKernelGGL(select_dec_kernel, dim3((unsigned)n_rows), dim3(SEL_NT), 0, st, a, *d);
    else
        hipLaunchKernelGGL(select_kernel, dim3((unsigned)n_rows), dim3(SEL_NT), 0, st, a);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_attend(const SeqInfo *tab, const DecodeTables *d, int batch, int topk,
                         float scale, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const Fp8Kv *fp8, const int32_t *sel, float *out, float *lse,
                         float *part, int nsplit, int64_t n_rows, const AttnMerge *merge,
                         hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    AttnArgs a = {};
    a.merge = merge != nullptr && d != nullptr;
    if (a.merge) {
        a.loc.topk = topk; a.loc.q_idx = merge->q_idx; a.loc.w = merge->w; a.loc.k_idx = nullptr;
        a.loc.k_blk = merge->k_blk; a.loc.keys = merge->keys; a.loc.cand_key = merge->cand_key;
        a.loc.cand_idx = merge->cand_idx; a.loc.ch = merge->ch; a.loc.max_chunks = merge->max_chunks;
        a.loc.sel = merge->sel;
    }
    a.tab = tab; a.batch = batch; a.topk = topk;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = q; a.k = k; a.v = v; a.sel = sel; a.out = out; a.lse = lse; a.part = part;
    a.k8 = fp8 ? fp8->k8 : nullptr; a.v8 = fp8 ? fp8->v8 : nullptr;
    a.k_scale = fp8 ? fp8->k_scale : nullptr; a.v_scale = fp8 ? fp8->v_scale : nullptr;
    a.nsplit = nsplit; a.nrows = n_rows;
    const int64_t waves = n_rows * HKV * nsplit;
    const int64_t wgs = (waves + ATT_NT / WAVE - 1) / (ATT_NT / WAVE);
    trace_before(4, st);
    if (d && fp8)
        hipLaunchKernelGGL(attend_dec_kernel<true>, dim3((unsigned)wgs), dim3(ATT_NT), 0, st, a,
                           *d);
    else if (d)
        hipLaunchKernelGGL(attend_dec_kernel<false>, dim3((unsigned)wgs), dim3(ATT_NT), 0, st, a,
                           *d);
    else if (fp8)
        hipLaunchKernelGGL(attend_kernel<true>, dim3((unsigned)wgs), dim3(ATT_NT), 0, st, a);
    else
        hipLaunchKernelGGL(attend_kernel<false>, dim3((unsigned)wgs), dim3(ATT_NT), 0, st, a);
    hipError_t e = trace_after(st, hipGetLastError());
    if (e != hipSuccess || nsplit == 1) return e;
    const int64_t cw = (n_rows * HQ + CMB_NT / WAVE - 1) / (CMB_NT / WAVE);
    trace_before(5, st);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)cw), dim3(CMB_NT), 0, st, part, nsplit,
                       n_rows, out, lse);
    return trace_after(st, hipGetLastError());
}

}  // namespace qsa
