// qsa_backward.hip -- gfx950 kernels of the attention backward over fixed selections.
// For the loss sum(dO * O) of the sparse GQA attention, with P the softmax of the
// scaled logits over a row's attended keys and D = rowsum(dO * O) per (row, head):
//   dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// dQ is formed row-major (each row reads its own keys); dK and dV key-major (each key
// block reads the rows that attend it), so no gradient is ever accumulated with
// atomics and the results do not depend on scheduling. The kernels:
//   bwd_prep     per-sequence table (key blocks, row chunks, count-matrix offsets)
//   bwd_rows     per row: leading selected entries (nsel) and D for its 24 heads
//   bwd_count    per (row chunk, key block): rows of the chunk that attend the block
//   bwd_colscan  per key block: exclusive prefix of its counts over the chunks, total
//   bwd_scan     exclusive prefix of the block totals -> list offsets
//   bwd_fill     the block -> rows lists, rows ascending within each list
//   bwd_dq       dQ (one wave per (row, KV head)), MFMA
//   bwd_dkv      dK, dV (one wave per (key block, KV head)) over the block's rows
// A row attends key block b when b is among its valid selected entries, or when b is
// its raw tail (b = nvis(t) with tokens 4b..t); either way exactly its keys at
// positions <= t, so the list entries need no kind flag.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// =============================================================== bwd_prep
constexpr int BPREP_NT = 256;

__global__ void __launch_bounds__(BPREP_NT)
bwd_prep_kernel(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int batch,
                BwdSeq *__restrict__ tab) {
    __shared__ int64_t sh[BPREP_NT / WAVE + 1];
    int64_t carry_kb = 0, carry_ch = 0, carry_m = 0;
    for (int base = 0; base < batch; base += BPREP_NT) {
        const int b = base + threadIdx.x;
        int32_t q0 = 0, nq = 0, k0 = 0, L = 0;
        int64_t nkb = 0, nch = 0;
        if (b < batch) {
            q0 = cu_q[b]; nq = cu_q[b + 1] - q0;
            k0 = cu_k[b]; L = cu_k[b + 1] - k0;
            nkb = (L + BS - 1) / BS;
            nch = (nq + BWD_CH - 1) / BWD_CH;
        }
        int64_t tkb, tch, tm;
        const int64_t ekb = block_excl_scan<int64_t, BPREP_NT>(nkb, sh, &tkb);
        const int64_t ech = block_excl_scan<int64_t, BPREP_NT>(nch, sh, &tch);
        const int64_t em = block_excl_scan<int64_t, BPREP_NT>(nkb * nch, sh, &tm);
        if (b < batch) {
            BwdSeq s;
            s.q0 = q0; s.nq = nq; s.k0 = k0; s.L = L;
            s.kb0 = (int32_t)(carry_kb + ekb);
            s.nkb = (int32_t)nkb;
            s.ch0 = (int32_t)(carry_ch + ech);
            s.nch = (int32_t)nch;
            s.m0 = carry_m + em;
            tab[b] = s;
        }
        carry_kb += tkb; carry_ch += tch; carry_m += tm;
    }
}

// =============================================================== bwd_rows
// One wave per query row. nsel = index of the first -1 of the row's selection (the
// attention reads entries up to it). D[h] = sum_d dO[h][d] * O[h][d]: lane (hg, c)
// takes dims 8c..8c+7 of heads hg, hg+4, ..., hg+20 and 16 lanes reduce each head.
constexpr int BROWS_NT = 256;

__global__ void __launch_bounds__(BROWS_NT)
bwd_rows_kernel(const int32_t *__restrict__ sel, int topk, const uint16_t *__restrict__ dout,
                const float *__restrict__ out, int64_t nrows, int32_t *__restrict__ nsel_out,
                float *__restrict__ delta) {
    const int64_t row = (int64_t)blockIdx.x * (BROWS_NT / WAVE) + threadIdx.x / WAVE;
    if (row >= nrows) return;
    const int l = lane_id();
    const int32_t *srow = sel + row * topk;
    int32_t v[KMAX / WAVE];
#pragma unroll
    for (int j = 0; j < KMAX / WAVE; ++j) v[j] = srow[min(64 * j + l, topk - 1)];
    int nsel = topk;
#pragma unroll
    for (int j = KMAX / WAVE - 1; j >= 0; --j) {
        const unsigned long long bal = __ballot(64 * j + l < topk && v[j] < 0);
        if (bal) nsel = 64 * j + __builtin_ctzll(bal);
    }
    if (l == 0) nsel_out[row] = nsel;

    const int c = l & 15, hg = l >> 4;
    float part[HQ / 4];
#pragma unroll
    for (int i = 0; i < HQ / 4; ++i) {
        const int h = hg + 4 * i;
        const u32x4 d8 = load16(dout + (row * HQ + h) * HD + 8 * c);
        const f32x4 o0 = *reinterpret_cast<const f32x4 *>(out + (row * HQ + h) * HD + 8 * c);
        const f32x4 o1 = *reinterpret_cast<const f32x4 *>(out + (row * HQ + h) * HD + 8 * c + 4);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            s += bf16_lo(d8[e]) * o0[2 * e] + bf16_hi(d8[e]) * o0[2 * e + 1];
            s += bf16_lo(d8[2 + e]) * o1[2 * e] + bf16_hi(d8[2 + e]) * o1[2 * e + 1];
        }
        part[i] = s;
    }
#pragma unroll
    for (int i = 0; i < HQ / 4; ++i) {
        float s = part[i];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (c == 0) delta[row * HQ + hg + 4 * i] = s;
    }
}

// =============================================================== block -> rows index
// Count matrix of sequence s: [nch][nkb] int32 at m0 (chunk-major). After bwd_colscan
// entry (c, b) holds the number of rows of chunks before c that attend block b, so the
// rows of chunk c go to list positions off[kb0 + b] + entry (c, b) onwards, in row
// order. List positions are int32 (the host bounds the total by Tq * (topk + 1)).
constexpr int BIDX_NT = 256;

struct ChunkView {
    BwdSeq s;
    int64_t row0;   // first row of the chunk
    int nrows;
    int64_t tbase;  // t = tbase + row
};

__device__ __forceinline__ ChunkView chunk_view(const BwdSeq *tab, int batch, int64_t chunk) {
    const int sb = find_seq(batch, chunk, [&](int i) { return (int64_t)tab[i].ch0; });
    ChunkView v;
    v.s = tab[sb];
    const int64_t k = chunk - v.s.ch0;
    v.row0 = v.s.q0 + k * BWD_CH;
    v.nrows = (int)min<int64_t>(BWD_CH, (int64_t)v.s.q0 + v.s.nq - v.row0);
    v.tbase = (int64_t)v.s.L - v.s.nq - v.s.q0;
    return v;
}

// Attended key block of entry i of a row (i == topk: the raw tail), or -1.
__device__ __forceinline__ int32_t entry_block(int32_t bid, int i, int nsel, int topk,
                                               int64_t nv, int ntail) {
    if (i < nsel) return (bid >= 0 && bid < nv) ? bid : -1;
    if (i == topk && ntail > 0) return (int32_t)nv;
    return -1;
}

__global__ void __launch_bounds__(BIDX_NT)
bwd_count_kernel(const BwdSeq *__restrict__ tab, int batch, const int32_t *__restrict__ sel,
                 int topk, const int32_t *__restrict__ nsel_of, int32_t *__restrict__ mat) {
    __shared__ int32_t cnt[BWD_CAP];
    const ChunkView cv = chunk_view(tab, batch, blockIdx.x);
    const int l = lane_id(), w = threadIdx.x / WAVE;
    int32_t *mrow = mat + cv.s.m0 + (int64_t)(blockIdx.x - cv.s.ch0) * cv.s.nkb;
    for (int r0 = 0; r0 < cv.s.nkb; r0 += BWD_CAP) {
        const int nr = min(BWD_CAP, cv.s.nkb - r0);
        for (int i = threadIdx.x; i < nr; i += BIDX_NT) cnt[i] = 0;
        __syncthreads();
        for (int j = w; j < cv.nrows; j += BIDX_NT / WAVE) {
            const int64_t row = cv.row0 + j;
            const int64_t t = cv.tbase + row;
            const int64_t nv = nvis_of(t);
            const int ntail = (int)(t + 1 - BS * nv);
            const int ns = nsel_of[row];
            const int32_t *srow = sel + row * topk;
            // entries 0 .. topk (index topk: the raw tail)
            int32_t bv[KMAX / WAVE + 1];
#pragma unroll
            for (int k = 0; k <= KMAX / WAVE; ++k) {
                const int i = 64 * k + l;
                bv[k] = i < ns ? srow[i] : -1;
            }
#pragma unroll
            for (int k = 0; k <= KMAX / WAVE; ++k) {
                const int i = 64 * k + l;
                const int32_t b = entry_block(bv[k], i, ns, topk, nv, ntail);
                if (b >= r0 && b < r0 + nr) atomicAdd(&cnt[b - r0], 1);
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nr; i += BIDX_NT) mrow[r0 + i] = cnt[i];
        __syncthreads();
    }
}

constexpr int BCOL_NT = 256;

__global__ void __launch_bounds__(BCOL_NT)
bwd_colscan_kernel(const BwdSeq *__restrict__ tab, int batch, int64_t nkb_total,
                   int32_t *__restrict__ mat, int32_t *__restrict__ tot) {
    const int64_t gb = (int64_t)blockIdx.x * BCOL_NT + threadIdx.x;
    if (gb >= nkb_total) return;
    const int sb = upper_index(batch, gb, [&](int i) { return (int64_t)tab[i].kb0; });
    const BwdSeq s = tab[sb];
    int32_t *col = mat + s.m0 + (gb - s.kb0);
    const int64_t stride = s.nkb;
    int32_t run = 0;
    int c = 0;
    for (; c + 8 <= s.nch; c += 8) {
        int32_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = col[(int64_t)(c + j) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) { col[(int64_t)(c + j) * stride] = run; run += x[j]; }
    }
    for (; c < s.nch; ++c) {
        const int32_t x = col[(int64_t)c * stride];
        col[(int64_t)c * stride] = run;
        run += x;
    }
    tot[gb] = run;
}

constexpr int BSCAN_NT = 1024;

// One workgroup: off[i] = sum_{j<i} tot[j] for i <= n, 4 consecutive entries a thread.
__global__ void __launch_bounds__(BSCAN_NT)
bwd_scan_kernel(const int32_t *__restrict__ tot, int64_t n, int32_t *__restrict__ off) {
    __shared__ int32_t scratch[BSCAN_NT / WAVE];
    int32_t carry = 0;
    for (int64_t base = 0; base < n; base += 4 * BSCAN_NT) {
        const int64_t i0 = base + 4 * threadIdx.x;
        int32_t x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = i0 + j < n ? tot[i0 + j] : 0;
        const int32_t sum = x[0] + x[1] + x[2] + x[3];
        int32_t total;
        int32_t run = carry + block_excl_scan_i32<BSCAN_NT>(sum, scratch, &total);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j < n) off[i0 + j] = run;
            run += x[j];
        }
        carry += total;
    }
    if (threadIdx.x == 0) off[n] = carry;
}

// Rows of the chunk one at a time (entries spread over the workgroup, a barrier between
// rows), so each list receives its rows in ascending order. Within a row the attended
// blocks are distinct unless the selection repeats a block; repeated entries write the
// same row, so the list contents do not depend on which lane wins.
__global__ void __launch_bounds__(BIDX_NT)
bwd_fill_kernel(const BwdSeq *__restrict__ tab, int batch, const int32_t *__restrict__ sel,
                int topk, const int32_t *__restrict__ nsel_of, const int32_t *__restrict__ mat,
                const int32_t *__restrict__ off, int32_t *__restrict__ list, int32_t list_cap) {
    __shared__ int32_t cur[BWD_CAP];
    const ChunkView cv = chunk_view(tab, batch, blockIdx.x);
    const int32_t *mrow = mat + cv.s.m0 + (int64_t)(blockIdx.x - cv.s.ch0) * cv.s.nkb;
    const int tid = threadIdx.x;
    constexpr int PER = (KMAX + 1 + BIDX_NT - 1) / BIDX_NT;  // entries (incl. tail) a thread
    for (int r0 = 0; r0 < cv.s.nkb; r0 += BWD_CAP) {
        const int nr = min(BWD_CAP, cv.s.nkb - r0);
        for (int i = tid; i < nr; i += BIDX_NT) cur[i] = off[cv.s.kb0 + r0 + i] + mrow[r0 + i];
        __syncthreads();
        int32_t bv[PER];
        int ns = 0;
        auto load_row = [&](int j) {
            const int64_t row = cv.row0 + j;
            ns = nsel_of[row];
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = k * BIDX_NT + tid;
                bv[k] = i < ns ? sel[row * topk + i] : -1;
            }
        };
        if (cv.nrows > 0) load_row(0);
        for (int j = 0; j < cv.nrows; ++j) {
            const int64_t row = cv.row0 + j;
            const int64_t t = cv.tbase + row;
            const int64_t nv = nvis_of(t);
            const int ntail = (int)(t + 1 - BS * nv);
            int32_t b[PER];
            const int ns_cur = ns;
#pragma unroll
            for (int k = 0; k < PER; ++k)
                b[k] = entry_block(bv[k], k * BIDX_NT + tid, ns_cur, topk, nv, ntail);
            if (j + 1 < cv.nrows) load_row(j + 1);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                if (b[k] >= r0 && b[k] < r0 + nr) {
                    const int p = atomicAdd(&cur[b[k] - r0], 1);
                    if (p < list_cap) list[p] = (int32_t)row;
                }
            }
            lds_barrier();
        }
        __syncthreads();
    }
}

// =============================================================== bwd_dq
// One wave per (row, KV head g), keys walked 32 positions at a time as in the forward:
//   S^T, dP^T [32 keys x 16 heads] = K Q^T, V dO^T (A: 2 x 16 key rows, B: the lane's
//   head, dims 32m + 8gr .. +7), P = exp(scale S - lse), dS = P (dP - D);
//   dQ^T [128 dims x 16 heads] += K^T dS^T, dS^T split into bf16 hi + lo (as P in the
//   forward) and K^T rows permuted so that row r of dim tile mt is dim 8r + mt.
// K and V are loaded as whole rows (16 lanes per row); the K rows are the K^T operand as
// loaded and, like V, reach the S^T / dP^T operand layout through a per-wave LDS tile.
constexpr int BDQ_NT = 256;

struct DqArgs {
    const BwdSeq *tab;
    int batch;
    int topk;
    float scale, scale_log2;
    const uint16_t *q, *k, *v, *dout;
    const float *lse, *delta;
    const int32_t *sel, *nsel;
    float *dq;
    int64_t nrows;
};

// K and V rows of the lane's 8 dS keys (keys 4gr..4gr+3 and 16+4gr..16+4gr+3 of the tile),
// dims 8col .. 8col+7: whole 256-byte rows per 16 lanes. K in this layout is the A operand
// of dQ^T = K^T dS^T; K and V also pass through LDS into the layout of S^T and dP^T.
struct DqTile {
    u32x4 kt[8];
    u32x4 vt[8];
    uint32_t valid;  // bit 4u+i: key j0 + 16u + 4gr + i is attended
};
constexpr int DQ_PITCH = 2 * HD + 16;          // LDS bytes per key row
constexpr int DQ_LDS = 2 * 32 * DQ_PITCH;      // a wave's K and V tiles

__global__ void __launch_bounds__(BDQ_NT) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(DqArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[(BDQ_NT / WAVE) * DQ_LDS];
    uint8_t *klds = lds + (threadIdx.x / WAVE) * DQ_LDS, *vlds = klds + 32 * DQ_PITCH;
    // waves in head-major order (every row of KV head 0, then of head 1): the waves in
    // flight gather one head's K/V rows, half the lines
    const int64_t item = __builtin_amdgcn_readfirstlane(
        (int)((int64_t)blockIdx.x * (BDQ_NT / WAVE) + threadIdx.x / WAVE));
    const int g = (int)(item / a.nrows);
    const int64_t row = item - (int64_t)g * a.nrows;
    if (g >= HKV) return;
    const int sb = find_seq(a.batch, row, [&](int i) { return (int64_t)a.tab[i].q0; });
    const BwdSeq S = a.tab[sb];
    const int64_t t = (int64_t)S.L - S.nq + (row - S.q0);
    const int64_t nv = nvis_of(t);
    const int ntail = (int)(t + 1 - BS * nv);
    const int nsel = a.nsel[row];
    const int32_t *srow = a.sel + row * a.topk;
    const int l = lane_id(), gr = l >> 4, col = l & 15;
    const int npos = 4 * (nsel + (ntail > 0 ? 1 : 0));

    const int head = g * GQ + min(col, GQ - 1);
    u32x4 qb[4], ob[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        qb[m] = load16(a.q + (row * HQ + head) * HD + 32 * m + 8 * gr);
        ob[m] = load16(a.dout + (row * HQ + head) * HD + 32 * m + 8 * gr);
    }
    const float lse2 = a.lse[row * HQ + head] * 1.4426950408889634f;
    const float del = a.delta[row * HQ + head];

    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t kv0 = S.k0;
    const int64_t safe_tok = kv0 + t;
    const uint16_t *kbase = a.k + g * HD;
    const uint16_t *vbase = a.v + g * HD;
    auto slot_token0 = [&](int sl, int32_t cur, bool &ok) -> int64_t {
        const int32_t bid = __shfl(cur, sl & 63);
        if (sl < nsel) {
            ok = bid >= 0 && bid < nv;
            return kv0 + (int64_t)BS * bid;
        }
        ok = sl == nsel && ntail > 0;
        return kv0 + (int64_t)BS * nv;
    };
    auto load_tile = [&](int j0, int32_t cur) -> DqTile {
        DqTile T;
        T.valid = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sl = (j0 >> 2) + 4 * u + gr;
            bool okb;
            const int64_t tok0 = slot_token0(sl, cur, okb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 4 * sl + i;
                const bool ok = okb && p < npos && (sl < nsel || i < ntail);
                const int64_t tok = ok ? tok0 + i : safe_tok;
                T.kt[4 * u + i] = load16(kbase + tok * (HKV * HD) + 8 * col);
                T.vt[4 * u + i] = load16(vbase + tok * (HKV * HD) + 8 * col);
                if (ok) T.valid |= 1u << (4 * u + i);
            }
        }
        return T;
    };
    // block ids of slots 64*grp .. 64*grp+63 (lane i: slot 64*grp + i) held in registers,
    // so the loop's only loads are the tiles: per iteration the current tile's K^T rows,
    // then the next tile (past the end: the row's own key). The load counter completes
    // in order, so the waits for the current tile and its K^T leave the next tile's
    // loads in flight.
    int32_t ids[KMAX / WAVE];
#pragma unroll
    for (int j = 0; j < KMAX / WAVE; ++j) ids[j] = srow[min(64 * j + l, a.topk - 1)];
    auto group_ids = [&](int grp) -> int32_t {
        int32_t c = ids[0];
#pragma unroll
        for (int j = 1; j < KMAX / WAVE; ++j)
            if (grp == j) c = ids[j];
        return c;
    };

    int cur_grp = 0;
    int32_t cur = group_ids(0);
    DqTile nxt = load_tile(0, cur);
    for (int j0 = 0; j0 < npos; j0 += 32) {
        const DqTile T = nxt;
        const int jn = j0 + 32;
        if ((jn >> 8) != cur_grp) { cur_grp = jn >> 8; cur = group_ids(cur_grp); }
        nxt = load_tile(jn, cur);
        // K and V rows into the S^T / dP^T A layout (lane: key 16u + col, dims 32m + 8gr)
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int off = (16 * (e >> 2) + 4 * gr + (e & 3)) * DQ_PITCH + 16 * col;
            *reinterpret_cast<u32x4 *>(klds + off) = T.kt[e];
            *reinterpret_cast<u32x4 *>(vlds + off) = T.vt[e];
        }
        wave_lds_sync();
        float ds[8];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, d4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int off = (16 * u + col) * DQ_PITCH + 2 * (32 * m + 8 * gr);
                s4 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4 *>(klds + off), qb[m], s4);
                d4 = mfma_bf16_16x16x32(*reinterpret_cast<const u32x4 *>(vlds + off), ob[m], d4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = (T.valid >> (4 * u + i)) & 1u;
                const float p = ok ? exp2f(s4[i] * a.scale_log2 - lse2) : 0.f;
                ds[4 * u + i] = p * (d4[i] - del);
            }
        }
        u32x4 dh, dl;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            const uint32_t h0 = f32_to_bf16_rne(ds[2 * q2]), h1 = f32_to_bf16_rne(ds[2 * q2 + 1]);
            const float r0 = ds[2 * q2] - __uint_as_float(h0 << 16);
            const float r1 = ds[2 * q2 + 1] - __uint_as_float(h1 << 16);
            dh[q2] = h0 | (h1 << 16);
            dl[q2] = f32_to_bf16_rne(r0) | (f32_to_bf16_rne(r1) << 16);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int q2 = mt >> 1;
            u32x4 ka;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                ka[kk] = bf16_pair(T.kt[2 * kk][q2], T.kt[2 * kk + 1][q2], mt & 1);
            acc[mt] = mfma_bf16_16x16x32(ka, dh, acc[mt]);
            acc[mt] = mfma_bf16_16x16x32(ka, dl, acc[mt]);
        }
    }

    // lane (gr, col): acc[mt][i] = dQ[head col][dim 8*(4gr+i) + mt] / scale
    if (col >= GQ) return;
    float *o = a.dq + (row * HQ + g * GQ + col) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int d0 = 8 * (4 * gr + i);
        const f32x4 lo4 = {acc[0][i] * a.scale, acc[1][i] * a.scale, acc[2][i] * a.scale,
                           acc[3][i] * a.scale};
        const f32x4 hi4 = {acc[4][i] * a.scale, acc[5][i] * a.scale, acc[6][i] * a.scale,
                           acc[7][i] * a.scale};
        *reinterpret_cast<f32x4 *>(o + d0) = lo4;
        *reinterpret_cast<f32x4 *>(o + d0 + 4) = hi4;
    }
}

// =============================================================== bwd_dkv
// One wave per (key block, KV head g), over the rows of the block's list in order. Per
// row: S^T, dP^T [4 keys (of 16) x 12 heads (of 16)] by MFMA with the block's K and V
// rows as the A operand (loaded once). The row's Q and dO are loaded as whole head rows
// (16 lanes per 256-byte row, 3 loads each for the 12 heads) into LDS as [head][dim],
// from where the MFMA B operands and the per-head values below are read; P and dS go
// through LDS as per-(head, key) values. dK and dV of the 4 keys at
// dims 2l, 2l+1 (register i: key i) are accumulated over the 12 heads with the fp32
// 4x4x1 MFMA (16 blocks of 4 x 4): lane l of block l/4 multiplies the value of key i
// held by lane 4(l/4) + i (dS or P, every block the same) by its own Q or dO element,
// one fp32 product per output as a VALU FMA would form it, at twice the VALU rate.
// The next row's Q, dO, lse and D are loaded while the current one is processed.
constexpr int BDKV_NT = 256;
constexpr int QPITCH = HD + 8;  // bf16 per LDS head row (272 bytes: 16-byte rows land on
                                // distinct banks)

struct DkvArgs {
    const BwdSeq *tab;
    int batch;
    float scale, scale_log2;
    const uint16_t *q, *k, *v, *dout;
    const float *lse, *delta;
    const int32_t *off, *list;
    const int32_t *mat, *tot;   // chunk prefixes of each list, list lengths
    float *dk, *dv;
    int64_t kb_lo, kb_hi;       // global key blocks of this launch
    int64_t nrows;
    int win;                    // row window: chunks [win * BWD_WCH, (win + 1) * BWD_WCH)
    int skip_multi;             // skip sequences with more than one window
};

struct DkvRow {
    u32x4 qr[3], orw[3];   // heads 4j + l/16 of the group, dims 8(l%16) .. +7
    float lse, del;
    int64_t t;
};

__global__ void __launch_bounds__(BDKV_NT) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkv_kernel(DkvArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sq[BDKV_NT / WAVE][GQ * QPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t so[BDKV_NT / WAVE][GQ * QPITCH];
    __shared__ __attribute__((aligned(16))) float sp[BDKV_NT / WAVE][GQ * 4];
    __shared__ __attribute__((aligned(16))) float sds[BDKV_NT / WAVE][GQ * 4];
    const int w = threadIdx.x / WAVE;
    const int64_t item = __builtin_amdgcn_readfirstlane(
        (int)((int64_t)blockIdx.x * (BDKV_NT / WAVE) + w));
    // (the two KV heads of a block on neighbouring waves: head-major order, which speeds
    // up dQ, measured slower here)
    const int64_t gb = a.kb_lo + (item >> 1);
    const int g = (int)(item & 1);
    if (gb >= a.kb_hi) return;
    const int sb = find_seq(a.batch, gb, [&](int i) { return (int64_t)a.tab[i].kb0; });
    const BwdSeq S = a.tab[sb];
    if (a.skip_multi && S.nch > BWD_WCH) return;
    const int b = (int)(gb - S.kb0);
    // the block's list entries from the rows of this window (lists are in row order)
    auto prefix = [&](int c) -> int32_t {
        return c >= S.nch ? a.tot[gb] : a.mat[S.m0 + (int64_t)c * S.nkb + b];
    };
    const int c0 = min(a.win * BWD_WCH, S.nch);
    const int32_t base = a.off[gb];
    const int lo = base + prefix(c0), hi = base + prefix(min(c0 + BWD_WCH, S.nch));
    if (a.win > 0 && lo >= hi) return;
    const int64_t tok0 = (int64_t)S.k0 + BS * b;
    const int nkeys = min(BS, S.L - BS * b);
    const int l = lane_id(), gr = l >> 4, col = l & 15;

    u32x4 ka[4], va[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int64_t tok = tok0 + min(col, nkeys - 1);
        ka[m] = load16(a.k + (tok * HKV + g) * HD + 32 * m + 8 * gr);
        va[m] = load16(a.v + (tok * HKV + g) * HD + 32 * m + 8 * gr);
        if (col >= nkeys) ka[m] = va[m] = u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t tbase = (int64_t)S.L - S.nq - S.q0;
    const int head = g * GQ + min(col, GQ - 1);

    // dk0[i], dk1[i]: dK of key i at dims 2l, 2l+1 (likewise dV)
    f32x4 dk0 = {0.f, 0.f, 0.f, 0.f}, dk1 = dk0, dv0 = dk0, dv1 = dk0;

    auto load_row = [&](int64_t row) -> DkvRow {
        row = min<int64_t>(max<int64_t>(row, 0), a.nrows - 1);  // list entries are rows
        DkvRow R;
        const int64_t rb = (row * HQ + g * GQ + (l >> 4)) * HD + 8 * (l & 15);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            R.qr[j] = load16(a.q + rb + (int64_t)4 * j * HD);
            R.orw[j] = load16(a.dout + rb + (int64_t)4 * j * HD);
        }
        R.lse = a.lse[row * HQ + head];
        R.del = a.delta[row * HQ + head];
        R.t = tbase + row;
        return R;
    };

    uint16_t *wq = sq[w], *wo = so[w];
    float *wp = sp[w], *wds = sds[w];
    const int hc = min(col, GQ - 1);   // head of the lane's S^T / dP^T column
    auto process = [&](const DkvRow &R) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int o = (4 * j + (l >> 4)) * QPITCH + 8 * (l & 15);
            *reinterpret_cast<u32x4 *>(wq + o) = R.qr[j];
            *reinterpret_cast<u32x4 *>(wo + o) = R.orw[j];
        }
        wave_lds_sync();
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f}, d4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const u32x4 qb = *reinterpret_cast<const u32x4 *>(wq + hc * QPITCH + 32 * m + 8 * gr);
            const u32x4 ob = *reinterpret_cast<const u32x4 *>(wo + hc * QPITCH + 32 * m + 8 * gr);
            s4 = mfma_bf16_16x16x32(ka[m], qb, s4);
            d4 = mfma_bf16_16x16x32(va[m], ob, d4);
        }
        // lanes (0, col < 12): keys i = 0..3 of head col
        if (gr == 0 && col < GQ) {
            const float lse2 = R.lse * 1.4426950408889634f;
            f32x4 p4, ds4;
#pragma unroll
            for (int i = 0; i < BS; ++i) {
                const bool ok = BS * b + i <= R.t;
                const float p = ok ? exp2f(s4[i] * a.scale_log2 - lse2) : 0.f;
                p4[i] = p;
                ds4[i] = p * (d4[i] - R.del);
            }
            *reinterpret_cast<f32x4 *>(wp + 4 * col) = p4;
            *reinterpret_cast<f32x4 *>(wds + 4 * col) = ds4;
        }
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const uint32_t qq = *reinterpret_cast<const uint32_t *>(wq + h * QPITCH + 2 * l);
            const uint32_t oo = *reinterpret_cast<const uint32_t *>(wo + h * QPITCH + 2 * l);
            const float pa = wp[4 * h + (l & 3)];    // P of key l % 4, head h
            const float da = wds[4 * h + (l & 3)];   // dS of key l % 4, head h
            dk0 = mfma_f32_4x4x1(da, bf16_lo(qq), dk0);
            dk1 = mfma_f32_4x4x1(da, bf16_hi(qq), dk1);
            dv0 = mfma_f32_4x4x1(pa, bf16_lo(oo), dv0);
            dv1 = mfma_f32_4x4x1(pa, bf16_hi(oo), dv1);
        }
        wave_lds_sync();
    };
    // Three row buffers used in turn (no register copies): each step issues the loads of
    // the row two entries ahead before it processes the current row, so the waits leave
    // two rows' loads in flight (two waves per SIMD hold the registers). Loads past the
    // end repeat the last entry's row.
    if (lo < hi) {
        auto row_id = [&](int e) -> int32_t {
            return __builtin_amdgcn_readfirstlane(a.list[min(e, hi - 1)]);
        };
        DkvRow A = load_row(row_id(lo));
        DkvRow B = load_row(row_id(lo + 1));
        for (int e = lo; e < hi; e += 3) {
            const DkvRow C = load_row(row_id(e + 2));
            __builtin_amdgcn_sched_barrier(0);
            process(A);
            if (e + 1 >= hi) break;
            A = load_row(row_id(e + 3));
            __builtin_amdgcn_sched_barrier(0);
            process(B);
            if (e + 2 >= hi) break;
            B = load_row(row_id(e + 4));
            __builtin_amdgcn_sched_barrier(0);
            process(C);
        }
    }
    // window 0 writes the block's gradients, later windows (later launches) add to them
#pragma unroll
    for (int i = 0; i < BS; ++i) {
        if (i < nkeys) {
            const int64_t o = ((tok0 + i) * HKV + g) * HD + 2 * l;
            float2 k2 = float2{dk0[i] * a.scale, dk1[i] * a.scale};
            float2 v2 = float2{dv0[i], dv1[i]};
            if (a.win > 0) {
                const float2 pk = *reinterpret_cast<const float2 *>(a.dk + o);
                const float2 pv = *reinterpret_cast<const float2 *>(a.dv + o);
                k2 = float2{pk.x + k2.x, pk.y + k2.y};
                v2 = float2{pv.x + v2.x, pv.y + v2.y};
            }
            *reinterpret_cast<float2 *>(a.dk + o) = k2;
            *reinterpret_cast<float2 *>(a.dv + o) = v2;
        }
    }
}

// =============================================================== launcher
hipError_t launch_backward(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_q_host,
                           const int32_t *cu_k_host, int batch, int topk,
                           float scale, int64_t n_rows, int64_t n_chunks, int64_t nkb_total,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const int32_t *sel, const float *out, const float *lse,
                           const uint16_t *dout, float *dq, float *dk, float *dv,
                           const BwdBuffers &bb, hipStream_t st, hipStream_t side,
                           hipEvent_t fork, hipEvent_t join) {
    hipError_t e;
    trace_before(6, st);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(1), dim3(BPREP_NT), 0, st, cu_q, cu_k, batch, bb.seq);
    if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
    if (n_rows > 0) {
        trace_before(7, st);
        const int64_t wg = (n_rows + BROWS_NT / WAVE - 1) / (BROWS_NT / WAVE);
        hipLaunchKernelGGL(bwd_rows_kernel, dim3((unsigned)wg), dim3(BROWS_NT), 0, st, sel, topk,
                           dout, out, n_rows, bb.nsel, bb.delta);
        if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
    }
    if (n_chunks > 0) {
        trace_before(8, st);
        hipLaunchKernelGGL(bwd_count_kernel, dim3((unsigned)n_chunks), dim3(BIDX_NT), 0, st,
                           bb.seq, batch, sel, topk, bb.nsel, bb.mat);
        if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
    }
    if (nkb_total > 0) {
        trace_before(9, st);
        hipLaunchKernelGGL(bwd_colscan_kernel, dim3((unsigned)((nkb_total + BCOL_NT - 1) / BCOL_NT)),
                           dim3(BCOL_NT), 0, st, bb.seq, batch, nkb_total, bb.mat, bb.tot);
        if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
        trace_before(10, st);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(BSCAN_NT), 0, st, bb.tot, nkb_total,
                           bb.off);
        if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
    }
    if (n_chunks > 0) {
        trace_before(11, st);
        hipLaunchKernelGGL(bwd_fill_kernel, dim3((unsigned)n_chunks), dim3(BIDX_NT), 0, st,
                           bb.seq, batch, sel, topk, bb.nsel, bb.mat, bb.off, bb.list,
                           (int32_t)(n_rows * (topk + 1)));
        if ((e = trace_after(st, hipGetLastError())) != hipSuccess) return e;
    }
    // dQ (row-major, writes dq only) and dK/dV (key-major, writes dk and dv only) read the
    // same inputs and the finished index: with a side stream they run concurrently
    hipStream_t sq = st;
    if (side && n_rows > 0 && nkb_total > 0) {
        if ((e = hipEventRecord(fork, st)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
        sq = side;
    }
    hipError_t edq = hipSuccess;
    if (n_rows > 0) {
        DqArgs a;
        a.tab = bb.seq; a.batch = batch; a.topk = topk;
        a.scale = scale; a.scale_log2 = scale * 1.4426950408889634f;
        a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse; a.delta = bb.delta;
        a.sel = sel; a.nsel = bb.nsel; a.dq = dq; a.nrows = n_rows;
        const int64_t wg = (n_rows * HKV + BDQ_NT / WAVE - 1) / (BDQ_NT / WAVE);
        trace_before(12, sq);
        hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)wg), dim3(BDQ_NT), 0, sq, a);
        edq = trace_after(sq, hipGetLastError());
    }
    // the dK/dV launches; then st waits for the side stream (also after an error)
    auto run_dkv = [&]() -> hipError_t {
    if (edq != hipSuccess) return edq;
    if (nkb_total > 0) {
        DkvArgs a;
        a.tab = bb.seq; a.batch = batch;
        a.scale = scale; a.scale_log2 = scale * 1.4426950408889634f;
        a.q = q; a.k = k; a.v = v; a.dout = dout; a.lse = lse; a.delta = bb.delta;
        a.off = bb.off; a.list = bb.list; a.mat = bb.mat; a.tot = bb.tot;
        a.dk = dk; a.dv = dv; a.nrows = n_rows;
        auto launch = [&](int64_t lo, int64_t hi, int win, int skip_multi) -> hipError_t {
            a.kb_lo = lo; a.kb_hi = hi; a.win = win; a.skip_multi = skip_multi;
            const int64_t wg = ((hi - lo) * HKV + BDKV_NT / WAVE - 1) / (BDKV_NT / WAVE);
            trace_before(13, st);
            hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)wg), dim3(BDKV_NT), 0, st, a);
            return trace_after(st, hipGetLastError());
        };
        // one launch for every sequence with a single row window, then one launch per
        // window of each longer sequence: the rows a launch gathers stay cache-resident
        if ((e = launch(0, nkb_total, 0, 1)) != hipSuccess) return e;
        int64_t kb0 = 0;
        for (int s = 0; s < batch; ++s) {
            const int64_t L = (int64_t)cu_k_host[s + 1] - cu_k_host[s];
            const int64_t nq = (int64_t)cu_q_host[s + 1] - cu_q_host[s];
            const int64_t nkb = (L + BS - 1) / BS, nch = (nq + BWD_CH - 1) / BWD_CH;
            if (nch > BWD_WCH)
                for (int w = 0; w * (int64_t)BWD_WCH < nch; ++w)
                    if ((e = launch(kb0, kb0 + nkb, w, 0)) != hipSuccess) return e;
            kb0 += nkb;
        }
    }
    return hipSuccess;
    };
    const hipError_t ekv = run_dkv();
    if (sq != st) {
        const hipError_t ej = hipEventRecord(join, sq);
        const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(st, join, 0) : ej;
        if (ekv == hipSuccess && ew != hipSuccess) return ew;
    }
    return ekv;
}

}  // namespace qsa
