// qsa_kernels.hip -- gfx950 kernels of the QSA hot path:
//   prep     per-sequence bookkeeping table (one workgroup)
//   compress micro-block key compression (HBM stream)
//   score    indexer scores, bf16 MFMA 16x16x32 with fp32 accumulation
//   select   exact per-row top-k by radix select in LDS
//   attend   sparse GQA attention over gathered micro-blocks (MFMA, online softmax)
//   combine  split-K merge of attention partials
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// =============================================================== prep
// One workgroup scans the sequences: first compressed block, first score tile and
// first score slot of each. Score rows are the positions t >= max(L-nq, 4*topk+3)
// (more visible blocks than the budget); they are tiled 4 rows at a time.
constexpr int PREP_NT = 1024;

__global__ void __launch_bounds__(PREP_NT)
prep_kernel(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k, int batch,
            int topk, SeqInfo *__restrict__ tab) {
    __shared__ int64_t sh[PREP_NT / WAVE + 1];
    int64_t carry_blk = 0, carry_tile = 0, carry_slot = 0;
    for (int base = 0; base < batch; base += PREP_NT) {
        const int b = base + threadIdx.x;
        int32_t q0 = 0, nq = 0, k0 = 0, L = 0;
        int64_t nblk = 0, ntile = 0, nslot = 0;
        if (b < batch) {
            q0 = cu_q[b]; nq = cu_q[b + 1] - q0;
            k0 = cu_k[b]; L = cu_k[b + 1] - k0;
            nblk = L / BS;
            int64_t ts = first_scored_pos(L, nq, topk);
            if (ts < L) {
                ntile = (L - ts + 3) / 4;
                nslot = slots_before(L) - slots_before(ts);
            }
        }
        int64_t tot;
        int64_t eb = block_excl_scan<int64_t, PREP_NT>(nblk, sh, &tot);
        int64_t sum_blk = tot;
        int64_t et = block_excl_scan<int64_t, PREP_NT>(ntile, sh, &tot);
        int64_t sum_tile = tot;
        int64_t es = block_excl_scan<int64_t, PREP_NT>(nslot, sh, &tot);
        int64_t sum_slot = tot;
        if (b < batch) {
            SeqInfo s;
            s.q0 = q0; s.nq = nq; s.k0 = k0; s.L = L;
            s.blk0 = (int32_t)(carry_blk + eb);
            s.tile0 = (int32_t)(carry_tile + et);
            s.s0 = carry_slot + es;
            tab[b] = s;
        }
        carry_blk += sum_blk; carry_tile += sum_tile; carry_slot += sum_slot;
    }
}

// =============================================================== compress
// Sum of the 4 indexer keys of each micro-block, exactly (double), rounded once to
// bf16. Thread = (block, 8 consecutive dims): 4 x 16-byte reads, one 16-byte write,
// so a wave streams 8 whole blocks (4 KiB in, 1 KiB out) with full coalescing.
constexpr int CMP_NT = 256;
constexpr int CMP_BLOCKS_PER_WG = CMP_NT / 8;

__global__ void __launch_bounds__(CMP_NT)
compress_kernel(const int32_t *__restrict__ cu_q, const int32_t *__restrict__ cu_k,
                const uint16_t *__restrict__ k_idx, uint16_t *__restrict__ k_blk,
                int incremental) {
    __shared__ int64_t red[CMP_NT / WAVE + 1];
    const int b = blockIdx.y;
    const int32_t k0 = cu_k[b], L = cu_k[b + 1] - k0;
    const int64_t nblk = L / BS;
    int64_t lo = 0;
    if (incremental) {
        const int32_t nq = cu_q[b + 1] - cu_q[b];
        lo = (int64_t)(L - nq) / BS;
    }
    const int64_t blk = lo + (int64_t)blockIdx.x * CMP_BLOCKS_PER_WG + threadIdx.x / 8;
    if (lo + (int64_t)blockIdx.x * CMP_BLOCKS_PER_WG >= nblk) return;  // whole WG idle

    // first block row of this sequence: sum of floor(L_i/4) over earlier sequences
    int64_t part = 0;
    for (int i = threadIdx.x; i < b; i += CMP_NT) part += (cu_k[i + 1] - cu_k[i]) / BS;
    int64_t tot;
    (void)block_excl_scan<int64_t, CMP_NT>(part, red, &tot);
    const int64_t blk0 = tot;

    if (blk >= nblk) return;
    const int c = threadIdx.x % 8;
    const uint16_t *src = k_idx + ((int64_t)k0 + blk * BS) * DI + c * 8;
    u32x4 r0 = load16(src), r1 = load16(src + DI), r2 = load16(src + 2 * DI),
          r3 = load16(src + 3 * DI);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        double s_lo = (((double)bf16_lo(r0[q]) + (double)bf16_lo(r1[q])) + (double)bf16_lo(r2[q])) +
                      (double)bf16_lo(r3[q]);
        double s_hi = (((double)bf16_hi(r0[q]) + (double)bf16_hi(r1[q])) + (double)bf16_hi(r2[q])) +
                      (double)bf16_hi(r3[q]);
        out[q] = f64_to_bf16_rne(s_lo) | (f64_to_bf16_rne(s_hi) << 16);
    }
    *reinterpret_cast<u32x4 *>(k_blk + (blk0 + blk) * DI + c * 8) = out;
}

// =============================================================== score
// Tile = 4 consecutive score rows of one sequence; MFMA rows = (row, indexer head)
// pairs (16 = 4 x 4), columns = 16 blocks, K = 64 indexer dims in two 16x16x32
// steps. The contraction order of the dims is permuted so that each lane reads
// 16 contiguous bytes of a block key per step (A and B use the same permutation):
// step m, lane group g holds dims 32m + 8g .. 32m + 8g + 7.
// Output lane (g, c) holds the 4 head dot products of row g and block c, so the
// score sum_h w_h relu(dot_h) is formed in-lane and stored as an order key.
constexpr int SCORE_NT = 256;

__global__ void __launch_bounds__(SCORE_NT)
score_kernel(const SeqInfo *__restrict__ tab, int batch, int topk,
             const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
             const uint16_t *__restrict__ k_blk, uint32_t *__restrict__ keys,
             int64_t chunk_blocks) {
    const int64_t tile = blockIdx.x;
    const int sb = upper_index(batch, tile, [&](int i) { return (int64_t)tab[i].tile0; });
    const SeqInfo s = tab[sb];
    const int64_t ts = first_scored_pos(s.L, s.nq, topk);
    const int64_t t0 = ts + 4 * (tile - s.tile0);
    const int nrows = (int)min<int64_t>(4, s.L - t0);
    const int64_t row0 = s.q0 + (t0 - (s.L - s.nq));
    const int64_t nv_max = nvis_of(t0 + nrows - 1);
    const int64_t lo = (int64_t)blockIdx.y * chunk_blocks;
    const int64_t hi = min<int64_t>(nv_max, lo + chunk_blocks);
    if (lo >= hi) return;

    const int l = lane_id(), g = l >> 4, c = l & 15;
    // A operand: q_idx of (row (c>>2), head (c&3)), dims of lane group g
    u32x4 qa[2];
    {
        const int rr = c >> 2, hh = c & 3;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (rr < nrows)
                qa[m] = load16(q_idx + ((row0 + rr) * HI + hh) * DI + 32 * m + 8 * g);
            else
                qa[m] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // output side: row g of the tile
    float wr[HI] = {0.f, 0.f, 0.f, 0.f};
    int64_t slot = 0, nv_row = 0;
    if (g < nrows) {
#pragma unroll
        for (int h = 0; h < HI; ++h) wr[h] = w[(row0 + g) * HI + h];
        slot = s.s0 + slots_before(t0 + g) - slots_before(ts);
        nv_row = nvis_of(t0 + g);
    }
    const uint16_t *kb = k_blk + (int64_t)s.blk0 * DI;
    const int wv = threadIdx.x / WAVE;
    for (int64_t base = lo + 16 * wv; base < hi; base += 16 * (SCORE_NT / WAVE)) {
        const int64_t blk = base + c;
        const int64_t blk_ld = blk < hi ? blk : hi - 1;
        const uint16_t *src = kb + blk_ld * DI + 8 * g;
        u32x4 b0 = load16(src), b1 = load16(src + 32);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_bf16_16x16x32(qa[0], b0, acc);
        acc = mfma_bf16_16x16x32(qa[1], b1, acc);
        float sc = wr[0] * fmaxf(acc[0], 0.f);
        sc += wr[1] * fmaxf(acc[1], 0.f);
        sc += wr[2] * fmaxf(acc[2], 0.f);
        sc += wr[3] * fmaxf(acc[3], 0.f);
        if (blk < nv_row) keys[slot + blk] = score_key(sc);
    }
}

// =============================================================== select
// One workgroup per query row. Rows within the budget keep blocks 0..nvis-1. Other
// rows: exact radix select of the topk-th largest key over 3 digit passes
// (12 + 12 + 8 bits) with LDS histograms, then one ordered pass that keeps every key
// above the threshold and the lowest-index keys equal to it, written in ascending
// block order through block-wide prefix counts.
constexpr int SEL_NT = 256;
constexpr int SEL_PER = 16;  // keys per thread per sweep (contiguous)

__global__ void __launch_bounds__(SEL_NT)
select_kernel(const SeqInfo *__restrict__ tab, int batch, int topk,
              const uint32_t *__restrict__ keys, int32_t *__restrict__ sel) {
    __shared__ uint32_t hist[4096];
    __shared__ int64_t scan_sh[SEL_NT / WAVE + 1];
    __shared__ uint32_t found[2];

    const int64_t row = blockIdx.x;
    const int sb = upper_index(batch, row, [&](int i) { return (int64_t)tab[i].q0; });
    const SeqInfo s = tab[sb];
    const int64_t t = (int64_t)s.L - s.nq + (row - s.q0);
    const int64_t nv = nvis_of(t);
    int32_t *out = sel + row * topk;
    const int tid = threadIdx.x;
    if (tid == 0) { found[0] = 0; found[1] = 0; }

    if (nv <= topk) {
        for (int i = tid; i < topk; i += SEL_NT) out[i] = i < nv ? i : -1;
        return;
    }
    const int64_t ts = first_scored_pos(s.L, s.nq, topk);
    const uint32_t *rk = keys + s.s0 + slots_before(t) - slots_before(ts);
    const int64_t n = nv;

    uint32_t prefix = 0, pmask = 0;
    int64_t need = topk;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass], nb = 1 << widths[pass];
        const uint32_t dmask = (uint32_t)nb - 1;
        for (int i = tid; i < nb; i += SEL_NT) hist[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < n; i += SEL_NT) {
            uint32_t kk = rk[i];
            if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1u);
        }
        __syncthreads();
        // thread j owns the per consecutive bins ending at nb - per*j (highest first)
        const int per = nb / SEL_NT;
        const int top = nb - per * tid;
        int64_t local = 0;
        for (int i = 1; i <= per; ++i) local += hist[top - i];
        int64_t tot;
        int64_t above = block_excl_scan<int64_t, SEL_NT>(local, scan_sh, &tot);
        if (above < need && need <= above + local) {
            int64_t run = above;
            for (int i = 1; i <= per; ++i) {
                const int bin = top - i;
                if (run + hist[bin] >= need) {
                    found[0] = (uint32_t)bin;
                    found[1] = (uint32_t)(run);
                    break;
                }
                run += hist[bin];
            }
        }
        __syncthreads();
        const uint32_t digit = found[0];
        need -= (int64_t)found[1];
        prefix |= digit << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    const uint32_t theta = prefix;  // the topk-th largest key; take `need` equal keys

    int64_t run_eq = 0, run_sel = 0;
    for (int64_t base = 0; base < n; base += (int64_t)SEL_NT * SEL_PER) {
        const int64_t i0 = base + (int64_t)tid * SEL_PER;
        uint32_t kk[SEL_PER];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < SEL_PER; ++e) {
            kk[e] = (i0 + e < n) ? rk[i0 + e] : 0u;
            n_eq += (i0 + e < n && kk[e] == theta);
        }
        int64_t tot_eq;
        int64_t eq_before = run_eq + block_excl_scan<int64_t, SEL_NT>(n_eq, scan_sh, &tot_eq);
        int n_take = 0;
        int64_t eq_run = eq_before;
        uint32_t take_mask = 0;
#pragma unroll
        for (int e = 0; e < SEL_PER; ++e) {
            bool valid = i0 + e < n;
            bool gt = valid && kk[e] > theta;
            bool eq = valid && kk[e] == theta;
            bool take = gt || (eq && eq_run < need);
            eq_run += eq;
            if (take) { take_mask |= 1u << e; ++n_take; }
        }
        int64_t tot_take;
        int64_t pos = run_sel + block_excl_scan<int64_t, SEL_NT>(n_take, scan_sh, &tot_take);
#pragma unroll
        for (int e = 0; e < SEL_PER; ++e)
            if (take_mask & (1u << e)) {
                if (pos < topk) out[pos] = (int32_t)(i0 + e);
                ++pos;
            }
        run_eq += tot_eq;
        run_sel += tot_take;
    }
}

// =============================================================== attend
// One wave per (query row, key/value head g, key split). The row's keys are the
// tokens of its kept blocks in ascending order, then its raw tail (treated as one
// more block slot with 0..3 valid tokens). A wave walks them 32 at a time:
//   S^T[32 keys x 16 heads] = K (A operand, 2 x 16 keys) * Q^T (B operand, 12 live
//   heads of group g): 4 MFMA 16x16x32 steps per 16 keys over the 128 dims, with the
//   dims permuted so each lane reads 16 contiguous bytes (step m, group gr holds
//   dims 32m + 8gr .. +7).
//   Online softmax per head in base 2; each lane owns one head (its column).
//   O^T[128 dims x 16 heads] += V^T * P^T: P^T is the lane's own 8 probabilities
//   (keys 4gr..4gr+3 and 16+4gr..16+4gr+3, the k-slots of its lane group), split
//   into bf16 hi + lo parts (2 MFMAs) to keep ~16 bits; V^T rows are permuted so row
//   r of dim-tile mt is dim 8r + mt, which lets each lane load 16 contiguous bytes of
//   V per key.
// S = 1: final output. S > 1: unnormalised partial (m, l, acc) for the combine.
constexpr int ATT_NT = 256;
// split partial record per (row, split, head): acc[128], m, l, 2 pad (16-byte aligned)
constexpr int PREC = HD + 4;

struct AttnArgs {
    const SeqInfo *tab;
    int batch;
    int topk;
    float scale_log2;  // softmax scale * log2(e)
    const uint16_t *q, *k, *v;
    const int32_t *sel;
    float *out, *lse;
    float *part;       // split partials (S > 1)
    int nsplit;
    int64_t nrows;
};

__device__ __forceinline__ int64_t part_stride_row(int nsplit) {
    return (int64_t)nsplit * HQ * PREC;
}

__global__ void __launch_bounds__(ATT_NT)
attend_kernel(AttnArgs a) {
    const int64_t item = (int64_t)blockIdx.x * (ATT_NT / WAVE) + threadIdx.x / WAVE;
    const int64_t row = item / (HKV * a.nsplit);
    if (row >= a.nrows) return;
    const int rem = (int)(item % (HKV * a.nsplit));
    const int g = rem / a.nsplit, sp = rem % a.nsplit;

    const int sb = upper_index(a.batch, row, [&](int i) { return (int64_t)a.tab[i].q0; });
    const SeqInfo s = a.tab[sb];
    const int64_t t = (int64_t)s.L - s.nq + (row - s.q0);
    const int64_t nv = nvis_of(t);
    const int ntail = (int)(t + 1 - BS * nv);
    const int32_t *srow = a.sel + row * a.topk;

    const int l = lane_id(), gr = l >> 4, col = l & 15;

    // number of leading selected entries (stop at the first -1)
    int nsel = a.topk;
    for (int i0 = 0; i0 < a.topk; i0 += WAVE) {
        int i = i0 + l;
        bool neg = i < a.topk && srow[i] < 0;
        unsigned long long bal = __ballot(neg);
        if (bal) { nsel = i0 + __builtin_ctzll(bal); break; }
    }
    const int nslot = nsel + (ntail > 0 ? 1 : 0);
    const int npos = 4 * nslot;
    int chunk = (npos + a.nsplit - 1) / a.nsplit;
    chunk = (chunk + 31) & ~31;
    const int p_lo = sp * chunk;
    const int p_hi = min(npos, p_lo + chunk);

    // Q^T operand: head g*12 + col, dims of lane group gr
    const int head = g * GQ + col;
    u32x4 qb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (col < GQ)
            qb[m] = load16(a.q + (row * HQ + head) * HD + 32 * m + 8 * gr);
        else
            qb[m] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t kvrow0 = (int64_t)s.k0;
    const int64_t safe_tok = kvrow0 + t;  // always a valid key row
    auto slot_block = [&](int slot, bool &ok) -> int64_t {
        if (slot < nsel) {
            int32_t bid = srow[slot];
            ok = bid >= 0 && bid < nv;
            return bid;
        }
        ok = (slot == nsel && ntail > 0);
        return nv;
    };
    auto key_token = [&](int p, bool &ok) -> int64_t {
        bool okb;
        int64_t bid = slot_block(p >> 2, okb);
        const int i = p & 3;
        ok = okb && p < p_hi && (p >> 2 < nsel || i < ntail);
        return ok ? kvrow0 + BS * bid + i : safe_tok;
    };

    for (int j0 = p_lo; j0 < p_hi; j0 += 32) {
        // ---- scores S^T for keys j0 .. j0+31
        f32x4 sc[2];
        bool kval[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            bool ok;
            const int64_t tok = key_token(j0 + 16 * u + col, ok);
            (void)ok;
            const uint16_t *kp = a.k + (tok * HKV + g) * HD + 8 * gr;
            f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) c4 = mfma_bf16_16x16x32(load16(kp + 32 * m), qb[m], c4);
            sc[u] = c4;
            kval[u] = false;
        }
        (void)kval;
        // lane (gr, col): sc[u][i] = logit of key j0 + 16u + 4gr + i for head col
        float z[8];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bool ok;
                (void)key_token(j0 + 16 * u + 4 * gr + i, ok);
                float zz = ok ? sc[u][i] * a.scale_log2 : -INFINITY;
                z[4 * u + i] = zz;
                mx = fmaxf(mx, zz);
            }
        }
        mx = wave_max_xor_16_32(mx);
        const float m_new = fmaxf(m_run, mx);
        if (m_new == -INFINITY) continue;  // nothing valid yet (whole wave agrees)
        const float alpha = exp2f(m_run - m_new);
        float p[8], rs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = z[e] == -INFINITY ? 0.f : exp2f(z[e] - m_new);
            rs += p[e];
        }
        rs = wave_sum_xor_16_32(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[mt] *= alpha;

        // P^T operand, hi and lo bf16 parts
        u32x4 ph, pl;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            uint32_t h0 = f32_to_bf16_rne(p[2 * q2]), h1 = f32_to_bf16_rne(p[2 * q2 + 1]);
            float r0 = p[2 * q2] - __uint_as_float(h0 << 16);
            float r1 = p[2 * q2 + 1] - __uint_as_float(h1 << 16);
            ph[q2] = h0 | (h1 << 16);
            pl[q2] = f32_to_bf16_rne(r0) | (f32_to_bf16_rne(r1) << 16);
        }
        // V rows of the lane's 8 keys, dims 8*col .. 8*col+7
        u32x4 vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bool ok;
            const int pe = j0 + (e < 4 ? 4 * gr + e : 16 + 4 * gr + (e - 4));
            const int64_t tok = key_token(pe, ok);
            vv[e] = load16(a.v + (tok * HKV + g) * HD + 8 * col);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int q2 = mt >> 1;
            u32x4 va;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                uint32_t x0 = vv[2 * kk][q2], x1 = vv[2 * kk + 1][q2];
                va[kk] = (mt & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u))
                                  : ((x0 & 0xffffu) | (x1 << 16));
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
            f32x4 lo4 = {acc[0][i] * inv, acc[1][i] * inv, acc[2][i] * inv, acc[3][i] * inv};
            f32x4 hi4 = {acc[4][i] * inv, acc[5][i] * inv, acc[6][i] * inv, acc[7][i] * inv};
            *reinterpret_cast<f32x4 *>(o + d0) = lo4;
            *reinterpret_cast<f32x4 *>(o + d0 + 4) = hi4;
        }
        if (a.lse && gr == 0)
            a.lse[row * HQ + head] = l_run > 0.f ? m_run * 0.69314718055994531f + logf(l_run)
                                                 : -INFINITY;
    } else {
        float *pp = a.part + row * part_stride_row(a.nsplit) +
                    ((int64_t)sp * HQ + head) * PREC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 8 * (4 * gr + i);
            f32x4 lo4 = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
            f32x4 hi4 = {acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
            *reinterpret_cast<f32x4 *>(pp + d0) = lo4;
            *reinterpret_cast<f32x4 *>(pp + d0 + 4) = hi4;
        }
        if (gr == 0) { pp[HD] = m_run; pp[HD + 1] = l_run; }
    }
}

// =============================================================== combine
// One wave per (row, head): log-sum-exp merge of the split partials, in split order.
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
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, pr[sp * sstride + HD]);
    float Lsum = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
        for (int sp = 0; sp < nsplit; ++sp) {
            const float *ps = pr + sp * sstride;
            const float ms = ps[HD];
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            Lsum += ps[HD + 1] * f;
            o0 += ps[2 * l] * f;
            o1 += ps[2 * l + 1] * f;
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float *o = out + (row * HQ + head) * HD;
    o[2 * l] = o0 * inv;
    o[2 * l + 1] = o1 * inv;
    if (lse && l == 0)
        lse[row * HQ + head] = Lsum > 0.f ? M * 0.69314718055994531f + logf(Lsum) : -INFINITY;
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
                           int incremental, hipStream_t st) {
    if (max_blocks <= 0 || batch <= 0) return hipSuccess;
    const int64_t gx = (max_blocks + CMP_BLOCKS_PER_WG - 1) / CMP_BLOCKS_PER_WG;
    trace_before(1, st);
    hipLaunchKernelGGL(compress_kernel, dim3((unsigned)gx, (unsigned)batch), dim3(CMP_NT), 0, st,
                       cu_q, cu_k, k_idx, k_blk, incremental);
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

hipError_t launch_select(const SeqInfo *tab, int batch, int topk, const uint32_t *keys,
                         int32_t *sel, int64_t n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    trace_before(3, st);
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)n_rows), dim3(SEL_NT), 0, st, tab, batch,
                       topk, keys, sel);
    return trace_after(st, hipGetLastError());
}

hipError_t launch_attend(const SeqInfo *tab, int batch, int topk, float scale,
                         const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const int32_t *sel, float *out, float *lse, float *part, int nsplit,
                         int64_t n_rows, hipStream_t st) {
    if (n_rows <= 0) return hipSuccess;
    AttnArgs a;
    a.tab = tab; a.batch = batch; a.topk = topk;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = q; a.k = k; a.v = v; a.sel = sel; a.out = out; a.lse = lse; a.part = part;
    a.nsplit = nsplit; a.nrows = n_rows;
    const int64_t waves = n_rows * HKV * nsplit;
    const int64_t wgs = (waves + ATT_NT / WAVE - 1) / (ATT_NT / WAVE);
    trace_before(4, st);
    hipLaunchKernelGGL(attend_kernel, dim3((unsigned)wgs), dim3(ATT_NT), 0, st, a);
    hipError_t e = trace_after(st, hipGetLastError());
    if (e != hipSuccess || nsplit == 1) return e;
    const int64_t cw = (n_rows * HQ + CMB_NT / WAVE - 1) / (CMB_NT / WAVE);
    trace_before(5, st);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)cw), dim3(CMB_NT), 0, st, part, nsplit,
                       n_rows, out, lse);
    return trace_after(st, hipGetLastError());
}

}  // namespace qsa
