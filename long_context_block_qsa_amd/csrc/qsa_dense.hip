// qsa_dense.hip -- attention of the query rows in the dense regime.
//
// A query at position t sees nvis(t) = floor((t+1)/4) complete blocks; while that is
// no more than the budget it keeps all of them (and its raw tail), so it attends every
// token 0..t: plain causal attention. QSA is full attention in this regime
// (blog.compendialabs.org, "Qwen Sparse Attention -- Full Attention When It Counts";
// budget of elzobrito.github.io, "Linear attention carries the stream; sparse
// attention retrieves detail"). Every such row of a sequence reads the same keys, so
// instead of gathering them row by row they are staged once per workgroup in LDS and
// shared by DN_ROWS consecutive query rows x the 12 query heads of one KV head.
//
// Workgroup = (dense tile of DN_ROWS = 16 rows, KV head g): its 192 query vectors (16
// rows x 12 heads, vector v = row * 12 + head) are 12 MFMA column tiles of 16, over 8
// waves. Per tile of 32 keys, each wave computes, for each of its column tiles,
//   S^T[32 keys x 16] = K (A operand from LDS, bf16) x Q^T (B operand, registers):
//     2 key halves x 4 steps of MFMA 16x16x32 over the 128 dims;
//   online softmax per query vector in base 2 (the reference maximum moves only when a
//     vector's maximum grows by more than 2^8, so probabilities stay at most 2^8);
//   O^T[128 dims x 32] += V^T (A operand, bf16 rows staged in LDS and read back
//     transposed, dim tile mt = dims 16mt .. 16mt + 15) x P^T: P is split into bf16 hi +
//     lo parts (about 16 significant bits), 2 x 8 dim tiles of MFMA 16x16x32 bf16 (the same precision as the sparse rows' kernel; P in
//     fp16 alone left errors of 5e-4 in the outputs, which the attention backward, fed
//     these outputs, carries into its gradients).
// Key order within the MFMA contraction is permuted as in the sparse kernel (k-slot
// 8gr + i holds key 4gr + i for i < 4 and 16 + 4gr + i - 4 otherwise), identically on
// both operands. Tiles are numbered from the end so that the longest rows start first.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

// The 12 column tiles of a (dense tile, KV head) go to CS workgroups of 12 / CS each.
// CS = 1 (8 waves): waves 0-3 take two each (tiles 2w, 2w + 1), waves 4-7 one each (tile
// 4 + w) and also stage the K/V tiles, so each SIMD (waves w and w + 4) carries three column
// tiles of MFMA work per key tile. CS = 2 (every thread staging, two key tiles in flight):
// 6 column tiles per workgroup, and twice the workgroups share each key tile (through the
// L2), for launches with too few dense tiles to fill the machine. Their 8 waves are two
// halves of 4 that take alternate key tiles (half h: tiles h, h + 2, h + 4, ...), so a
// workgroup's chain of key tiles is half as long; at the end the second half hands its
// running maxima, sums and accumulators to the first through LDS, which merges the two
// softmax states and writes the rows. In half 0 waves 0-1 take two column tiles and waves
// 2-3 one; half 1 the other way round, so every SIMD (waves w and w + 4) carries three.
constexpr int DN_KEYS = 32;
// LDS row pitches (bytes): 68 dwords for K (the 16 lanes of a 16-byte row read cover the 64
// banks), 72 for V (the transposing 8-byte reads of 32 lanes cover them)
constexpr int DN_KPITCH = 2 * HD + 16;
constexpr int DN_VPITCH = 2 * HD + 32;
constexpr int DN_KTILE = DN_KEYS * DN_KPITCH;
constexpr int DN_VTILE = DN_KEYS * DN_VPITCH;
constexpr int DN_HALF_LDS = 2 * (DN_KTILE + DN_VTILE);   // two K and two V tile buffers
constexpr int DN_STAGE_NT = DN_KEYS * 8;  // threads that stage a tile (32 bytes of K and V each)
constexpr int DN_XCH = 34;                // floats per lane and column tile handed between halves
constexpr int DN_NT = 8 * WAVE;          // threads of a workgroup (both variants)
static_assert(DN_ROWS * GQ == 16 * (4 * 2 + 4 * 1), "12 column tiles over the 8 waves");
static_assert(DN_ROWS * GQ / 2 == 16 * (2 * 2 + 2 * 1), "6 column tiles over a half's 4 waves");
static_assert(4 * WAVE == DN_STAGE_NT, "4 waves stage a tile");
static_assert(6 * DN_XCH * WAVE * 4 <= 2 * DN_HALF_LDS, "the hand-over fits the tiles");

struct DenseArgs {
    const SeqInfo *tab;
    int batch, topk;
    float scale_log2;
    const uint16_t *q, *k, *v;
    float *out, *lse;
    int32_t *sel;   // not null: the tiles also write their rows' selections
    int64_t n_tiles;
};

// The workgroup's dense tile: its sequence, first row and position, row count.
struct DenseTile {
    SeqInfo s;
    int64_t row0, t0, t_last;
    int nrows;
};

// One wave's part of a workgroup: NQ column tiles from column tile ct0 (query vectors
// 16 ct0 .. 16 (ct0 + NQ) - 1), the key loop with the workgroup's barriers (every wave runs
// the same number of iterations), and, for the staging waves, the K/V staging.
// AHEAD: key tiles whose loads the staging threads keep in flight (1 or 2).
// KS: halves of the workgroup taking alternate key tiles (1 or 2); `half` is this wave's,
// xch the LDS of the hand-over (it reuses the tile buffers) and c0 the workgroup's first
// column tile.
template <int NQ, bool STAGE, int STAGE_T0, int AHEAD, int KS>
__device__ __forceinline__ void dense_wave(const DenseArgs &a, const DenseTile &dt, int g,
                                           int ct0, uint8_t *ks0, uint8_t *vs0, int half,
                                           float *xch, int c0) {
    static_assert(AHEAD == 1 || AHEAD == 2, "one or two tiles ahead");
    static_assert(KS == 1 || KS == 2, "one or two halves");
    constexpr int STRIDE = KS * DN_KEYS;   // keys from one of this half's tiles to the next
    const int tid = threadIdx.x, l = lane_id(), gr = l >> 4, col = l & 15;
    const int64_t row0 = dt.row0, t0 = dt.t0, t_last = dt.t_last;
    const int nrows = dt.nrows;
    // this wave's rows: those of its query vectors
    const int r_lo = (16 * ct0) / GQ, r_hi = (16 * (ct0 + NQ) - 1) / GQ;

    // Q^T operands: column tile nt, lane column col -> query vector v = 16 (ct0 + nt) + col
    // = (row v / 12, head v % 12); dims 32m + 8gr .. +7 of step m
    u32x4 qb[NQ][4];
    int64_t tpos[NQ];
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt) {
        const int vq = 16 * (ct0 + nt) + col, rr = vq / GQ, hh = vq % GQ;
        const bool ok = rr < nrows;
        tpos[nt] = ok ? t0 + rr : -1;
        const uint16_t *qp = a.q + ((row0 + (ok ? rr : 0)) * HQ + g * GQ + hh) * HD + 8 * gr;
#pragma unroll
        for (int m = 0; m < 4; ++m) qb[nt][m] = ok ? load16(qp + 32 * m) : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t wave_tmax = r_lo < nrows ? t0 + min(r_hi, nrows - 1) : -1;
    const int64_t wave_tmin = t0 + r_lo;   // tiles up to here need no causal mask

    f32x4 acc[NQ][8];
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the reference maxima start at a finite floor: a vector whose keys in some tile are
    // all masked (a row before the first key of its half's tiles) then gets p = 0, not NaN
    float m_run[NQ], l_run[NQ];
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt) { m_run[nt] = -1e30f; l_run[nt] = 0.f; }

    // staging: thread STAGE_T0 + i -> (key i / 8, 32-byte piece i % 8) of the K and V rows
    const int st = tid - STAGE_T0;
    const int sk = (st >> 3) & (DN_KEYS - 1), sp = st & 7;
    const uint16_t *kbase = a.k + (int64_t)dt.s.k0 * (HKV * HD) + g * HD + 16 * sp;
    const uint16_t *vbase = a.v + (int64_t)dt.s.k0 * (HKV * HD) + g * HD + 16 * sp;
    auto load_stage = [&](int64_t j0, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
        const int64_t j = min<int64_t>(j0 + sk, t_last);   // keys past the tile's rows: masked
        kr[0] = load16(kbase + j * (HKV * HD));
        kr[1] = load16(kbase + j * (HKV * HD) + 8);
        vr[0] = load16(vbase + j * (HKV * HD));
        vr[1] = load16(vbase + j * (HKV * HD) + 8);
    };
    auto store_stage = [&](int buf, const u32x4 (&kr)[2], const u32x4 (&vr)[2]) {
        uint8_t *kd = ks0 + buf * DN_KTILE + sk * DN_KPITCH + 32 * sp;
        uint8_t *vd = vs0 + buf * DN_VTILE + sk * DN_VPITCH + 32 * sp;
        *reinterpret_cast<u32x4 *>(kd) = kr[0];
        *reinterpret_cast<u32x4 *>(kd + 16) = kr[1];
        *reinterpret_cast<u32x4 *>(vd) = vr[0];
        *reinterpret_cast<u32x4 *>(vd + 16) = vr[1];
    };

    // a half's tiles (keys j0 = base + STRIDE i) alternate between its two LDS buffers:
    // tile i + 1 is written while tile i is read, and one barrier per step makes it visible
    // (and frees tile i's buffer). The staging registers hold tile i + 1 (AHEAD = 1: loaded
    // at the start of tile i), or tiles i + 1 and i + 2 (AHEAD = 2: tile i in set i % 2,
    // tile i + 3 loaded once tile i + 1 is stored). A half with no tile left at a step
    // (the second half, when the tile count is odd) still takes part in its barrier.
    const int64_t base = (int64_t)DN_KEYS * half;
    u32x4 kr0[2], vr0[2], kr1[2], vr1[2];
    if constexpr (STAGE) {
        load_stage(base, kr0, vr0);   // past t_last (no tile for this half): clamped, unused
        store_stage(0, kr0, vr0);
        if constexpr (AHEAD == 2) {
            if (base + STRIDE <= t_last) load_stage(base + STRIDE, kr1, vr1);
            if (base + 2 * STRIDE <= t_last) load_stage(base + 2 * STRIDE, kr0, vr0);
        }
    }
    __syncthreads();
    auto step = [&](int64_t j0, int buf, u32x4 (&krn)[2], u32x4 (&vrn)[2]) {
        const bool more = j0 + STRIDE <= t_last;
        if constexpr (STAGE && AHEAD == 1)
            if (more) load_stage(j0 + STRIDE, krn, vrn);   // next tile in flight
        const uint8_t *ks = ks0 + buf * DN_KTILE;
        const uint8_t *vs = vs0 + buf * DN_VTILE;
        if (j0 <= wave_tmax) {                         // uniform over the wave
            // ---- S^T: lane (gr, col) of column tile nt holds keys j0 + 16u + 4gr + i
            float z[NQ][8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 c[NQ];
#pragma unroll
                for (int nt = 0; nt < NQ; ++nt) c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x4 ka = *reinterpret_cast<const u32x4 *>(
                        ks + (16 * u + col) * DN_KPITCH + 2 * (32 * m + 8 * gr));
#pragma unroll
                    for (int nt = 0; nt < NQ; ++nt) c[nt] = mfma_bf16_16x16x32(ka, qb[nt][m], c[nt]);
                }
                if (j0 + DN_KEYS - 1 <= wave_tmin) {   // uniform: every key visible
#pragma unroll
                    for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) z[nt][4 * u + i] = c[nt][i] * a.scale_log2;
                } else {
#pragma unroll
                    for (int nt = 0; nt < NQ; ++nt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t j = j0 + 16 * u + 4 * gr + i;
                            z[nt][4 * u + i] = j <= tpos[nt] ? c[nt][i] * a.scale_log2 : -INFINITY;
                        }
                }
            }
            // ---- V^T operands of the 8 dim tiles: lane (gr, col) of tile mt holds dim
            // 16mt + col at k-slots 8gr .. 8gr + 7 (keys 4gr + r, then 16 + 4gr + r). Two
            // transposing reads per tile: lane 4r + q of a 16-lane group addresses the 4 dims
            // 16mt + 4q .. + 3 of key 4gr + r (+ 16), and lane col receives dim 16mt + col
            // of those 4 keys.
            u32x4 va[8];
            {
                const uint8_t *vb = vs + (4 * gr + (col >> 2)) * DN_VPITCH + 8 * (col & 3);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const uint2 k0 = lds_read_tr16(vb + 32 * mt);
                    const uint2 k1 = lds_read_tr16(vb + 16 * DN_VPITCH + 32 * mt);
                    va[mt] = u32x4{k0.x, k0.y, k1.x, k1.y};
                }
            }
            // ---- per column tile: online softmax per query vector, P^T as bf16 hi + lo,
            // O^T += V^T P^T
#pragma unroll
            for (int nt = 0; nt < NQ; ++nt) {
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) mx = fmaxf(mx, z[nt][e]);
                mx = wave_max_xor_16_32(mx);
                if (mx > m_run[nt] + 8.f) {   // per lane; the column's 4 lanes agree
                    const float m_new = mx;
                    const float alpha = exp2f(m_run[nt] - m_new);
                    l_run[nt] *= alpha;
#pragma unroll
                    for (int mt = 0; mt < 8; ++mt) acc[nt][mt] *= alpha;
                    m_run[nt] = m_new;
                }
                // masked keys (z = -inf) give 0, since m_run is always finite
                float p[8], rs = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(z[nt][e] - m_run[nt]);
                    rs += p[e];
                }
                l_run[nt] += wave_sum_xor_16_32(rs);
                u32x4 ph, pl;
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const uint32_t hh = pack_bf16x2_rne(p[2 * q2], p[2 * q2 + 1]);
                    ph[q2] = hh;
                    pl[q2] = pack_bf16x2_rne(p[2 * q2] - __uint_as_float(hh << 16),
                                             p[2 * q2 + 1] - __uint_as_float(hh & 0xffff0000u));
                }
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    acc[nt][mt] = mfma_bf16_16x16x32(va[mt], ph, acc[nt][mt]);
                    acc[nt][mt] = mfma_bf16_16x16x32(va[mt], pl, acc[nt][mt]);
                }
            }
        }
        if constexpr (STAGE) {
            if (more) store_stage(buf ^ 1, krn, vrn);   // tile i + 1 into the buffer of i - 1
            if constexpr (AHEAD == 2)
                if (j0 + 3 * STRIDE <= t_last) load_stage(j0 + 3 * STRIDE, krn, vrn);
        }
        __syncthreads();   // tile i + 1 staged, every wave done with tile i
    };
    // steps: the first half's tile count, the same in both halves
    const int64_t n_steps = (t_last / DN_KEYS + KS) / KS;
    if constexpr (AHEAD == 1) {
        int buf = 0;
        for (int64_t i = 0; i < n_steps; ++i, buf ^= 1) step(base + STRIDE * i, buf, kr0, vr0);
    } else {
        for (int64_t i = 0; i < n_steps; i += 2) {
            step(base + STRIDE * i, 0, kr1, vr1);
            if (i + 1 >= n_steps) break;
            step(base + STRIDE * (i + 1), 1, kr0, vr0);
        }
    }

    // two halves: the second hands its state to the first (the tile buffers are free after
    // the last step's barrier), which merges: m = max(m0, m1), each half's sum and
    // accumulators scaled by 2^(m_h - m). Layout: [column tile - c0][34 floats][64 lanes].
    if constexpr (KS == 2) {
        if (half == 1) {
#pragma unroll
            for (int nt = 0; nt < NQ; ++nt) {
                float *x = xch + (ct0 + nt - c0) * DN_XCH * WAVE + l;
#pragma unroll
                for (int e = 0; e < 32; ++e) x[e * WAVE] = acc[nt][e >> 2][e & 3];
                x[32 * WAVE] = m_run[nt];
                x[33 * WAVE] = l_run[nt];
            }
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int nt = 0; nt < NQ; ++nt) {
            const float *x = xch + (ct0 + nt - c0) * DN_XCH * WAVE + l;
            const float m1 = x[32 * WAVE], m = fmaxf(m_run[nt], m1);
            const float s0 = exp2f(m_run[nt] - m), s1 = exp2f(m1 - m);
            l_run[nt] = l_run[nt] * s0 + x[33 * WAVE] * s1;
#pragma unroll
            for (int e = 0; e < 32; ++e)
                acc[nt][e >> 2][e & 3] = acc[nt][e >> 2][e & 3] * s0 + x[e * WAVE] * s1;
            m_run[nt] = m;
        }
    }

    // lane (gr, col), column tile nt: acc[nt][mt][i] = O[vector 16(ct0 + nt) + col]
    // [dim 16mt + 4gr + i]
#pragma unroll
    for (int nt = 0; nt < NQ; ++nt) {
        const int vq = 16 * (ct0 + nt) + col, rr = vq / GQ, hh = vq % GQ;
        if (rr >= nrows) continue;
        const int64_t row = row0 + rr;
        const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
        float *o = a.out + (row * HQ + g * GQ + hh) * HD;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<f32x4 *>(o + 16 * mt + 4 * gr) = acc[nt][mt] * inv;
        if (a.lse && gr == 0)
            a.lse[row * HQ + g * GQ + hh] =
                l_run[nt] > 0.f ? m_run[nt] * 0.69314718055994531f + logf(l_run[nt]) : -INFINITY;
    }
}

template <int CS>
__global__ void __launch_bounds__(DN_NT) attend_dense_kernel(DenseArgs a) {
    // CS = 1: two tile buffers of K and of V; CS = 2: two of each per half
    __shared__ __attribute__((aligned(16))) uint8_t lds[CS * DN_HALF_LDS];
    const int g = blockIdx.y / CS, part = blockIdx.y % CS;
    const int64_t tile = a.n_tiles - 1 - (int64_t)blockIdx.x;
    const int sb = find_seq(a.batch, tile, [&](int i) { return (int64_t)a.tab[i].dtile0; });
    DenseTile dt;
    dt.s = a.tab[sb];
    const int64_t nd = dense_rows_of(dt.s.L, dt.s.nq, a.topk);
    const int64_t i0 = (tile - dt.s.dtile0) * DN_ROWS;       // first dense row of the tile
    dt.t0 = (int64_t)dt.s.L - dt.s.nq + i0;                   // its position
    dt.nrows = (int)min<int64_t>(DN_ROWS, nd - i0);
    dt.row0 = dt.s.q0 + i0;
    dt.t_last = dt.t0 + dt.nrows - 1;
    // a call with no scored rows leaves the selections to this kernel: a dense row keeps
    // every visible block (ascending), then -1 (one workgroup of the tile writes them)
    if (a.sel && blockIdx.y == 0) {
        for (int e = threadIdx.x; e < dt.nrows * a.topk; e += DN_NT) {
            const int rr = e / a.topk, i = e - rr * a.topk;
            a.sel[(dt.row0 + rr) * a.topk + i] = i < nvis_of(dt.t0 + rr) ? i : -1;
        }
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    if constexpr (CS == 1) {
        uint8_t *ks = lds, *vs = lds + 2 * DN_KTILE;
        if (w < 4) dense_wave<2, false, 4 * WAVE, 1, 1>(a, dt, g, 2 * w, ks, vs, 0, nullptr, 0);
        else dense_wave<1, true, 4 * WAVE, 1, 1>(a, dt, g, 4 + w, ks, vs, 0, nullptr, 0);
    } else {
        const int c0 = 6 * part, half = w >> 2, wl = w & 3;
        uint8_t *ks = lds + half * DN_HALF_LDS, *vs = ks + 2 * DN_KTILE;
        float *xch = reinterpret_cast<float *>(lds);
        if (half == 0) {
            if (wl < 2) dense_wave<2, true, 0, 2, 2>(a, dt, g, c0 + 2 * wl, ks, vs, 0, xch, c0);
            else dense_wave<1, true, 0, 2, 2>(a, dt, g, c0 + 2 + wl, ks, vs, 0, xch, c0);
        } else {
            if (wl < 2)
                dense_wave<1, true, 4 * WAVE, 2, 2>(a, dt, g, c0 + 4 + wl, ks, vs, 1, xch, c0);
            else
                dense_wave<2, true, 4 * WAVE, 2, 2>(a, dt, g, c0 + 2 * (wl - 2), ks, vs, 1, xch,
                                                    c0);
        }
    }
}

hipError_t launch_attend_dense(const SeqInfo *tab, int batch, int topk, float scale,
                               const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               float *out, float *lse, int32_t *sel, int64_t n_tiles,
                               hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    DenseArgs a;
    a.tab = tab; a.batch = batch; a.topk = topk;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.sel = sel; a.n_tiles = n_tiles;
    trace_before(15, st);
    // fewer (dense tile, KV head) workgroups than CUs: each tile's column tiles go to two
    if (n_tiles * HKV < 256)
        hipLaunchKernelGGL(attend_dense_kernel<2>, dim3((unsigned)n_tiles, HKV * 2),
                           dim3(DN_NT), 0, st, a);
    else
        hipLaunchKernelGGL(attend_dense_kernel<1>, dim3((unsigned)n_tiles, HKV),
                           dim3(DN_NT), 0, st, a);
    return trace_after(st, hipGetLastError());
}

}  // namespace qsa
