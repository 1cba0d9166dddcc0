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
// Workgroup = (dense tile of DN_ROWS = 16 rows, KV head g); 4 waves of 4 rows each.
// A wave's 48 query vectors (4 rows x 12 heads) are 3 MFMA column tiles of 16. Per
// tile of 32 keys:
//   S^T[32 keys x 48] = K (A operand from LDS, bf16) x Q^T (B operand, registers):
//     3 column tiles x 2 key halves x 4 steps of MFMA 16x16x32 over the 128 dims;
//   online softmax per query vector in base 2 (the reference maximum moves only when a
//     vector's maximum grows by more than 2^8, so probabilities stay at most 2^8);
//   O^T[128 dims x 48] += V^T (A operand, fp16 rows staged in LDS) x P^T (fp16):
//     8 dim tiles x 3 column tiles of MFMA 16x16x32 f16. V is converted bf16 -> fp16
//     once, when the workgroup stages it (bf16 values of N(0,1)-sized data are exact
//     in fp16 unless tinier than 2^-14, where the fp16 step is 2^-24); P in fp16 keeps
//     11 bits.
// Key order within the MFMA contraction is permuted as in the sparse kernel (k-slot
// 8gr + i holds key 4gr + i for i < 4 and 16 + 4gr + i - 4 otherwise), identically on
// both operands. Tiles are numbered from the end so that the longest rows start first.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values as one word of fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
    const f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
}

constexpr int DN_NT = 256;
constexpr int DN_KEYS = 32;
constexpr int DN_NQ = 3;                  // column tiles of 16 query vectors per wave
constexpr int DN_PITCH = 2 * HD + 16;     // LDS row pitch (bytes) of the K and V tiles
static_assert(DN_ROWS == 4 * (DN_NT / WAVE), "4 rows per wave");
static_assert(DN_NQ * 16 == 4 * GQ, "a wave's 4 rows x 12 heads fill 3 column tiles");

struct DenseArgs {
    const SeqInfo *tab;
    int batch, topk;
    float scale_log2;
    const uint16_t *q, *k, *v;
    float *out, *lse;
    int64_t n_tiles;
};

__global__ void __launch_bounds__(DN_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
attend_dense_kernel(DenseArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[DN_KEYS * DN_PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t vs[DN_KEYS * DN_PITCH];
    const int g = blockIdx.y;
    const int64_t tile = a.n_tiles - 1 - (int64_t)blockIdx.x;
    const int sb = find_seq(a.batch, tile, [&](int i) { return (int64_t)a.tab[i].dtile0; });
    const SeqInfo s = a.tab[sb];
    const int64_t nd = dense_rows_of(s.L, s.nq, a.topk);
    const int64_t i0 = (tile - s.dtile0) * DN_ROWS;          // first dense row of the tile
    const int64_t t0 = (int64_t)s.L - s.nq + i0;              // its position
    const int nrows = (int)min<int64_t>(DN_ROWS, nd - i0);
    const int64_t row0 = s.q0 + i0;
    const int64_t t_last = t0 + nrows - 1;
    const int tid = threadIdx.x, w = tid / WAVE, l = lane_id(), gr = l >> 4, col = l & 15;
    const int wrows = min(4, nrows - 4 * w);                  // this wave's rows (may be <= 0)

    // Q^T operands: column tile nt, lane column col -> query vector 16nt + col = (row
    // 4w + v / 12, head v % 12); dims 32m + 8gr .. +7 of step m
    u32x4 qb[DN_NQ][4];
    int64_t tpos[DN_NQ];
#pragma unroll
    for (int nt = 0; nt < DN_NQ; ++nt) {
        const int vq = 16 * nt + col, rr = vq / GQ, hh = vq % GQ;
        const bool ok = rr < wrows;
        tpos[nt] = ok ? t0 + 4 * w + rr : -1;
        const uint16_t *qp =
            a.q + ((row0 + (ok ? 4 * w + rr : 0)) * HQ + g * GQ + hh) * HD + 8 * gr;
#pragma unroll
        for (int m = 0; m < 4; ++m) qb[nt][m] = ok ? load16(qp + 32 * m) : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t wave_tmax = wrows > 0 ? t0 + 4 * w + wrows - 1 : -1;

    f32x4 acc[DN_NQ][8];
#pragma unroll
    for (int nt = 0; nt < DN_NQ; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[DN_NQ], l_run[DN_NQ];
#pragma unroll
    for (int nt = 0; nt < DN_NQ; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }

    // staging: thread -> (key tid / 8, 32-byte piece tid % 8) of the K and V rows
    const int sk = tid >> 3, sp = tid & 7;
    const uint16_t *kbase = a.k + (int64_t)s.k0 * (HKV * HD) + g * HD + 16 * sp;
    const uint16_t *vbase = a.v + (int64_t)s.k0 * (HKV * HD) + g * HD + 16 * sp;
    auto load_stage = [&](int64_t j0, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
        const int64_t j = min<int64_t>(j0 + sk, t_last);   // keys past the tile's rows: masked
        kr[0] = load16(kbase + j * (HKV * HD));
        kr[1] = load16(kbase + j * (HKV * HD) + 8);
        vr[0] = load16(vbase + j * (HKV * HD));
        vr[1] = load16(vbase + j * (HKV * HD) + 8);
    };
    auto store_stage = [&](const u32x4 (&kr)[2], const u32x4 (&vr)[2]) {
        uint8_t *kd = ks + sk * DN_PITCH + 32 * sp;
        uint8_t *vd = vs + sk * DN_PITCH + 32 * sp;
        *reinterpret_cast<u32x4 *>(kd) = kr[0];
        *reinterpret_cast<u32x4 *>(kd + 16) = kr[1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_f16(bf16_lo(vr[h][e]), bf16_hi(vr[h][e]));
            *reinterpret_cast<u32x4 *>(vd + 16 * h) = o;
        }
    };

    u32x4 kr[2], vr[2];
    load_stage(0, kr, vr);
    store_stage(kr, vr);
    __syncthreads();
    for (int64_t j0 = 0; j0 <= t_last; j0 += DN_KEYS) {
        const bool more = j0 + DN_KEYS <= t_last;
        if (more) load_stage(j0 + DN_KEYS, kr, vr);   // next tile in flight during compute
        if (j0 <= wave_tmax) {                         // uniform over the wave
            // ---- S^T: lane (gr, col) of column tile nt holds keys j0 + 16u + 4gr + i
            float z[DN_NQ][8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 c[DN_NQ];
#pragma unroll
                for (int nt = 0; nt < DN_NQ; ++nt) c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const u32x4 ka = *reinterpret_cast<const u32x4 *>(
                        ks + (16 * u + col) * DN_PITCH + 2 * (32 * m + 8 * gr));
#pragma unroll
                    for (int nt = 0; nt < DN_NQ; ++nt) c[nt] = mfma_bf16_16x16x32(ka, qb[nt][m], c[nt]);
                }
#pragma unroll
                for (int nt = 0; nt < DN_NQ; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t j = j0 + 16 * u + 4 * gr + i;
                        z[nt][4 * u + i] = j <= tpos[nt] ? c[nt][i] * a.scale_log2 : -INFINITY;
                    }
            }
            // ---- online softmax per query vector (column), P^T in fp16
            u32x4 ph[DN_NQ];
#pragma unroll
            for (int nt = 0; nt < DN_NQ; ++nt) {
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
                float p[8], rs = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = z[nt][e] == -INFINITY ? 0.f : exp2f(z[nt][e] - m_run[nt]);
                    rs += p[e];
                }
                l_run[nt] += wave_sum_xor_16_32(rs);
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) ph[nt][q2] = pack_f16(p[2 * q2], p[2 * q2 + 1]);
            }
            // ---- O^T += V^T P^T: lane rows are dims 8col + mt, its k-slot keys as above
            u32x4 vrow[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vrow[e] = *reinterpret_cast<const u32x4 *>(
                    vs + (16 * (e >> 2) + 4 * gr + (e & 3)) * DN_PITCH + 16 * col);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                u32x4 va;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    va[kk] = bf16_pair(vrow[2 * kk][mt >> 1], vrow[2 * kk + 1][mt >> 1], mt & 1);
#pragma unroll
                for (int nt = 0; nt < DN_NQ; ++nt)
                    acc[nt][mt] = mfma_f16_16x16x32(va, ph[nt], acc[nt][mt]);
            }
        }
        __syncthreads();   // every wave is done with this tile
        if (more) store_stage(kr, vr);
        __syncthreads();
    }

    // lane (gr, col), column tile nt: acc[nt][mt][i] = O[vector 16nt + col][dim 8(4gr+i) + mt]
#pragma unroll
    for (int nt = 0; nt < DN_NQ; ++nt) {
        const int vq = 16 * nt + col, rr = vq / GQ, hh = vq % GQ;
        if (rr >= wrows) continue;
        const int64_t row = row0 + 4 * w + rr;
        const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
        float *o = a.out + (row * HQ + g * GQ + hh) * HD;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 8 * (4 * gr + i);
            const f32x4 lo4 = {acc[nt][0][i] * inv, acc[nt][1][i] * inv, acc[nt][2][i] * inv,
                               acc[nt][3][i] * inv};
            const f32x4 hi4 = {acc[nt][4][i] * inv, acc[nt][5][i] * inv, acc[nt][6][i] * inv,
                               acc[nt][7][i] * inv};
            *reinterpret_cast<f32x4 *>(o + d0) = lo4;
            *reinterpret_cast<f32x4 *>(o + d0 + 4) = hi4;
        }
        if (a.lse && gr == 0)
            a.lse[row * HQ + g * GQ + hh] =
                l_run[nt] > 0.f ? m_run[nt] * 0.69314718055994531f + logf(l_run[nt]) : -INFINITY;
    }
}

hipError_t launch_attend_dense(const SeqInfo *tab, int batch, int topk, float scale,
                               const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               float *out, float *lse, int64_t n_tiles, hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    DenseArgs a;
    a.tab = tab; a.batch = batch; a.topk = topk;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.n_tiles = n_tiles;
    trace_before(15, st);
    hipLaunchKernelGGL(attend_dense_kernel, dim3((unsigned)n_tiles, HKV), dim3(DN_NT), 0, st, a);
    return trace_after(st, hipGetLastError());
}

}  // namespace qsa
