// qsa_device.h -- device-side constants, types and helpers shared by the QSA
// kernels (gfx950, wave64). Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// The layer's fixed shape: 24 query heads over 2 key/value heads of width 128
// ("24 query heads paired with only 2 key-value (KV) heads", axbrief.com,
// "Shifting from Tokens to Micro-Blocks"), a 4-head x 64 indexer, 4-token
// micro-blocks (hellomarvisaitoday.com, FAQ) and a budget of at most 512 blocks
// (elzobrito.github.io, "Linear attention carries the stream; sparse attention
// retrieves detail").
constexpr int HQ = 24;
constexpr int HKV = 2;
constexpr int HD = 128;
constexpr int GQ = HQ / HKV;   // query heads per key/value head
constexpr int HI = 4;
constexpr int DI = 64;
constexpr int BS = 4;
constexpr int KMAX = 512;
constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Per-sequence bookkeeping, built once per call into the workspace.
struct SeqInfo {
    int32_t q0;     // first query row
    int32_t nq;     // query rows (its last nq tokens)
    int32_t k0;     // first key row
    int32_t L;      // length
    int32_t blk0;   // first compressed-block row
    int32_t tile0;  // first score tile (4 query rows that need scoring)
    int64_t s0;     // first score slot
};

// Host-computed row and tile tables passed as kernel arguments when a call has few
// query rows (decode): no table kernel and no device-side sequence lookup.
constexpr int DEC_MAX = 64;
struct DecRow {
    int32_t k0;     // first key row of the row's sequence
    int32_t t;      // position of the query token
    int32_t blk0;   // first compressed-block row of the sequence
    int32_t pad;
    int64_t slot;   // first score slot of the row (rows with nvis > topk)
};
struct DecTile {
    int32_t row0;   // first query row of the tile
    int32_t nrows;  // 1..4 consecutive rows of one sequence
    int32_t new_lo; // sequence-local blocks [new_lo, new_hi) hold a query token
    int32_t new_hi;
};
struct DecodeTables {
    DecRow row[DEC_MAX];
    DecTile tile[DEC_MAX];
};

// What a kernel needs to know about one query row.
struct RowView {
    int64_t k0, t, blk0, slot;
};

// ---------------------------------------------------------------- visibility

// Blocks whose 4 tokens are all at or before position t.
__device__ __forceinline__ int64_t nvis_of(int64_t t) { return (t + 1) / BS; }

// F(t) = sum_{u<t} nvis(u): score slots used by positions 0..t-1.
__device__ __forceinline__ int64_t slots_before(int64_t t) {
    int64_t m = t / 4, r = t % 4;
    return 2 * m * (m - 1) + m * (r + 1);
}

// First position whose row needs scoring (more visible blocks than the budget).
__device__ __forceinline__ int64_t first_scored_pos(int32_t L, int32_t nq, int32_t topk) {
    int64_t a = (int64_t)L - nq, b = 4 * (int64_t)topk + 3;
    return a > b ? a : b;
}

// Largest b with key(b) <= x over a non-decreasing table (x >= key(0)).
template <typename F>
__device__ __forceinline__ int upper_index(int n, int64_t x, F key) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (key(mid) <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Same, with one round of loads: lane i reads entry i, i+64, ... (up to 1024
// entries) and the count of entries <= x comes from ballots. Wave-uniform result.
template <typename F>
__device__ __forceinline__ int find_seq(int n, int64_t x, F key) {
    if (n > 1024) return upper_index(n, x, key);
    const int l = __lane_id();
    int cnt = 0;
    for (int j0 = 0; j0 < n; j0 += 256) {   // 4 unconditional loads per round
        int64_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = key(min(j0 + 64 * j + l, n - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            cnt += __popcll(__ballot(j0 + 64 * j + l < n && v[j] <= x));
    }
    return cnt - 1;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// double -> bf16 bits, round to nearest even, overflow to infinity. bf16 keeps 8
// significant bits and the fp32 exponent range: the quantum of |x| in [2^e, 2^e+1)
// is 2^(max(e,-126)-7).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e = (int)((u >> 52) & 0x7ff) - 1023;
    int qe = (e < -126 ? -126 : e) - 7;
    double r = ldexp(rint(ldexp(a, -qe)), qe);
    if (r >= 0x1p128) return sign | 0x7f80u;
    return sign | (__float_as_uint((float)r) >> 16);
}

// Order-preserving key of an fp32 score: larger score <-> larger key; -0 == +0.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave / block

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        T o = __shfl_up(v, d);
        if (l >= d) v += o;
    }
    return v;
}

// Inclusive prefix sum of int32 over a wave with DPP row shifts and row broadcasts
// (4 shifts within each 16-lane row, then rows 1/3 add row 0/2's last lane and rows
// 2/3 add lane 31).
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Block-wide exclusive prefix sum of int32 with two barriers; scratch: NT/64 ints.
template <int NT>
__device__ __forceinline__ int32_t block_excl_scan_i32(int32_t v, int32_t *scratch,
                                                       int32_t *total) {
    constexpr int NW = NT / WAVE;
    const int w = threadIdx.x / WAVE;
    const int32_t inc = wave_incl_scan_i32(v);
    if (lane_id() == WAVE - 1) scratch[w] = inc;
    __syncthreads();
    int32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int32_t x = scratch[i];
        before += i < w ? x : 0;
        tot += x;
    }
    *total = tot;
    __syncthreads();  // scratch is rewritten by the next call
    return before + inc - v;
}

// Block-wide exclusive prefix sum; `scratch` holds >= nwaves+1 elements of T.
// Returns the exclusive prefix and writes the block total to *total.
template <typename T, int NT>
__device__ __forceinline__ T block_excl_scan(T v, T *scratch, T *total) {
    constexpr int NW = NT / WAVE;
    const int w = threadIdx.x / WAVE, l = lane_id();
    T inc = wave_incl_scan(v);
    if (l == WAVE - 1) scratch[w] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        T run = 0;
        for (int i = 0; i < NW; ++i) { T x = scratch[i]; scratch[i] = run; run += x; }
        scratch[NW] = run;
    }
    __syncthreads();
    T r = scratch[w] + inc - v;
    *total = scratch[NW];
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------- selection

// Digit plans of the radix select over 32-bit order keys (most significant first).
// WIDE: 11 + 11 + 10 bits (2048-bin histograms) for long rows; NARROW: 4 x 8 bits.
struct DigitPlan {
    int n;
    int shift[4];
    int width[4];
};
constexpr DigitPlan kWide = {3, {21, 10, 0, 0}, {11, 11, 10, 0}};
constexpr int kHistBins = 2048;
constexpr DigitPlan kNarrow = {4, {24, 16, 8, 0}, {8, 8, 8, 8}};

// The k-th largest of n keys (1 <= k <= n) by a most-significant-digit radix select
// with LDS histograms. Returns theta (that key) and `need`, how many keys equal to
// theta belong to the k largest (ties go to the lowest positions). All NT threads
// of the workgroup must call it. hist: LDS, 2^max(width) entries; scan_sh: LDS,
// NT/64+1 entries; found: LDS, 2 entries.
template <int NT, typename KeyPtr>
__device__ __forceinline__ void radix_kth(KeyPtr keys, int64_t n, int64_t k,
                                          const DigitPlan &plan, uint32_t *hist,
                                          int32_t *scan_sh, uint32_t *found,
                                          uint32_t *theta_out, int64_t *need_out) {
    static_assert(NT == 256, "bin ownership assumes 256 threads");
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int64_t need = k;
#pragma unroll 1
    for (int pass = 0; pass < plan.n; ++pass) {
        const int shift = plan.shift[pass], nb = 1 << plan.width[pass];
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int i = tid; i < nb; i += NT) hist[i] = 0u;
        if (tid == 0) { found[0] = 0u; found[1] = 0u; }
        __syncthreads();
        // keys are read in batches of 8 before their atomics, so the loads overlap
        for (int64_t i0 = tid; i0 < n; i0 += 8 * NT) {
            uint32_t kk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t i = i0 + (int64_t)e * NT;
                kk[e] = i < n ? keys[i] : 0u;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t i = i0 + (int64_t)e * NT;
                if (i < n && (kk[e] & pmask) == prefix)
                    atomicAdd(&hist[(kk[e] >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        // thread j owns `per` consecutive bins ending at nb - per*j (highest bins first)
        const int per = nb / NT;
        const int top = nb - per * tid;
        int32_t local = 0;
        for (int i = 1; i <= per; ++i) local += (int32_t)hist[top - i];
        int32_t tot;
        const int64_t above = block_excl_scan_i32<NT>(local, scan_sh, &tot);
        if (above < need && need <= above + (int64_t)local) {
            int64_t run = above;
            for (int i = 1; i <= per; ++i) {
                const int bin = top - i;
                if (run + hist[bin] >= need) {
                    found[0] = (uint32_t)bin;
                    found[1] = (uint32_t)run;
                    break;
                }
                run += hist[bin];
            }
        }
        __syncthreads();
        need -= (int64_t)found[1];
        prefix |= found[0] << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    *theta_out = prefix;
    *need_out = need;
}

// Ordered pass after radix_kth: walks the n keys in position order and keeps every
// key above theta and the first `need` keys equal to it, writing their ids
// (idx[i], or i when idx is null, plus idx_base) and optionally keys to consecutive
// output slots
// (at most cap). Optionally counts kept entries per group of `group` positions in
// LDS (group_cnt). Returns the number kept. All NT threads must call it.
template <int NT, int PER, typename KeyPtr, typename IdxPtr>
__device__ __forceinline__ int64_t emit_kept(KeyPtr keys, IdxPtr idx,
                                             int64_t n, uint32_t theta, int64_t need,
                                             int32_t *out_idx, uint32_t *out_key, int64_t cap,
                                             int32_t *scan_sh, uint32_t *group_cnt,
                                             int group, int32_t idx_base = 0) {
    const int tid = threadIdx.x;
    int64_t run_eq = 0, run_sel = 0;
#pragma unroll 1
    for (int64_t base = 0; base < n; base += (int64_t)NT * PER) {
        const int64_t i0 = base + (int64_t)tid * PER;
        uint32_t kk[PER];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const bool valid = i0 + e < n;
            kk[e] = valid ? keys[i0 + e] : 0u;
            n_eq += (valid && kk[e] == theta);
        }
        int32_t tot_eq;
        int64_t eq_run = run_eq + block_excl_scan_i32<NT>(n_eq, scan_sh, &tot_eq);
        int n_take = 0;
        uint32_t take_mask = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const bool valid = i0 + e < n;
            const bool eq = valid && kk[e] == theta;
            const bool take = (valid && kk[e] > theta) || (eq && eq_run < need);
            eq_run += eq;
            if (take) { take_mask |= 1u << e; ++n_take; }
        }
        int32_t tot_take;
        int64_t pos = run_sel + block_excl_scan_i32<NT>(n_take, scan_sh, &tot_take);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (take_mask & (1u << e)) {
                if (pos < cap) {
                    out_idx[pos] = (idx ? idx[i0 + e] : (int32_t)(i0 + e)) + idx_base;
                    if (out_key) out_key[pos] = kk[e];
                }
                if (group_cnt) atomicAdd(&group_cnt[(i0 + e) / group], 1u);
                ++pos;
            }
        }
        run_eq += tot_eq;
        run_sel += tot_take;
    }
    return run_sel;
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace qsa
