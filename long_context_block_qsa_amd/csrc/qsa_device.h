// qsa_device.h -- device-side constants, types and helpers shared by the QSA
// kernels (gfx950, wave64). Internal to the library.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// The layer's fixed shape: 24 query heads sharing 2 key/value heads of width 128
// (axbrief.com, "Shifting from Tokens to Micro-Blocks"), a 4-head x 64 indexer,
// 4-token micro-blocks (hellomarvisaitoday.com, FAQ) and a budget of at most 512
// blocks (elzobrito.github.io, "Linear attention carries the stream; sparse attention
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    int32_t dtile0; // first dense tile (DN_ROWS query rows that keep every visible block)
    int32_t pad_;
};

// Query rows per tile of the dense-regime attention (rows with no more visible blocks
// than the budget attend every token up to their own position).
constexpr int DN_ROWS = 16;

// Per-sequence table of the attention backward. Key blocks are the ceil(L/4) groups of
// 4 tokens of a sequence (the last one may be partial: it is only attended raw); query
// rows are cut into chunks of BWD_CH consecutive rows of one sequence.
constexpr int BWD_CH = 256;
constexpr int BWD_CAP = 16384;  // key blocks counted per LDS pass of the index kernels
constexpr int BWD_WCH = 32;     // row chunks per window of the dK/dV kernel (8192 rows)
struct BwdSeq {
    int32_t q0, nq, k0, L;
    int32_t kb0;   // first key block (global numbering over all sequences)
    int32_t nkb;   // ceil(L / 4)
    int32_t ch0;   // first row chunk
    int32_t nch;   // ceil(nq / BWD_CH)
    int64_t m0;    // first entry of the sequence's [nch][nkb] count matrix
};

// Host-computed row and tile tables passed as kernel arguments when a call has few
// query rows (decode): no table kernel and no device-side sequence lookup.
constexpr int DEC_MAX = 64;

// Control block at the start of the workspace: counters through which workgroups of
// one kernel hand work to each other. Zero before a call; every call leaves it zero.
//   [0, 64)    per score tile: chunks (or chunk groups) merged so far
//   [64, 320)  per (tile, group of chunks): chunks scored so far
//   [320, 384) per query row: the row needs the exact selection
constexpr int CTL_TILE = 0;
constexpr int CTL_GROUP = 64;
constexpr int CTL_EXACT = 320;
constexpr int CTL_WORDS = 1024;
struct DecRow {
    int32_t k0;     // first key row of the row's sequence
    int32_t t;      // position of the query token
    int32_t blk0;   // first compressed-block row of the sequence
    int32_t tile;   // score tile of the row (-1: not scored)
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

// Query rows of a sequence in the dense regime: positions L - nq .. first scored - 1.
__device__ __forceinline__ int64_t dense_rows_of(int32_t L, int32_t nq, int32_t topk) {
    const int64_t ts = first_scored_pos(L, nq, topk), e = ts < L ? ts : L;
    const int64_t n = e - ((int64_t)L - nq);
    return n > 0 ? n : 0;
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

// Two fp32 values as one word of bf16 (low half = a), round to nearest even: the
// gfx950 conversion instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
    const bf16x2_t h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Third word of a raw buffer resource (gfx9 family: untyped 32-bit data, no swizzle).
constexpr int kBufWord3 = 0x00020000;

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

// Words of the `found` LDS array radix_kth needs with NT threads.
template <int NT> constexpr int radix_found_words() { return 2 + 2 * (NT / 64); }

// The k-th largest of n keys (1 <= k <= n) by a most-significant-digit radix select
// with LDS histograms. Returns theta (that key) and `need`, how many keys equal to
// theta belong to the k largest (ties go to the lowest positions). Each pass also
// ORs and ANDs the keys it counts: when they agree on every bit below the pass's digit,
// the bin found holds a single key value and the select stops there (scores of small-
// integer indexer data leave the low bits of their keys constant, so the last of the
// three passes is skipped). All NT threads of the workgroup must call it. hist: LDS,
// 2^max(width) entries; scan_sh: LDS, NT/64+1 entries; found: LDS,
// radix_found_words<NT>() entries.
template <int NT, typename KeyPtr>
__device__ __forceinline__ void radix_kth(KeyPtr keys, int64_t n, int64_t k,
                                          const DigitPlan &plan, uint32_t *hist,
                                          int32_t *scan_sh, uint32_t *found,
                                          uint32_t *theta_out, int64_t *need_out) {
    static_assert(NT == 256, "bin ownership assumes 256 threads");
    constexpr int NW = NT / WAVE;
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
        uint32_t k_or = 0u, k_and = 0xffffffffu;
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
                if (i < n && (kk[e] & pmask) == prefix) {
                    atomicAdd(&hist[(kk[e] >> shift) & dmask], 1u);
                    k_or |= kk[e];
                    k_and &= kk[e];
                }
            }
        }
#pragma unroll
        for (int d = 1; d < WAVE; d <<= 1) {
            k_or |= (uint32_t)__shfl_xor((int)k_or, d);
            k_and &= (uint32_t)__shfl_xor((int)k_and, d);
        }
        if (lane_id() == 0) {
            found[2 + tid / WAVE] = k_or;
            found[2 + NW + tid / WAVE] = k_and;
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
        uint32_t b_or = 0u, b_and = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            b_or |= found[2 + i];
            b_and &= found[2 + NW + i];
        }
        __syncthreads();
        const uint32_t low = (1u << shift) - 1u;   // bits below this pass's digit
        if (((b_or ^ b_and) & low) == 0u) {        // uniform: every thread read the same words
            prefix |= b_or & low;
            break;
        }
    }
    *theta_out = prefix;
    *need_out = need;
}

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Ordered pass after radix_kth: keeps every key above theta and the first `need` keys
// equal to it (by position), writing their positions in ascending order to out_idx (at
// most cap); returns the number kept. Thread t reads element e of a batch at position
// base + e*NT + t, so every load instruction reads consecutive keys. A kept key's slot is
// its rank in position order: the kept keys of earlier elements, of earlier waves at the
// same element, and of lower lanes (a ballot). Per-(wave, element) counts of equal and of
// kept keys go through `cnt` (LDS, 4 * (NT/64) * PER ints; two barriers per batch, the
// two halves used by alternate batches). All NT threads must call it.
template <int NT, int PER, typename KeyPtr>
__device__ __forceinline__ int64_t emit_kept(KeyPtr keys, int64_t n, uint32_t theta,
                                             int64_t need, int32_t *out_idx, int64_t cap,
                                             int32_t *cnt) {
    constexpr int NW = NT / WAVE;
    static_assert(PER <= WAVE, "one lane per element writes the wave's counts");
    const int tid = threadIdx.x, w = tid / WAVE, l = lane_id();
    int64_t run_eq = 0, run_sel = 0;
    int par = 0;
#pragma unroll 1
    for (int64_t base = 0; base < n; base += (int64_t)NT * PER, par ^= 1) {
        int32_t *ceq = cnt + par * 2 * NW * PER;   // [wave][element]: keys equal to theta
        int32_t *ctk = ceq + NW * PER;             // [wave][element]: kept keys
        uint32_t kk[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int64_t i = base + (int64_t)e * NT + tid;
            kk[e] = i < n ? keys[i] : 0u;
        }
        unsigned long long beq[PER];
        int v = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            beq[e] = __ballot(base + (int64_t)e * NT + tid < n && kk[e] == theta);
            v = l == e ? (int)__popcll(beq[e]) : v;
        }
        if (l < PER) ceq[w * PER + l] = v;
        __syncthreads();
        // equal keys before each element of this lane; then which keys are kept
        int64_t eq_pre = run_eq;
        int eq_tot = 0;
        unsigned long long btk[PER];
        v = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            int before_w = 0, col = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int c = ceq[i * PER + e];
                before_w += i < w ? c : 0;
                col += c;
            }
            const bool valid = base + (int64_t)e * NT + tid < n;
            const bool eq = (beq[e] >> l) & 1ull;
            const bool take = (valid && kk[e] > theta) ||
                              (eq && eq_pre + before_w + lanes_below(beq[e]) < need);
            btk[e] = __ballot(take);
            v = l == e ? (int)__popcll(btk[e]) : v;
            eq_pre += col;
            eq_tot += col;
        }
        if (l < PER) ctk[w * PER + l] = v;
        __syncthreads();
        int64_t pos = run_sel;
        int tk_tot = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            int before_w = 0, col = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const int c = ctk[i * PER + e];
                before_w += i < w ? c : 0;
                col += c;
            }
            if ((btk[e] >> l) & 1ull) {
                const int64_t slot = pos + before_w + lanes_below(btk[e]);
                if (slot < cap) out_idx[slot] = (int32_t)(base + (int64_t)e * NT + tid);
            }
            pos += col;
            tk_tot += col;
        }
        run_eq += eq_tot;
        run_sel += tk_tot;
    }
    return run_sel;
}

// ---------------------------------------------------------------- wave-level select

// Workgroup barrier that orders LDS only (outstanding global stores are not waited for).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS accesses (lanes exchange data through LDS).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
}

// Lanes below this one in a ballot mask.

// Wave-wide max / min of uint32 with DPP row shifts and row broadcasts (the result is
// complete in lane 63 and read from there).
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}

// Exact top-k (1 <= k) of the valid keys one wave holds in registers, with no
// workgroup barrier: lane l holds positions PER*l .. PER*l+PER-1 (REG_MAJOR: positions
// e*64 + l), ok[e] marks the valid ones. Order: key descending, equal keys by
// ascending position. Radix select with
// 8-bit digits over a wave-private 256-bin LDS histogram (`hist`), starting at the
// highest bit where the keys differ and stopping as soon as the bin that holds the
// k-th key is kept whole; when the digits run out, that bin is one key value and its
// keys are kept by position. Returns this lane's kept mask (bit e); all valid keys
// when there are at most k.
template <int PER, bool REG_MAJOR = false>
__device__ __forceinline__ uint32_t wave_topk_hist(const uint32_t (&x)[PER],
                                                   const bool (&ok)[PER], int k,
                                                   uint32_t *__restrict__ hist) {
    const int l = lane_id();
    int nvalid = 0;
    uint32_t mx = 0u, mn = 0xffffffffu, all = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        nvalid += __popcll(__ballot(ok[e]));
        if (ok[e]) { mx = max(mx, x[e]); mn = min(mn, x[e]); all |= 1u << e; }
    }
    if (nvalid <= k) return all;
    mx = wave_max_dpp(mx);
    mn = wave_min_dpp(mn);
    const uint32_t diff = mx ^ mn;
    int hb = diff ? 32 - __builtin_clz(diff) : 0;   // low bits that vary
    uint32_t pmask = hb >= 32 ? 0u : ~((1u << hb) - 1u);
    uint32_t prefix = mx & pmask;
    int need = k;
    bool whole = false;   // the final bin is kept whole
    while (hb > 0) {
        const int shift = hb > 8 ? hb - 8 : 0;
        const int nb = 1 << (hb - shift);
        const uint32_t dmask = (uint32_t)nb - 1u;
        *reinterpret_cast<u32x4 *>(&hist[4 * l]) = u32x4{0u, 0u, 0u, 0u};
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (ok[e] && (x[e] & pmask) == prefix)
                atomicAdd(&hist[(x[e] >> shift) & dmask], 1u);
        wave_lds_sync();
        // lane l owns bins nb-1-4l .. nb-4-4l (highest first)
        int h[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = nb - 1 - 4 * l - i;
            h[i] = b >= 0 ? (int)hist[b] : 0;
            local += h[i];
        }
        const int incl = wave_incl_scan_i32(local);
        const int above = incl - local;
        const bool cross = above < need && need <= incl;
        int digit = 0, run = above, m = 0;
        if (cross) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (run + h[i] >= need) { digit = nb - 1 - 4 * l - i; m = h[i]; break; }
                run += h[i];
            }
        }
        const int src = (int)__builtin_ctzll(__ballot(cross));
        digit = __builtin_amdgcn_readlane(digit, src);
        run = __builtin_amdgcn_readlane(run, src);
        m = __builtin_amdgcn_readlane(m, src);
        need -= run;
        prefix |= (uint32_t)digit << shift;
        pmask |= dmask << shift;
        hb = shift;
        wave_lds_sync();  // the histogram is cleared again by the next pass
        if (m == need) { whole = true; break; }
    }
    uint32_t mask = 0u;
    if (REG_MAJOR) {
        // equal keys before (e, l): all lanes at e' < e, then lanes below l at e
        int eq_run = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t hi_bits = x[e] & pmask;
            const bool eq = ok[e] && !whole && hi_bits == prefix;
            const unsigned long long b = __ballot(eq);
            if (ok[e] && (hi_bits > prefix || (whole && hi_bits == prefix))) mask |= 1u << e;
            else if (eq && eq_run + lanes_below(b) < need) mask |= 1u << e;
            eq_run += __popcll(b);
        }
        return mask;
    }
    int eq_below = 0;
    if (!whole) {
#pragma unroll
        for (int e = 0; e < PER; ++e) eq_below += lanes_below(__ballot(ok[e] && x[e] == prefix));
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (!ok[e]) continue;
        const uint32_t hi_bits = x[e] & pmask;
        if (hi_bits > prefix || (whole && hi_bits == prefix)) mask |= 1u << e;
        else if (hi_bits == prefix) {
            if (eq_below < need) mask |= 1u << e;
            ++eq_below;
        }
    }
    return mask;
}

// Exclusive prefix over the wave of small per-lane counts (0 <= cnt <= MAXC).
template <int MAXC>
__device__ __forceinline__ int wave_excl_small(int cnt) {
    int pre = 0;
#pragma unroll
    for (int c = 1; c <= MAXC; ++c) pre += lanes_below(__ballot(cnt >= c));
    return pre;
}

// ---------------------------------------------------------------- write-through access
// Data handed from one workgroup to another inside a kernel (possibly on another
// XCD, whose L2 is not coherent with this one) is stored and loaded at agent scope.
//
// The hand-off protocol (producer: store_wt of the data, wait_vmem, __syncthreads, one
// relaxed agent-scope atomicAdd on a counter; consumer: the atomicAdd that completes
// the count, __syncthreads, load_wt of the data) uses relaxed atomics only, so the HIP
// memory model alone does not order it: the order comes from the CDNA hardware, by
// these facts of the gfx9 (CDNA3/CDNA4) ISA and of the compiler's atomic lowering:
//   1. an agent-scope atomic store or load is issued with device-scope cache bits, so
//      the store is written through every non-coherent cache level (the XCD's L2
//      included) and the load is served from the device-coherent level, never from a
//      stale line in this XCD's L2;
//   2. on gfx9, vector stores count in vmcnt and a store leaves the count only once it
//      is acknowledged at the scope it was issued with, so after `s_waitcnt vmcnt(0)`
//      every store_wt of the wave is visible device-wide;
//   3. the counter atomic is performed at the device-coherent level and is issued after
//      the barrier that follows every wave's wait, so a consumer that sees its count
//      complete issues its loads after all the producers' data is visible.
// A release/acquire atomic at agent scope would give the same order by the memory
// model, at the cost of a write-back of the whole L2 (release) and an invalidation of
// it (acquire) per hand-off; the data stored this way is exactly what needs no such
// write-back. Code that hands data over must keep to the protocol: only store_wt /
// load_wt / load16_wt on the handed-over words, and the wait before the barrier.
__device__ __forceinline__ void store_wt(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_wt(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_wt(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_wt(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_wt(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes as two 8-byte agent-scope loads (p 16-byte aligned)
__device__ __forceinline__ u32x4 load16_wt(const void *p) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
// Waits until every vector memory operation this wave issued has completed (stores
// included); the "memory" clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// ---------------------------------------------------------------- block top-k (registers)

// LDS of block_topk_regs.
struct TopkSmem {
    uint32_t hist[256];
    uint32_t red[2][16];
    int32_t scan[16];
    int32_t found[4];
    __attribute__((aligned(16))) uint32_t bin_key[64];   // read 16 bytes at a time
    int32_t bin_pos[64];
    uint32_t take_bits[64];   // bit p: position p of the final bin is kept (n <= 2048)
};

// Top-k of n keys (1 <= k <= n <= 2048) that the NT threads of a workgroup hold in
// registers: thread t holds positions PER*t .. PER*t+PER-1 (positions >= n are
// ignored). Order: key descending, equal keys by ascending position. Sets bit e of
// *kept when position PER*t+e is among the k, and *first to this thread's rank
// among kept positions (kept positions ordered by position); returns k.
// Method: a histogram of up to DB bits (the highest bits where the keys differ; DB
// = 8 uses sm.hist, DB = 11 the caller's 2048-word `wide` array) finds the bin that
// holds the k-th key; bins above it are kept whole. When that bin holds at most 64
// keys they are ranked exactly by one wave (all pairs); otherwise the bin is refined
// with the next 8 bits, down to single key values, where equal keys are kept by
// position.
template <int NT, int PER, int DB = 8>
__device__ __forceinline__ int block_topk_regs(const uint32_t (&x)[PER], int n, int k,
                                               TopkSmem &sm, uint32_t *kept, int *first,
                                               uint32_t *wide = nullptr) {
    static_assert(NT == 256, "bins are owned by threads in groups of nb / 256");
    static_assert(DB == 8 || DB == 11, "digit widths: 8 or 11 bits");
    constexpr int NW = NT / WAVE;
    const int tid = threadIdx.x, l = lane_id(), w = tid / WAVE;

    // common high bits of all valid keys
    uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
    for (int e = 0; e < PER; ++e)
        if (PER * tid + e < n) { mx = max(mx, x[e]); mn = min(mn, x[e]); }
    mx = wave_max_dpp(mx);
    mn = wave_min_dpp(mn);
    if (l == 0) { sm.red[0][w] = mx; sm.red[1][w] = mn; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) { mx = max(mx, sm.red[0][i]); mn = min(mn, sm.red[1][i]); }
    const uint32_t diff = mx ^ mn;
    int hb = diff ? 32 - __builtin_clz(diff) : 0;
    uint32_t pmask = hb >= 32 ? 0u : ~((1u << hb) - 1u);
    uint32_t prefix = mx & pmask;
    int need = k;
    int mode = 0;   // 1: keep the whole final bin, 2: ranked bitmap, 3: equal keys by position
    bool first_pass = true;

    while (true) {
        if (hb == 0) { mode = 3; break; }            // the final bin is one key value
        const int width = (DB == 11 && first_pass) ? 11 : 8;
        uint32_t *hist = (DB == 11 && first_pass) ? wide : sm.hist;
        const int shift = hb > width ? hb - width : 0;
        const int nb = 1 << (hb - shift);
        const int bpt = nb > NT ? nb / NT : 1;        // bins per thread
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int i = tid; i < nb; i += NT) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (PER * tid + e < n && (x[e] & pmask) == prefix)
                atomicAdd(&hist[(x[e] >> shift) & dmask], 1u);
        __syncthreads();
        // thread t owns bins nb-bpt*(t+1) .. nb-1-bpt*t (highest bins first)
        const int top = nb - bpt * tid;
        int local = 0;
        for (int i = 1; i <= bpt; ++i) local += top - i >= 0 ? (int)hist[top - i] : 0;
        int tot;
        const int above = block_excl_scan_i32<NT>(local, sm.scan, &tot);
        if (top > 0 && above < need && need <= above + local) {
            int run = above;
            for (int i = 1; i <= bpt; ++i) {
                const int b = top - i;
                const int h = (int)hist[b];
                if (run + h >= need) {
                    sm.found[0] = b;
                    sm.found[1] = run;
                    sm.found[2] = h;
                    break;
                }
                run += h;
            }
        }
        __syncthreads();
        const int T = sm.found[0], A = sm.found[1], m = sm.found[2];
        need -= A;
        prefix |= (uint32_t)T << shift;
        pmask |= dmask << shift;
        hb = shift;
        first_pass = false;
        __syncthreads();
        if (m == need) { mode = 1; break; }
        if (m <= 64) { mode = 2; break; }
    }

    if (mode == 2) {
        // compact the final bin's keys in position order, rank them in one wave
        int c = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) c += (PER * tid + e < n && (x[e] & pmask) == prefix);
        int tot;
        int off = block_excl_scan_i32<NT>(c, sm.scan, &tot);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (PER * tid + e < n && (x[e] & pmask) == prefix) {
                sm.bin_key[off] = x[e];
                sm.bin_pos[off] = PER * tid + e;
                ++off;
            }
        }
        for (int i = tid; i < 64; i += NT) sm.take_bits[i] = 0u;
        __syncthreads();
        if (w == 0) {
            const int m = tot;
            const uint32_t kj = l < m ? sm.bin_key[l] : 0u;
            const int pj = l < m ? sm.bin_pos[l] : 0;
            // rank = keys above kj plus equal keys earlier in position order (the
            // compaction kept position order); the bin's keys are read 4 at a time by
            // broadcast LDS reads
            int rank = 0;
            for (int i0 = 0; i0 < m; i0 += 4) {
                const u32x4 k4 = *reinterpret_cast<const u32x4 *>(&sm.bin_key[i0]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rank += i0 + e < m && (k4[e] > kj || (k4[e] == kj && i0 + e < l));
            }
            if (l < m && rank < need) atomicOr(&sm.take_bits[pj >> 5], 1u << (pj & 31));
        }
        __syncthreads();
    }

    // mode 3: among the (equal) keys of the final bin keep the first `need` by position
    int eq_before = 0;
    if (mode == 3) {
        int c = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) c += (PER * tid + e < n && (x[e] & pmask) == prefix);
        int tot;
        eq_before = block_excl_scan_i32<NT>(c, sm.scan, &tot);
    }
    uint32_t mask = 0u;
    int nt = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int pos = PER * tid + e;
        if (pos >= n) continue;
        const uint32_t hi_bits = x[e] & pmask;
        bool take = hi_bits > prefix;
        if (hi_bits == prefix) {
            if (mode == 1) take = true;
            else if (mode == 2) take = (sm.take_bits[pos >> 5] >> (pos & 31)) & 1u;
            else { take = eq_before < need; ++eq_before; }
        }
        if (take) { mask |= 1u << e; ++nt; }
    }
    int tot;
    *first = block_excl_scan_i32<NT>(nt, sm.scan, &tot);
    *kept = mask;
    return tot;
}

// ---------------------------------------------------------------- FP8 (OCP E4M3)

// 8 E4M3 bytes -> 8 bf16 (exact: E4M3 values have 4 significant bits and a narrower
// exponent range than bf16), in the byte order of the input.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint2 b) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? b.y : b.x;
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
        r[2 * h] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
        r[2 * h + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
    }
    return r;
}

// E4M3 rounding of an fp32 value: nearest, ties to even; finite magnitudes beyond 448
// saturate to 448. The quantum is 2^(e-3) for |y| = 1.f * 2^e in the normal range
// (|y| >= 2^-6) and 2^-9 below it.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (!(a > 0.f)) return sign;
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    const int qe = (e < -6 ? -6 : e) - 3;
    float r = ldexpf(rintf(ldexpf(a, -qe)), qe);
    r = fminf(r, 448.0f);
    if (r < 0x1p-6f) return sign | (uint32_t)(r * 512.0f);
    const uint32_t rb = __float_as_uint(r);
    const uint32_t eb = ((rb >> 23) & 0xffu) - 120u;   // unbiased + 7
    return sign | (eb << 3) | ((rb >> 20) & 7u);
}

// 16 independent 4 x 4 fp32 outer products: lane l (block l/4, column l%4) adds
// a[lane 4(l/4) + i] * b[lane l] to c[i].
__device__ __forceinline__ f32x4 mfma_f32_4x4x1(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The low (odd = false) or high (odd = true) bf16 halves of x0 and x1 as one pair
// {x0 half, x1 half}: one byte permute.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t x0, uint32_t x1, bool odd) {
    return __builtin_amdgcn_perm(x1, x0, odd ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace qsa
