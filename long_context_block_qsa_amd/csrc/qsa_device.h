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

// Control block at the start of the workspace: counters through which the workgroups of
// one kernel learn which of them finishes a piece of work. Zero before a call; every call
// leaves it zero.
//   [0, 64)    per decode score tile: chunks scored so far (tiles of rows too long to be
//              merged from chunk candidates, whose last workgroup selects them exactly)
constexpr int CTL_TILE = 0;
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

// Max and sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that hold one column
// of an MFMA 16x16 result), in every lane of a full wave. gfx950's row-swap permutes do
// the exchange in the VALU instead of an LDS permute: a 16-lane (32-lane) swap of a value
// with itself leaves each lane the pair {v[l], v[l ^ 16]} ({v[l], v[l ^ 32]}) across its
// two results, whichever way round, and both lanes of a pair add the same two operands,
// so the result is the same in all four lanes and equals that of the LDS-permute sums.
__device__ __forceinline__ float wave_max_xor_16_32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
// WIDE: 11 + 11 + 10 bits (2048-bin histograms).
struct DigitPlan {
    int n;
    int shift[4];
    int width[4];
};
constexpr DigitPlan kWide = {3, {21, 10, 0, 0}, {11, 11, 10, 0}};
constexpr DigitPlan kWideFirst = {1, {21, 0, 0, 0}, {11, 0, 0, 0}};   // first digit only
constexpr DigitPlan kWideRest = {2, {10, 0, 0, 0}, {11, 10, 0, 0}};   // after it
constexpr int kHistBins = 2048;

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
// A select may also start below the first digit: prefix0 / pmask0 give the bits already
// fixed (only keys matching them count) and k is then the rank among those keys. On
// return *exact_out (if given) tells whether theta is the k-th key itself (every digit
// refined, or the bin found held one key value) or only its bits under pmask so far.
template <int NT, typename KeyPtr>
__device__ __forceinline__ void radix_kth(KeyPtr keys, int64_t n, int64_t k,
                                          const DigitPlan &plan, uint32_t *hist,
                                          int32_t *scan_sh, uint32_t *found,
                                          uint32_t *theta_out, int64_t *need_out,
                                          uint32_t prefix0 = 0u, uint32_t pmask0 = 0u,
                                          bool *exact_out = nullptr) {
    static_assert(NT == 256, "bin ownership assumes 256 threads");
    constexpr int NW = NT / WAVE;
    const int tid = threadIdx.x;
    // a row holds fewer than 2^31 keys (its blocks of an int32 length): 32-bit positions
    const uint32_t n32 = (uint32_t)n;
    uint32_t prefix = prefix0, pmask = pmask0;
    int64_t need = k;
    bool exact = false;
#pragma unroll 1
    for (int pass = 0; pass < plan.n; ++pass) {
        const int shift = plan.shift[pass], nb = 1 << plan.width[pass];
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int i = tid; i < nb; i += NT) hist[i] = 0u;
        if (tid == 0) { found[0] = 0u; found[1] = 0u; }
        __syncthreads();
        // keys are read in batches of 8 before their atomics, so the loads overlap; whole
        // batches need no bounds checks
        uint32_t k_or = 0u, k_and = 0xffffffffu;
        auto count = [&](uint32_t x) {
            if ((x & pmask) == prefix) {
                atomicAdd(&hist[(x >> shift) & dmask], 1u);
                k_or |= x;
                k_and &= x;
            }
        };
        uint32_t i0 = tid;
        for (; i0 + 7u * NT < n32; i0 += 8 * NT) {
            uint32_t kk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kk[e] = keys[i0 + (uint32_t)e * NT];
#pragma unroll
            for (int e = 0; e < 8; ++e) count(kk[e]);
        }
        if (i0 < n32) {
            uint32_t kk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t i = i0 + (uint32_t)e * NT;
                kk[e] = i < n32 ? keys[i] : 0u;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (i0 + (uint32_t)e * NT < n32) count(kk[e]);
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
            exact = true;
            break;
        }
        if (shift == 0) exact = true;
    }
    *theta_out = prefix;
    *need_out = need;
    if (exact_out) *exact_out = exact;
}

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Per-(element, wave) counts of a batch of an ordered pass, c[e * NW + w] (element e of
// wave w holds the keys at base + e * NT + 64 w + lane): their exclusive prefix in position
// order (element-major, then wave) for this wave's elements into pre[] (wave-uniform), and
// the batch total. Every wave derives it from the table itself: one LDS read per lane, a DPP
// scan and register reads, instead of adding up the table per element.
template <int NW, int PER>
__device__ __forceinline__ int batch_prefix(const int32_t *c, int w, int (&pre)[PER]) {
    constexpr int NC = NW * PER;
    static_assert(NC <= WAVE, "a batch's counts fit one wave");
    const int l = lane_id();
    const int x = l < NC ? c[l] : 0;
    const int incl = wave_incl_scan_i32(x);
    const int excl = incl - x;
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[e] = __builtin_amdgcn_readlane(excl, e * NW + w);
    return __builtin_amdgcn_readlane(incl, NC - 1);
}

// Ordered pass after radix_kth: keeps every key above theta and the first `need` keys
// equal to it (by position), writing their positions in ascending order to out_idx (at
// most cap); returns the number kept. Thread t reads element e of a batch at position
// base + e*NT + t, so every load instruction reads consecutive keys. A kept key's slot is
// its rank in position order: the kept keys of earlier elements, of earlier waves at the
// same element (batch_prefix), and of lower lanes (a ballot). Per-(element, wave) counts of
// equal and of kept keys go through `cnt` (LDS, 4 * (NT/64) * PER ints; two barriers per
// batch, the two halves used by alternate batches). All NT threads must call it.
template <int NT, int PER, typename KeyPtr>
__device__ __forceinline__ int64_t emit_kept(KeyPtr keys, int64_t n, uint32_t theta,
                                             int64_t need, int32_t *out_idx, int64_t cap,
                                             int32_t *cnt) {
    constexpr int NW = NT / WAVE;
    constexpr int NC = NW * PER;
    static_assert(PER <= WAVE, "one lane per element writes the wave's counts");
    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    // fewer than 2^31 keys, so positions, counts and slots are 32-bit
    const uint32_t n32 = (uint32_t)n;
    const int need32 = (int)need, cap32 = (int)min<int64_t>(cap, INT32_MAX);
    int run_eq = 0, run_sel = 0;
    int par = 0;
#pragma unroll 1
    for (uint32_t base = 0; base < n32; base += (uint32_t)NT * PER, par ^= 1) {
        int32_t *ceq = cnt + par * 2 * NC;   // [element][wave]: keys equal to theta
        int32_t *ctk = ceq + NC;             // [element][wave]: kept keys
        uint32_t kk[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t i = base + (uint32_t)(e * NT + tid);
            kk[e] = i < n32 ? keys[i] : 0u;
        }
        unsigned long long beq[PER];
        int v = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            beq[e] = __ballot(base + (uint32_t)(e * NT + tid) < n32 && kk[e] == theta);
            v = l == e ? (int)__popcll(beq[e]) : v;
        }
        if (l < PER) ceq[l * NW + w] = v;
        __syncthreads();
        // equal keys before each element of this lane; then which keys are kept
        int pre[PER];
        const int eq_tot = batch_prefix<NW, PER>(ceq, w, pre);
        unsigned long long btk[PER];
        v = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const bool valid = base + (uint32_t)(e * NT + tid) < n32;
            const bool eq = (beq[e] >> l) & 1ull;
            const bool take = (valid && kk[e] > theta) ||
                              (eq && run_eq + pre[e] + lanes_below(beq[e]) < need32);
            btk[e] = __ballot(take);
            v = l == e ? (int)__popcll(btk[e]) : v;
        }
        if (l < PER) ctk[l * NW + w] = v;
        __syncthreads();
        const int tk_tot = batch_prefix<NW, PER>(ctk, w, pre);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if ((btk[e] >> l) & 1ull) {
                const int slot = run_sel + pre[e] + lanes_below(btk[e]);
                if (slot < cap32) out_idx[slot] = (int32_t)(base + (uint32_t)(e * NT + tid));
            }
        }
        run_eq += eq_tot;
        run_sel += tk_tot;
    }
    return run_sel;
}

// Ordered pass that lists in LDS, by ascending position, the positions of the keys above
// hi (a_pos) and the keys in [lo, hi] with their positions (c_key, c_pos); the caller
// knows both counts fit. Element e of a batch is position base + e*NT + t, as in
// emit_kept; a key's slot is the number of listed keys before it (earlier elements,
// earlier waves at the same element, lower lanes). cnt: LDS, 4 * (NT/64) * PER ints (two
// halves used by alternate batches, one barrier per batch). All NT threads must call it.
template <int NT, int PER, typename KeyPtr>
__device__ __forceinline__ void collect_bin(KeyPtr keys, int64_t n, uint32_t lo, uint32_t hi,
                                            int32_t *a_pos, uint32_t *c_key, int32_t *c_pos,
                                            int32_t *cnt) {
    constexpr int NW = NT / WAVE;
    constexpr int NC = NW * PER;
    static_assert(PER <= WAVE, "one lane per element writes the wave's counts");
    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    int run_a = 0, run_c = 0;
    int par = 0;
    const uint32_t n32 = (uint32_t)n;   // fewer than 2^31 keys
#pragma unroll 1
    for (uint32_t base = 0; base < n32; base += (uint32_t)NT * PER, par ^= 1) {
        int32_t *ca = cnt + par * 2 * NC;   // [element][wave]: keys above hi
        int32_t *cc = ca + NC;              // [element][wave]: keys in [lo, hi]
        uint32_t kk[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t i = base + (uint32_t)(e * NT + tid);
            kk[e] = i < n32 ? keys[i] : 0u;
        }
        unsigned long long ba[PER], bc[PER];
        int va = 0, vc = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const bool valid = base + (uint32_t)(e * NT + tid) < n32;
            ba[e] = __ballot(valid && kk[e] > hi);
            bc[e] = __ballot(valid && kk[e] >= lo && kk[e] <= hi);
            va = l == e ? (int)__popcll(ba[e]) : va;
            vc = l == e ? (int)__popcll(bc[e]) : vc;
        }
        if (l < PER) { ca[l * NW + w] = va; cc[l * NW + w] = vc; }
        __syncthreads();
        int pa[PER], pc[PER];
        const int ta = batch_prefix<NW, PER>(ca, w, pa);
        const int tc = batch_prefix<NW, PER>(cc, w, pc);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int32_t pos = (int32_t)(base + (uint32_t)(e * NT + tid));
            if ((ba[e] >> l) & 1ull) a_pos[run_a + pa[e] + lanes_below(ba[e])] = pos;
            if ((bc[e] >> l) & 1ull) {
                const int sl = run_c + pc[e] + lanes_below(bc[e]);
                c_key[sl] = kk[e];
                c_pos[sl] = pos;
            }
        }
        run_a += ta;
        run_c += tc;
    }
    __syncthreads();
}

// Number of entries of the ascending list v[0..n) below x.
__device__ __forceinline__ int lower_bound_i32(const int32_t *v, int n, int32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (v[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
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

// Wave-wide OR / AND of uint32 (DPP row shifts and broadcasts, result from lane 63).
__device__ __forceinline__ uint32_t wave_or_dpp(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}
__device__ __forceinline__ uint32_t wave_and_dpp(uint32_t v) {
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xf, 0xf, false);
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xf, 0xf, false);
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false);
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false);
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false);
    v &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}

// Exact top-k (1 <= k) of the valid keys one wave holds in registers: lane l holds
// positions PER*l .. PER*l+PER-1, ok[e] marks the valid ones. Order: key descending,
// equal keys by ascending position. Returns this lane's kept mask (bit e); all valid
// keys when there are at most k.
// Method: a bitwise search for the k-th largest key theta, from the highest bit where
// the keys differ down, over the bits that differ between some keys only (the others
// are the same in every key, theta's included): a bit is set in theta when at least k
// keys reach it, counted with ballots (no LDS, no atomics), and the search stops as
// soon as exactly k keys reach theta. Keys above theta are kept, then keys equal to
// theta by position while fewer than k are kept. (A histogram radix select was several
// times slower: with small-integer scores many keys share a bin and its LDS atomics
// serialize.)
template <int PER>
__device__ __forceinline__ uint32_t wave_topk_bits(const uint32_t (&x)[PER],
                                                   const bool (&ok)[PER], int k) {
    unsigned long long okm[PER];
    int nvalid = 0;
    uint32_t o = 0u, an = 0xffffffffu, all = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        okm[e] = __ballot(ok[e]);
        nvalid += __popcll(okm[e]);
        if (ok[e]) { o |= x[e]; an &= x[e]; all |= 1u << e; }
    }
    if (nvalid <= k) return all;
    o = wave_or_dpp(o);
    an = wave_and_dpp(an);
    uint32_t theta = an;      // every key has the bits set in all keys
    uint32_t rem = o ^ an;    // bits that differ between keys, searched high to low
    bool exact = false;       // exactly k keys are >= theta
    while (rem) {
        const uint32_t bit = 1u << (31 - __builtin_clz(rem));
        rem ^= bit;
        const uint32_t c = theta | bit;
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) cnt += __popcll(__ballot(x[e] >= c) & okm[e]);
        if (cnt >= k) {
            theta = c;
            if (cnt == k) { exact = true; break; }
        }
    }
    uint32_t mask = 0u;
    if (exact) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (ok[e] && x[e] >= theta) mask |= 1u << e;
        return mask;
    }
    int gt = 0, eq_below = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        gt += __popcll(__ballot(x[e] > theta) & okm[e]);
        eq_below += lanes_below(__ballot(x[e] == theta) & okm[e]);
    }
    const int need = k - gt;   // keys equal to theta to keep, the first by position
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (!ok[e]) continue;
        if (x[e] > theta) mask |= 1u << e;
        else if (x[e] == theta) {
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

// ---------------------------------------------------------------- memory waits
// No kernel here passes data from one workgroup to another while both run: data one
// workgroup writes is read by a later kernel, or by the same workgroup after a barrier.
// (Between workgroups only arrival counts pass, by device-scope atomics.)
// Waits until every vector memory operation this wave issued has completed (stores
// included); the "memory" clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// ---------------------------------------------------------------- block top-k (registers)

// LDS of block_topk_radix.
struct TopkSmem {
    uint32_t hist[3][256];
    uint32_t red[2][16];
    int32_t scan[16];
};

// Top-k of n keys (1 <= k, n <= 256 * PER <= 8192) that the 256 threads of a workgroup hold in
// registers: thread t holds positions PER*t .. PER*t+PER-1 (positions >= n are
// ignored). Order: key descending, equal keys by ascending position. Sets bit e of
// *kept when position PER*t+e is among the k, and *first to this thread's rank among
// kept positions (kept positions ordered by position); returns the number kept
// (min(k, n)).
// Method: radix select with 8-bit digits over the bits that differ between keys (an
// OR / AND of all keys gives them; lower bits that never differ are not refined), one
// workgroup barrier per digit: the threads add their keys to a 256-bin LDS histogram,
// and after the barrier every wave scans the bins itself (so all waves find the bin
// holding the k-th key without another barrier). Three histograms rotate: a pass
// fills one and clears the one the next pass fills, which no wave reads any more.
// Bins above the k-th key's are kept whole, as is its own bin once all of it fits;
// otherwise its keys are equal and the first by position are kept. One scan of packed
// per-thread counts then ranks the kept positions.
template <int NT, int PER>
__device__ __forceinline__ int block_topk_radix(const uint32_t (&x)[PER], int n, int k,
                                                TopkSmem &sm, uint32_t *kept, int *first) {
    static_assert(NT == 256, "one histogram bin per thread");
    static_assert(NT * PER <= 8192, "packed 16-bit counts");
    constexpr int NW = NT / WAVE;
    const int tid = threadIdx.x, l = lane_id(), w = tid / WAVE;
    bool ok[PER];
    uint32_t o = 0u, an = 0xffffffffu;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        ok[e] = PER * tid + e < n;
        if (ok[e]) { o |= x[e]; an &= x[e]; }
    }
    if (n <= k) {   // every valid position is kept (uniform)
        uint32_t m = 0u;
#pragma unroll
        for (int e = 0; e < PER; ++e) m |= ok[e] ? 1u << e : 0u;
        *kept = m;
        *first = min(PER * tid, max(n, 0));
        return max(n, 0);
    }
    sm.hist[0][tid] = 0u;
    o = wave_or_dpp(o);
    an = wave_and_dpp(an);
    if (l == 0) { sm.red[0][w] = o; sm.red[1][w] = an; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) { o |= sm.red[0][i]; an &= sm.red[1][i]; }
    const uint32_t vary = o ^ an;
    int hb = vary ? 32 - __builtin_clz(vary) : 0;       // bits >= hb: the same in all keys
    const int lo = vary ? __builtin_ctz(vary) : 0;      // bits < lo: the same in all keys
    uint32_t pmask = hb >= 32 ? 0u : ~((1u << hb) - 1u);
    uint32_t prefix = o & pmask;
    int need = k;
    bool whole = false;   // the final bin is kept whole
    for (int pass = 0; hb > lo; ++pass) {   // uniform over the workgroup
        const int shift = max(hb - 8, lo);
        const int nb = 1 << (hb - shift);
        const uint32_t dmask = (uint32_t)nb - 1u;
        uint32_t *h = sm.hist[pass % 3];
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (ok[e] && (x[e] & pmask) == prefix) atomicAdd(&h[(x[e] >> shift) & dmask], 1u);
        sm.hist[(pass + 1) % 3][tid] = 0u;
        __syncthreads();
        // lane l of every wave owns bins nb-1-4l .. nb-4-4l (highest first)
        int hc[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bn = nb - 1 - 4 * l - i;
            hc[i] = bn >= 0 ? (int)h[bn] : 0;
            local += hc[i];
        }
        const int incl = wave_incl_scan_i32(local);
        const int above = incl - local;
        const bool cross = above < need && need <= incl;
        int digit = 0, run = above, m = 0;
        if (cross) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (run + hc[i] >= need) { digit = nb - 1 - 4 * l - i; m = hc[i]; break; }
                run += hc[i];
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
        if (m == need) { whole = true; break; }
    }
    // per thread: keys kept outright (high bits above the prefix, or equal to it when
    // the final bin is kept whole) and keys equal to the final value, packed for one scan
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (!ok[e]) continue;
        const uint32_t hi = x[e] & pmask;
        n_gt += hi > prefix || (whole && hi == prefix);
        n_eq += !whole && hi == prefix;
    }
    int tot;
    const int before = block_excl_scan_i32<NT>((n_gt << 16) | n_eq, sm.scan, &tot);
    const int take = k - (tot >> 16);   // keys of the final value kept, the first by position
    int eq_before = before & 0xffff;
    *first = (before >> 16) + min(take, eq_before);
    uint32_t mask = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (!ok[e]) continue;
        const uint32_t hi = x[e] & pmask;
        if (hi > prefix || (whole && hi == prefix)) mask |= 1u << e;
        else if (hi == prefix) {
            if (eq_before < take) mask |= 1u << e;
            ++eq_before;
        }
    }
    *kept = mask;
    return k;
}

// ---------------------------------------------------------------- FP8 (OCP E4M3)

// 8 E4M3 bytes -> 8 bf16 (exact: E4M3 values have 4 significant bits and a narrower
// exponent range than bf16), in the byte order of the input.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint2 b) {
    // gfx950's scaled conversion, scale 1: two E4M3 bytes (the low or the high pair of a
    // word) to two bf16 in one instruction, exactly (every E4M3 value is a bf16 value)
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? b.y : b.x;
        r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
        r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
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

// Transposing LDS read of gfx950 (ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// receives as its 16-bit element r (r = 0..3) element i % 4 of the four 16-bit values
// that lane 4r + i / 4 of the group addresses (8 bytes, 8-byte aligned, in LDS).
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p));
    return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace qsa
