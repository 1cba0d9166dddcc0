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

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

}  // namespace qsa
