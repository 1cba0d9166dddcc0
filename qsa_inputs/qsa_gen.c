/*
 * qsa_gen.c -- seeded, counter-based input generator shared by the oracle checks
 * and the GPU runs. It holds none of the attention method's arithmetic: it only
 * turns (seed, tensor id, element index) into pseudo-random values, so that any
 * slice of any tensor can be produced on its own, in parallel, bit-identically.
 *
 * Stream: draw(seed, tensor, i) = mix(base + (i + 1) * GAMMA) with
 * base = mix(mix(seed) ^ (tensor * GAMMA2)), where mix is the SplitMix64 output
 * function (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014) and GAMMA its golden-ratio increment.
 *
 * Normal values: Box-Muller on draws 2i and 2i+1 (cosine branch only), scaled,
 * rounded to fp32 by the C cast and then to bf16 with round-to-nearest-even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL
#define GAMMA2 0xd1b54a32d192ed03ULL

static uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static uint64_t stream_base(uint64_t seed, uint32_t tensor)
{
    return mix(mix(seed + GAMMA) ^ ((uint64_t)(tensor + 1) * GAMMA2));
}

static uint64_t draw(uint64_t base, uint64_t i) { return mix(base + (i + 1) * GAMMA); }

static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep it quiet */
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    int kind; /* 0 normal bf16, 1 uniform int bf16, 2 weights f32, 3 raw u64 */
    uint64_t base, offset, lo_i, hi_i;
    double scale;
    int32_t lo, hi;
    void *out;
} gen_job;

static void *gen_run(void *arg)
{
    gen_job *j = (gen_job *)arg;
    for (uint64_t k = j->lo_i; k < j->hi_i; ++k) {
        uint64_t i = j->offset + k;
        switch (j->kind) {
        case 0: {
            uint64_t d0 = draw(j->base, 2 * i), d1 = draw(j->base, 2 * i + 1);
            double u1 = (double)((d0 >> 11) + 1) * 0x1p-53; /* (0, 1] */
            double u2 = (double)(d1 >> 11) * 0x1p-53;       /* [0, 1) */
            double z = sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
            ((uint16_t *)j->out)[k] = float_to_bf16((float)(z * j->scale));
            break;
        }
        case 1: {
            uint64_t span = (uint64_t)(j->hi - j->lo + 1);
            int32_t val = j->lo + (int32_t)(draw(j->base, i) % span);
            ((uint16_t *)j->out)[k] = float_to_bf16((float)val);
            break;
        }
        case 2:
            ((float *)j->out)[k] = 1.0f + (float)(draw(j->base, i) & 1u);
            break;
        default:
            ((uint64_t *)j->out)[k] = draw(j->base, i);
            break;
        }
    }
    return NULL;
}

static void gen_parallel(gen_job proto, uint64_t n, int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > 128)
        threads = 128;
    if (n < (uint64_t)threads * 65536u)
        threads = 1;
    pthread_t tid[128];
    gen_job jobs[128];
    for (int t = 0; t < threads; ++t) {
        jobs[t] = proto;
        jobs[t].lo_i = n * (uint64_t)t / (uint64_t)threads;
        jobs[t].hi_i = n * (uint64_t)(t + 1) / (uint64_t)threads;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tid[t], NULL, gen_run, &jobs[t]);
    gen_run(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tid[t], NULL);
}

/* N(0, scale^2) as bf16 bit patterns, elements [offset, offset + n). */
void qsa_gen_normal_bf16(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                         double scale, uint16_t *out, int threads)
{
    gen_job j = {0, stream_base(seed, tensor), offset, 0, 0, scale, 0, 0, out};
    gen_parallel(j, n, threads);
}

/* Integers uniform in [lo, hi] (draw mod span), stored exactly as bf16. */
void qsa_gen_uniform_int_bf16(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
                              int32_t lo, int32_t hi, uint16_t *out, int threads)
{
    gen_job j = {1, stream_base(seed, tensor), offset, 0, 0, 0.0, lo, hi, out};
    gen_parallel(j, n, threads);
}

/* Per-(token, head) indexer weights in {1, 2}. */
void qsa_gen_weights(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n, float *out,
                     int threads)
{
    gen_job j = {2, stream_base(seed, tensor), offset, 0, 0, 0.0, 0, 0, out};
    gen_parallel(j, n, threads);
}

/* Raw 64-bit draws (for placement decisions made by the caller). */
void qsa_gen_u64(uint64_t seed, uint32_t tensor, uint64_t offset, uint64_t n, uint64_t *out,
                 int threads)
{
    gen_job j = {3, stream_base(seed, tensor), offset, 0, 0, 0.0, 0, 0, out};
    gen_parallel(j, n, threads);
}
