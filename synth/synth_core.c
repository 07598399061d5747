/*
 * synth_core.c -- the counter-based random streams behind synth/__init__.py.
 *
 * Input generation only: nothing here is part of the gated activations.
 * Value i of the stream with key k is the SplitMix64 finaliser of
 * k + (i + 1) * 0x9E3779B97F4A7C15 (Steele, Lea, Flood, OOPSLA 2014).
 * Uniforms in (0, 1] take the top 53 bits plus one, times 2^-53.  Normal j is
 * the Box-Muller cosine branch on uniforms 2j and 2j + 1.  Every value
 * depends only on (key, index), so the work splits over threads freely and
 * the output is the same for any thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t x)
{
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static inline uint64_t raw_at(uint64_t key, int64_t i)
{
    return mix64(key + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull);
}

static inline double uniform_at(uint64_t key, int64_t i)
{
    return ((double)(raw_at(key, i) >> 11) + 1.0) * 0x1.0p-53;
}

typedef struct {
    uint64_t key;
    int64_t start, lo, hi;
    double scale, shift;
    double *out;
} job_t;

static void *normal_job(void *arg)
{
    const job_t *j = (const job_t *)arg;
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t n = j->lo; n < j->hi; ++n) {
        const int64_t c = 2 * (j->start + n);
        const double u1 = uniform_at(j->key, c);
        const double u2 = uniform_at(j->key, c + 1);
        j->out[n] = j->shift + j->scale * (sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
    }
    return 0;
}

/* out[n] = shift + scale * normal(start + n), n in [0, count). */
void synth_normal(uint64_t key, int64_t start, int64_t count, double scale, double shift,
                  double *out, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (count < (1 << 16)) threads = 1;
    pthread_t tid[64];
    job_t jobs[64];
    for (int t = 0; t < threads; ++t) {
        jobs[t].key = key;
        jobs[t].start = start;
        jobs[t].lo = count * t / threads;
        jobs[t].hi = count * (t + 1) / threads;
        jobs[t].scale = scale;
        jobs[t].shift = shift;
        jobs[t].out = out;
        if (t > 0) pthread_create(&tid[t], 0, normal_job, &jobs[t]);
    }
    normal_job(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], 0);
}

void synth_raw64(uint64_t key, int64_t start, int64_t count, uint64_t *out)
{
    for (int64_t n = 0; n < count; ++n) out[n] = raw_at(key, start + n);
}

void synth_uniform(uint64_t key, int64_t start, int64_t count, double *out)
{
    for (int64_t n = 0; n < count; ++n) out[n] = uniform_at(key, start + n);
}

/* Round a double to bf16 bits the way the Python recipes do: to the nearest
 * float first (C cast), then ties-to-even on the float's top 16 bits. */
static inline uint16_t bf16_bits(double v)
{
    union { float f; uint32_t u; } c;
    c.f = (float)v;
    return (uint16_t)((c.u + 0x7FFFu + ((c.u >> 16) & 1u)) >> 16);
}

typedef struct {
    uint64_t key;
    int64_t d, ld, lo, hi;     /* rows [lo, hi) */
    double scale, shift;
    uint16_t *out;
} rows_job_t;

static void *rows_job(void *arg)
{
    const rows_job_t *j = (const rows_job_t *)arg;
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t r = j->lo; r < j->hi; ++r) {
        for (int64_t i = 0; i < j->d; ++i) {
            const int64_t c = 2 * (r * j->d + i);
            const double u1 = uniform_at(j->key, c);
            const double u2 = uniform_at(j->key, c + 1);
            const double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
            j->out[r * j->ld + i] = bf16_bits(j->shift + j->scale * z);
        }
    }
    return 0;
}

/* out[r * ld + i] = bf16(shift + scale * normal(r * d + i)) for r < rows, i < d. */
void synth_normal_rows_bf16(uint64_t key, int64_t rows, int64_t d, double scale, double shift,
                            uint16_t *out, int64_t ld, int threads)
{
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (rows * d < (1 << 16) || rows < threads) threads = 1;
    pthread_t tid[64];
    rows_job_t jobs[64];
    for (int t = 0; t < threads; ++t) {
        jobs[t] = (rows_job_t){key, d, ld, rows * t / threads, rows * (t + 1) / threads,
                               scale, shift, out};
        if (t > 0) pthread_create(&tid[t], 0, rows_job, &jobs[t]);
    }
    rows_job(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], 0);
}
