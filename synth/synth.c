/*
 * synth.c -- seeded, counter-based generator of synthetic inputs.
 *
 * This module produces random numbers and nothing else: it holds none of the
 * decode step's arithmetic.  Both the oracle and the GPU library are fed from
 * it, so the two see identical bits.
 *
 * Stream definition (the only thing a second implementation would need):
 *
 *   mix64(z)   = the SplitMix64 output finaliser (Steele, Lea, Flood, "Fast
 *                splittable pseudorandom number generators", OOPSLA 2014):
 *                  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                  z ^= z >> 27; z *= 0x94D049BB133111EB;
 *                  z ^= z >> 31.
 *   r(s, k, n) = mix64(s + 0x9E3779B97F4A7C15 * ((k << 40) | n))
 *                s = seed, k = stream id (< 2^24), n = counter (< 2^40).
 *   u_open(r)  = (r >> 11) * 2^-53, with 0 replaced by 2^-53   (in (0, 1])
 *   u_half(r)  = (r >> 11) * 2^-53                              (in [0, 1))
 *
 *   Normal values come in Box-Muller pairs: pair m uses
 *     u1 = u_open(r(s,k,2m)), u2 = u_open(r(s,k,2m+1)),
 *     rho = sqrt(-2 ln u1),
 *     value[2m]   = (float)(mean + std * rho * cos(2 pi u2)),
 *     value[2m+1] = (float)(mean + std * rho * sin(2 pi u2)).
 *   Uniform integers: value[i] = floor(u_half(r(s,k,i)) * bound).
 *
 * Every value depends only on (seed, stream, index), so the output does not
 * depend on the number of threads used to produce it.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t draw(uint64_t seed, uint64_t stream, uint64_t n) {
    return mix64(seed + SYNTH_GOLDEN * ((stream << 40) | n));
}

static inline double u_open(uint64_t r) {
    uint64_t m = r >> 11;
    return m ? (double)m * 0x1p-53 : 0x1p-53;
}

static inline double u_half(uint64_t r) { return (double)(r >> 11) * 0x1p-53; }

uint64_t synth_raw(uint64_t seed, uint64_t stream, uint64_t n) { return draw(seed, stream, n); }

typedef struct {
    float* out;
    int32_t* iout;
    uint64_t begin, end; /* element range [begin, end) of the whole tensor */
    uint64_t offset;     /* index of out[0] within the tensor */
    uint64_t seed, stream;
    double mean, std;
    int64_t bound;
} job_t;

static void normal_range(const job_t* j) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t i = j->begin;
    while (i < j->end) {
        uint64_t m = i >> 1;
        double u1 = u_open(draw(j->seed, j->stream, 2 * m));
        double u2 = u_open(draw(j->seed, j->stream, 2 * m + 1));
        double rho = sqrt(-2.0 * log(u1));
        double z0 = rho * cos(two_pi * u2);
        double z1 = rho * sin(two_pi * u2);
        if ((i & 1) == 0) {
            j->out[i - j->offset] = (float)(j->mean + j->std * z0);
            ++i;
            if (i >= j->end) break;
        }
        j->out[i - j->offset] = (float)(j->mean + j->std * z1);
        ++i;
    }
}

static void uniform_range(const job_t* j) {
    for (uint64_t i = j->begin; i < j->end; ++i)
        j->iout[i - j->offset] = (int32_t)(u_half(draw(j->seed, j->stream, i)) * (double)j->bound);
}

static void* normal_thread(void* p) { normal_range((const job_t*)p); return NULL; }
static void* uniform_thread(void* p) { uniform_range((const job_t*)p); return NULL; }

#define SYNTH_MAX_THREADS 256

static void run_jobs(job_t base, uint64_t count, int threads, void* (*fn)(void*)) {
    if (count == 0) return;
    if (threads < 1) threads = 1;
    if (threads > SYNTH_MAX_THREADS) threads = SYNTH_MAX_THREADS;
    if ((uint64_t)threads > count / 65536 + 1) threads = (int)(count / 65536 + 1);
    job_t jobs[SYNTH_MAX_THREADS];
    pthread_t tid[SYNTH_MAX_THREADS];
    int started[SYNTH_MAX_THREADS];
    uint64_t chunk = (count + (uint64_t)threads - 1) / (uint64_t)threads;
    chunk = (chunk + 1) & ~(uint64_t)1; /* keep Box-Muller pairs inside one chunk */
    for (int t = 0; t < threads; ++t) {
        jobs[t] = base;
        jobs[t].begin = base.begin + (uint64_t)t * chunk;
        jobs[t].end = jobs[t].begin + chunk;
        if (jobs[t].begin > base.end) jobs[t].begin = base.end;
        if (jobs[t].end > base.end) jobs[t].end = base.end;
        started[t] = (t > 0) && pthread_create(&tid[t], NULL, fn, &jobs[t]) == 0;
        if (t > 0 && !started[t]) fn(&jobs[t]);
    }
    fn(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
}

/* out[0..count) = elements [first, first+count) of normal stream (seed, stream). */
void synth_fill_normal(float* out, uint64_t first, uint64_t count, uint64_t seed, uint64_t stream,
                       double mean, double std, int threads) {
    job_t j = {0};
    j.out = out;
    j.begin = first;
    j.end = first + count;
    j.offset = first;
    j.seed = seed;
    j.stream = stream;
    j.mean = mean;
    j.std = std;
    run_jobs(j, count, threads, normal_thread);
}

/* out[0..count) = elements [first, first+count) of the uniform integer stream in [0, bound). */
void synth_fill_uniform_int(int32_t* out, uint64_t first, uint64_t count, uint64_t seed,
                            uint64_t stream, int64_t bound, int threads) {
    job_t j = {0};
    j.iout = out;
    j.begin = first;
    j.end = first + count;
    j.offset = first;
    j.seed = seed;
    j.stream = stream;
    j.bound = bound;
    run_jobs(j, count, threads, uniform_thread);
}
