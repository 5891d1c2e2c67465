/*
 * Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.
 *
 * This file holds no arithmetic of the IKBO method: it only draws numbers.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-based: the i-th draw of a stream whose
 * state starts at `key` is mix(key + (i + 1) * GOLDEN), the same value the sequential
 * generator returns on its (i + 1)-th call. So any slice of a stream can be produced
 * directly, in parallel, without drawing what comes before it.
 *
 * Uniforms take the top 53 bits: u = (x >> 11) * 2^-53 in [0, 1).
 * Normals use Box–Muller on the draw pair (2i, 2i + 1), cosine branch only:
 *   n_i = sqrt(-2 ln u1) * cos(2 pi u2),  u1 = ((x_{2i} >> 11) + 1) * 2^-53 in (0, 1].
 * A scaled normal is formed in fp64, rounded to fp32 (round-to-nearest-even, the C cast),
 * and, for bf16 outputs, rounded again fp32 -> bf16 round-to-nearest-even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SM_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_at(uint64_t key, uint64_t i) { return sm_mix(key + (i + 1) * SM_GOLDEN); }

/* Key of the stream that feeds one named tensor (tag) of one workload (seed). */
uint64_t synth_stream_key(uint64_t seed, uint64_t tag) {
    return sm_mix(sm_mix(seed + SM_GOLDEN) ^ (tag * 0xD1B54A32D192ED03ULL));
}

uint64_t synth_raw(uint64_t key, uint64_t i) { return sm_at(key, i); }

static inline double unif_at(uint64_t key, uint64_t i) { return (double)(sm_at(key, i) >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t i) {
    double u1 = (double)((sm_at(key, 2 * i) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(sm_at(key, 2 * i + 1) >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_UNIF_F64 = 3 };

typedef struct {
    uint64_t key;
    int64_t start, n;
    double scale;
    int kind;
    void *out;
} job_t;

static void *run_job(void *arg) {
    job_t *j = (job_t *)arg;
    for (int64_t t = 0; t < j->n; ++t) {
        uint64_t i = (uint64_t)(j->start + t);
        switch (j->kind) {
        case OUT_F64: ((double *)j->out)[t] = normal_at(j->key, i) * j->scale; break;
        case OUT_F32: ((float *)j->out)[t] = (float)(normal_at(j->key, i) * j->scale); break;
        case OUT_BF16: ((uint16_t *)j->out)[t] = f32_to_bf16_rne((float)(normal_at(j->key, i) * j->scale)); break;
        default: ((double *)j->out)[t] = unif_at(j->key, i); break;
        }
    }
    return 0;
}

static int elem_size(int kind) { return kind == OUT_BF16 ? 2 : (kind == OUT_F32 ? 4 : 8); }

/* Fill out[0..n) with draws start..start+n of stream `key`; kind selects the output form. */
void synth_fill(uint64_t key, int64_t start, int64_t n, double scale, int kind, void *out, int nthreads) {
    if (n <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < 65536) nthreads = 1;
    pthread_t th[64];
    job_t jobs[64];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    int launched = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t s = t * chunk, e = s + chunk < n ? s + chunk : n;
        if (s >= e) break;
        jobs[t].key = key;
        jobs[t].start = start + s;
        jobs[t].n = e - s;
        jobs[t].scale = scale;
        jobs[t].kind = kind;
        jobs[t].out = (char *)out + s * elem_size(kind);
        if (nthreads == 1) {
            run_job(&jobs[t]);
        } else {
            pthread_create(&th[t], 0, run_job, &jobs[t]);
            ++launched;
        }
    }
    for (int t = 0; t < launched; ++t) pthread_join(th[t], 0);
}
