/*
 * Seeded synthetic inputs shared by the GPU path and the CPU oracle.
 *
 * This file holds no arithmetic of the decode method itself: it only turns
 * (seed, stream, index) into random bits and from those into the input
 * tensors both sides consume (bf16 weights, prompt ids, pre-filled KV rows).
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; finalizer constants as
 * published by S. Vigna).  Draw i of stream s under seed k is the (i+1)-th
 * SplitMix64 output from the state base(k, s) = mix(mix(k) ^ (s * C)), so any
 * element can be computed independently of the others (counter-based).
 * Normals use the Box-Muller transform on two consecutive draws, whose cosine
 * and sine branches give two consecutive normals.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ull
#define STREAM_MULT 0xD1B54A32D192ED03ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed + GOLDEN_GAMMA) ^ (stream * STREAM_MULT));
}

/* i-th output (0-based) of SplitMix64 started at state `base`. */
static inline uint64_t draw(uint64_t base, uint64_t i) {
    return mix64(base + (i + 1) * GOLDEN_GAMMA);
}

uint64_t synth_draw_u64(uint64_t seed, uint64_t stream, uint64_t index) {
    return draw(stream_base(seed, stream), index);
}

/* Box-Muller on draws 2j, 2j+1 gives the pair of standard normals 2j
 * (cosine branch) and 2j+1 (sine branch) of the stream. */
static inline void normal_pair(uint64_t base, uint64_t j, double *n0, double *n1) {
    uint64_t a = draw(base, 2 * j), b = draw(base, 2 * j + 1);
    double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
    double r = sqrt(-2.0 * log(u1)), t = 6.283185307179586476925 * u2;
    *n0 = r * cos(t);
    *n1 = r * sin(t);
}
/* Standard normal number `index` of the stream. */
static inline double normal_at(uint64_t base, uint64_t index) {
    double n0, n1;
    normal_pair(base, index >> 1, &n0, &n1);
    return (index & 1) ? n1 : n0;
}

double synth_normal_at(uint64_t seed, uint64_t stream, uint64_t index) {
    return normal_at(stream_base(seed, stream), index);
}

/* float -> bf16 bits, round to nearest even (input encoding only). */
static inline uint16_t to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    uint64_t base, offset, begin, end;
    double mean, std;
    uint16_t *out_bf16;
    int32_t *out_ids;
    uint32_t modulus;
} job_t;

static void *normal_worker(void *p) {
    job_t *j = (job_t *)p;
    uint64_t i = j->begin;
    while (i < j->end) {
        const uint64_t g = j->offset + i;  /* global index */
        double n0, n1;
        normal_pair(j->base, g >> 1, &n0, &n1);
        if ((g & 1) == 0 && i + 1 < j->end) {  /* both members of the pair are ours */
            j->out_bf16[i] = to_bf16_bits((float)(j->mean + j->std * n0));
            j->out_bf16[i + 1] = to_bf16_bits((float)(j->mean + j->std * n1));
            i += 2;
        } else {
            j->out_bf16[i] = to_bf16_bits((float)(j->mean + j->std * ((g & 1) ? n1 : n0)));
            i += 1;
        }
    }
    return NULL;
}

static void *ids_worker(void *p) {
    job_t *j = (job_t *)p;
    for (uint64_t i = j->begin; i < j->end; ++i)
        j->out_ids[i] = (int32_t)(draw(j->base, j->offset + i) % j->modulus);
    return NULL;
}

static void run_jobs(job_t *proto, uint64_t n, int nthreads, void *(*fn)(void *)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if ((uint64_t)nthreads > n / 65536 + 1) nthreads = (int)(n / 65536 + 1);
    pthread_t th[64];
    int launched[64] = {0};
    job_t jobs[64];
    uint64_t per = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].begin = (uint64_t)t * per < n ? (uint64_t)t * per : n;
        jobs[t].end = jobs[t].begin + per < n ? jobs[t].begin + per : n;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].begin >= jobs[t].end) continue;
        launched[t] = pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!launched[t]) fn(&jobs[t]);
    }
    fn(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (launched[t]) pthread_join(th[t], NULL);
}

/* out[i] = bf16(mean + std * N_i), N_i = normal number (offset + i) of (seed, stream). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                       double mean, double std, uint16_t *out, int nthreads) {
    job_t proto = {0};
    proto.base = stream_base(seed, stream);
    proto.offset = offset;
    proto.mean = mean;
    proto.std = std;
    proto.out_bf16 = out;
    run_jobs(&proto, n, nthreads, normal_worker);
}

/* out[i] = draw(offset + i) mod modulus: uniform token ids in [0, modulus). */
void synth_uniform_ids(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                       uint32_t modulus, int32_t *out, int nthreads) {
    job_t proto = {0};
    proto.base = stream_base(seed, stream);
    proto.offset = offset;
    proto.modulus = modulus ? modulus : 1;
    proto.out_ids = out;
    run_jobs(&proto, n, nthreads, ids_worker);
}
