/*
 * Seeded synthetic inputs: i.i.d. N(0,1) values, reproducible bit for bit.
 *
 * The attention pages derive the 1/sqrt(d_k) scale from the assumption that
 * every component of q and k is independent with mean 0 and variance 1
 * (AIInfraGuide "Self-Attention" page, section 6.1).  The workloads are
 * synthetic tensors drawn from exactly that distribution.
 *
 * This file holds no attention arithmetic.  It is the only code that both the
 * oracle side and the GPU side of the tests use: the same bytes are handed to
 * both, so a host libm difference can never split them.
 *
 * Generator (all public definitions):
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014), used in counter mode: output i of stream
 *     `seed` is mix64(seed + (i + 1) * 0x9E3779B97F4A7C15).
 *   - Box-Muller transform (1958): a pair of uniforms (u1 in (0,1],
 *     u2 in [0,1)) gives r = sqrt(-2 ln u1), z0 = r cos(2 pi u2),
 *     z1 = r sin(2 pi u2), computed in double.
 *   - Element 2p is z0 and element 2p+1 is z1 of pair p, which uses outputs
 *     2p and 2p+1.  Elements are numbered in row-major order of the tensor.
 *   - Rounding: double -> float round-to-nearest-even (the C cast), then
 *     float -> bfloat16 round-to-nearest-even on the bit pattern.
 *
 * Counter mode makes every element independent of every other, so the work
 * splits over threads with no effect on the values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t attn_gen_splitmix64(uint64_t seed, uint64_t index) {
    return mix64(seed + (index + 1) * GOLDEN);
}

/* Element `e` of stream `seed`, in double. */
static inline double normal_at(uint64_t seed, uint64_t e) {
    const uint64_t pair = e >> 1;
    const uint64_t x1 = mix64(seed + (2 * pair + 1) * GOLDEN);
    const uint64_t x2 = mix64(seed + (2 * pair + 2) * GOLDEN);
    const double two_m53 = 1.0 / 9007199254740992.0; /* 2^-53 */
    const double u1 = (double)((x1 >> 11) + 1) * two_m53; /* (0, 1] */
    const double u2 = (double)(x2 >> 11) * two_m53;       /* [0, 1) */
    const double r = sqrt(-2.0 * log(u1));
    const double a = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7F800000u) == 0x7F800000u) { /* inf / nan: keep, quiet nan */
        return (uint16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
    }
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2 };

typedef struct {
    uint64_t seed, first, n;
    void* out;
    int kind;
} job_t;

static void* run_job(void* arg) {
    const job_t* j = (const job_t*)arg;
    for (uint64_t i = 0; i < j->n; ++i) {
        const double z = normal_at(j->seed, j->first + i);
        if (j->kind == OUT_F64) {
            ((double*)j->out)[i] = z;
        } else if (j->kind == OUT_F32) {
            ((float*)j->out)[i] = (float)z;
        } else {
            ((uint16_t*)j->out)[i] = f32_to_bf16_rne((float)z);
        }
    }
    return 0;
}

/* Fill out[0..n) with elements first..first+n of stream `seed`. */
static int fill(uint64_t seed, uint64_t first, uint64_t n, void* out, int kind, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < (1u << 16)) nthreads = 1;
    pthread_t th[256];
    job_t jobs[256];
    const size_t esize = kind == OUT_F64 ? 8 : (kind == OUT_F32 ? 4 : 2);
    const uint64_t per = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        const uint64_t lo = (uint64_t)t * per;
        if (lo >= n) break;
        const uint64_t cnt = (n - lo < per) ? n - lo : per;
        jobs[t].seed = seed;
        jobs[t].first = first + lo;
        jobs[t].n = cnt;
        jobs[t].out = (char*)out + lo * esize;
        jobs[t].kind = kind;
        if (t == 0) continue; /* run on the calling thread below */
        if (pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) return -1;
        started = t;
    }
    run_job(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
    return 0;
}

int attn_gen_normal_f64(uint64_t seed, uint64_t first, uint64_t n, double* out, int nthreads) {
    return fill(seed, first, n, out, OUT_F64, nthreads);
}

int attn_gen_normal_f32(uint64_t seed, uint64_t first, uint64_t n, float* out, int nthreads) {
    return fill(seed, first, n, out, OUT_F32, nthreads);
}

int attn_gen_normal_bf16(uint64_t seed, uint64_t first, uint64_t n, uint16_t* out, int nthreads) {
    return fill(seed, first, n, out, OUT_BF16, nthreads);
}
