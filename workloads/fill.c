/*
 * Seeded synthetic fills for the per-layer n-gram embedding workloads.
 *
 * This file holds random-number generation and the storage encodings of
 * generated values only; it computes no step of the lookup path (no hashing,
 * no gathering, no dequantisation, no projection, gate or convolution).  Both
 * the oracle and the GPU library receive what it writes as plain inputs.
 *
 * Every element is a pure function of (seed, element index), so the bytes do
 * not depend on how many threads fill a buffer.
 *
 * Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), evaluated at a counter:
 * value i of a stream is the (i+1)-th output of SplitMix64 started at `seed`.
 *
 * Normal variates: Irwin-Hall sum of twelve 16-bit uniforms minus 6 (mean 0,
 * variance 1, support [-6, 6]); three SplitMix64 outputs per element.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1u) * SM64_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline double irwin_hall12(uint64_t seed, uint64_t i) {
    uint64_t w[3];
    uint32_t s = 0;
    w[0] = sm64_at(seed, 3u * i);
    w[1] = sm64_at(seed, 3u * i + 1u);
    w[2] = sm64_at(seed, 3u * i + 2u);
    for (int k = 0; k < 3; ++k)
        for (int b = 0; b < 64; b += 16) s += (uint32_t)((w[k] >> b) & 0xFFFFu);
    /* each uniform is (x + 0.5) / 65536 with x in [0, 65535] */
    return ((double)s + 6.0) / 65536.0 - 6.0;
}

static inline double uniform01(uint64_t seed, uint64_t i) {
    return (double)(sm64_at(seed, i) >> 11) * (1.0 / 9007199254740992.0);
}

/* Storage encoding of a generated float as bfloat16, round to nearest even. */
static inline uint16_t store_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/*
 * Storage encoding of a generated float as OCP float8 e4m3fn (bias 7, no
 * infinities, 0x7F/0xFF NaN, largest finite 448), round to nearest even,
 * saturating at +-448.
 */
static inline uint8_t store_e4m3fn(float x) {
    uint8_t sign = signbit(x) ? 0x80u : 0x00u;
    double a = fabs((double)x);
    if (!(a < 448.0)) return (uint8_t)(sign | 0x7Eu); /* saturate (also NaN input) */
    if (a < 0.015625) { /* below 2^-6: subnormal grid m * 2^-9 */
        double m = nearbyint(a * 512.0);                /* 0..8; 8 is the smallest normal */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int k;
    double f = frexp(a, &k);              /* a = f * 2^k, f in [0.5, 1) */
    int e = k - 1;                        /* a = (2f) * 2^e, 2f in [1, 2) */
    double m = nearbyint((2.0 * f - 1.0) * 8.0);
    if (m >= 8.0) { m = 0.0; e += 1; }
    int code = ((e + 7) << 3) | (int)m;
    if (code > 0x7E) code = 0x7E;
    return (uint8_t)(sign | code);
}

typedef struct {
    int kind;
    void* out;
    void* out2;
    int64_t begin, end;
    uint64_t seed;
    double a, b;
    int32_t dim;
} job_t;

enum { JOB_NORMAL_BF16 = 0, JOB_UNIFORM_BF16 = 1, JOB_FP8_ROWS = 2, JOB_NORMAL_F32 = 3, JOB_UNIFORM_BYTES = 4 };

static void run_job(job_t* j) {
    if (j->kind == JOB_NORMAL_BF16) {
        uint16_t* o = (uint16_t*)j->out;
        for (int64_t i = j->begin; i < j->end; ++i)
            o[i] = store_bf16((float)(irwin_hall12(j->seed, (uint64_t)i) * j->a));
    } else if (j->kind == JOB_UNIFORM_BF16) {
        uint16_t* o = (uint16_t*)j->out;
        for (int64_t i = j->begin; i < j->end; ++i)
            o[i] = store_bf16((float)(j->a + (j->b - j->a) * uniform01(j->seed, (uint64_t)i)));
    } else if (j->kind == JOB_UNIFORM_BYTES) { /* integers in [a, b] */
        uint8_t* o = (uint8_t*)j->out;
        const double span = j->b - j->a + 1.0;
        for (int64_t i = j->begin; i < j->end; ++i) {
            double v = j->a + floor(span * uniform01(j->seed, (uint64_t)i));
            o[i] = (uint8_t)(v > j->b ? j->b : v);
        }
    } else if (j->kind == JOB_NORMAL_F32) {
        float* o = (float*)j->out;
        for (int64_t i = j->begin; i < j->end; ++i)
            o[i] = (float)(irwin_hall12(j->seed, (uint64_t)i) * j->a);
    } else { /* JOB_FP8_ROWS: rows [begin, end) of a [rows][dim] table */
        uint8_t* q = (uint8_t*)j->out;
        float* scale = (float*)j->out2;
        float x[1024 * 8];
        for (int64_t r = j->begin; r < j->end; ++r) {
            float mx = 0.0f;
            for (int32_t c = 0; c < j->dim; ++c) {
                x[c] = (float)(irwin_hall12(j->seed, (uint64_t)(r * j->dim + c)) * j->a);
                float ax = fabsf(x[c]);
                if (ax > mx) mx = ax;
            }
            float s = mx > 0.0f ? mx / 448.0f : 1.0f;
            scale[r] = s;
            for (int32_t c = 0; c < j->dim; ++c) q[r * j->dim + c] = store_e4m3fn(x[c] / s);
        }
    }
}

static void* thread_main(void* p) {
    run_job((job_t*)p);
    return NULL;
}

static void run_parallel(job_t proto, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < 65536 || nthreads == 1) {
        proto.begin = 0;
        proto.end = n;
        run_job(&proto);
        return;
    }
    pthread_t th[256];
    job_t jobs[256];
    int started = 0;
    int64_t per = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].begin = t * per < n ? t * per : n;
        jobs[t].end = (t + 1) * per < n ? (t + 1) * per : n;
        if (pthread_create(&th[t], NULL, thread_main, &jobs[t]) == 0) {
            ++started;
        } else {
            run_job(&jobs[t]);
            jobs[t].kind = -1;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].kind != -1) pthread_join(th[t], NULL);
    (void)started;
}

/* out[i] = bf16(sigma * normal(seed, i)), i in [0, n) */
void gen_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, double sigma, int nthreads) {
    job_t j = {JOB_NORMAL_BF16, out, NULL, 0, 0, seed, sigma, 0.0, 0};
    run_parallel(j, n, nthreads);
}

/* out[i] = float(sigma * normal(seed, i)) */
void gen_normal_f32(float* out, int64_t n, uint64_t seed, double sigma, int nthreads) {
    job_t j = {JOB_NORMAL_F32, out, NULL, 0, 0, seed, sigma, 0.0, 0};
    run_parallel(j, n, nthreads);
}

/* out[i] = bf16(lo + (hi - lo) * uniform(seed, i)) */
void gen_uniform_bf16(uint16_t* out, int64_t n, uint64_t seed, double lo, double hi, int nthreads) {
    job_t j = {JOB_UNIFORM_BF16, out, NULL, 0, 0, seed, lo, hi, 0};
    run_parallel(j, n, nthreads);
}

/*
 * FP8 table with one fp32 scale per row: row r draws x = sigma * normal(seed,
 * r*dim + c), scale[r] = max|x| / 448 (1 for an all-zero row), and stores
 * q[r][c] = e4m3fn(x / scale[r]).  dim <= 8192.
 */
int gen_fp8_table(uint8_t* q, float* scale, int64_t rows, int32_t dim, uint64_t seed, double sigma,
                  int nthreads) {
    if (dim <= 0 || dim > 8192) return 1;
    job_t j = {JOB_FP8_ROWS, q, scale, 0, 0, seed, sigma, 0.0, dim};
    run_parallel(j, rows, nthreads);
    return 0;
}

/* out[i] = lo + floor((hi - lo + 1) * uniform(seed, i)), 0 <= lo <= hi <= 255 */
void gen_uniform_bytes(uint8_t* out, int64_t n, uint64_t seed, int lo, int hi, int nthreads) {
    job_t j = {JOB_UNIFORM_BYTES, out, NULL, 0, 0, seed, (double)lo, (double)hi, 0};
    run_parallel(j, n, nthreads);
}

/* Encoding helpers exposed so tests can check the generator's own encoders. */
uint16_t gen_store_bf16(float f) { return store_bf16(f); }
uint8_t gen_store_e4m3fn(float x) { return store_e4m3fn(x); }
