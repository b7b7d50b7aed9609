/*
 * synth.c -- seeded, counter-based synthetic inputs for the row-reduction
 * library and for its oracle.
 *
 * This module is shared by both sides of every parity check, so it holds
 * none of the arithmetic of softmax, RMSNorm or cross-entropy: it only turns
 * (seed, stream, element index) into numbers.  Any row can be regenerated on
 * its own, because element (row, col) of an M x N matrix depends only on
 * seed, stream and idx = row * N + col, never on M or on other rows.
 *
 * Generator: the splitmix64 output mix (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), applied as a hash:
 *     key  = seed ^ (stream << 56) ^ idx
 *     h_k  = mix64(key + (k + 1) * 0x9E3779B97F4A7C15)    for sub-draw k = 0, 1
 * Uniform in [0,1): u = (h >> 11) * 2^-53.
 * Normal (Box-Muller, cosine branch): z = sqrt(-2 ln(1 - u0)) cos(2 pi u1).
 * Values are formed in double, rounded to fp32 by the C cast (round to
 * nearest even) and, for bf16, from fp32 to bf16 by round to nearest even.
 * Labels: ((h0 >> 32) * N) >> 32, uniform in [0, N).
 *
 * Streams used by the tests and the bench: x = 0, weight = 1, labels = 2,
 * spikes = 3.
 *
 * All entry points are plain C with pointers and sizes; large fills are split
 * over POSIX threads by rows (nthreads <= 0 means "one per online CPU").
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { SYNTH_F32 = 0, SYNTH_BF16 = 1 };

static const uint64_t GOLDEN_GAMMA = 0x9E3779B97F4A7C15ULL;

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t stream, uint64_t idx, unsigned k) {
    uint64_t key = seed ^ (stream << 56) ^ idx;
    return mix64(key + (uint64_t)(k + 1) * GOLDEN_GAMMA);
}

static inline double unit(uint64_t h) { return (double)(h >> 11) * 0x1.0p-53; }

/* fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN. */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline void put(void *out, int dtype, int64_t i, double v) {
    float f = (float)v;
    if (dtype == SYNTH_F32) ((float *)out)[i] = f;
    else ((uint16_t *)out)[i] = f32_to_bf16(f);
}

/* ---- row-parallel driver ------------------------------------------------ */

enum { K_NORMAL = 0, K_UNIFORM = 1, K_SPIKES = 2 };

typedef struct {
    int kind;
    uint64_t seed, stream;
    const int64_t *row_ids; /* NULL: rows row0 .. row0+nrows-1 */
    int64_t row0, nrows, N;
    double a, b;            /* normal: sigma, mean; uniform: lo, hi; spikes: p, value */
    int dtype;
    void *out;
    int64_t r_begin, r_end; /* this thread's slice of [0, nrows) */
} job_t;

static void run_rows(const job_t *j) {
    for (int64_t r = j->r_begin; r < j->r_end; ++r) {
        int64_t row = j->row_ids ? j->row_ids[r] : j->row0 + r;
        uint64_t base = (uint64_t)row * (uint64_t)j->N;
        int64_t o = r * j->N;
        for (int64_t c = 0; c < j->N; ++c) {
            uint64_t idx = base + (uint64_t)c;
            switch (j->kind) {
            case K_NORMAL: {
                double u0 = unit(draw(j->seed, j->stream, idx, 0));
                double u1 = unit(draw(j->seed, j->stream, idx, 1));
                double z = sqrt(-2.0 * log(1.0 - u0)) * cos(6.283185307179586 * u1);
                put(j->out, j->dtype, o + c, j->b + j->a * z);
                break;
            }
            case K_UNIFORM: {
                double u = unit(draw(j->seed, j->stream, idx, 0));
                put(j->out, j->dtype, o + c, j->a + (j->b - j->a) * u);
                break;
            }
            case K_SPIKES: {
                double u = unit(draw(j->seed, j->stream, idx, 0));
                if (u < j->a) put(j->out, j->dtype, o + c, j->b);
                break;
            }
            }
        }
    }
}

static void *thread_main(void *p) {
    run_rows((const job_t *)p);
    return NULL;
}

static void run(job_t proto, int nthreads) {
    if (proto.nrows <= 0 || proto.N <= 0) return;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 64) nthreads = 64;
    int64_t work = proto.nrows * proto.N;
    if (work < (int64_t)1 << 18 || nthreads == 1 || proto.nrows == 1) {
        proto.r_begin = 0;
        proto.r_end = proto.nrows;
        run_rows(&proto);
        return;
    }
    if (nthreads > proto.nrows) nthreads = (int)proto.nrows;
    pthread_t tid[64];
    job_t jobs[64];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].r_begin = proto.nrows * t / nthreads;
        jobs[t].r_end = proto.nrows * (t + 1) / nthreads;
        if (pthread_create(&tid[t], NULL, thread_main, &jobs[t]) == 0) started = t + 1;
        else { run_rows(&jobs[t]); }
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* ---- exported entry points --------------------------------------------- */

/* mean + sigma * N(0,1) per element, written as fp32 or bf16 bits. */
void synth_normal(uint64_t seed, uint64_t stream, const int64_t *row_ids, int64_t row0,
                  int64_t nrows, int64_t N, double sigma, double mean, int dtype, void *out,
                  int nthreads) {
    job_t j = {K_NORMAL, seed, stream, row_ids, row0, nrows, N, sigma, mean, dtype, out, 0, 0};
    run(j, nthreads);
}

/* U(lo, hi) per element. */
void synth_uniform(uint64_t seed, uint64_t stream, const int64_t *row_ids, int64_t row0,
                   int64_t nrows, int64_t N, double lo, double hi, int dtype, void *out,
                   int nthreads) {
    job_t j = {K_UNIFORM, seed, stream, row_ids, row0, nrows, N, lo, hi, dtype, out, 0, 0};
    run(j, nthreads);
}

/* Overwrite each element, independently with probability p, by `value`. */
void synth_spikes(uint64_t seed, uint64_t stream, const int64_t *row_ids, int64_t row0,
                  int64_t nrows, int64_t N, double p, double value, int dtype, void *out,
                  int nthreads) {
    job_t j = {K_SPIKES, seed, stream, row_ids, row0, nrows, N, p, value, dtype, out, 0, 0};
    run(j, nthreads);
}

/* One int32 label per row, uniform in [0, N); element index is the row. */
void synth_labels(uint64_t seed, uint64_t stream, const int64_t *row_ids, int64_t row0,
                  int64_t nrows, int64_t N, int32_t *out) {
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t row = row_ids ? row_ids[r] : row0 + r;
        uint64_t h = draw(seed, stream, (uint64_t)row, 0);
        out[r] = (int32_t)(((h >> 32) * (uint64_t)N) >> 32);
    }
}

/* Element-wise fp32 -> bf16 (round to nearest even), for hand-built inputs. */
void synth_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}
