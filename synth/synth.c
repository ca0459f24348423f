/*
 * Seeded synthetic inputs shared by the oracle side and the GPU side.
 *
 * This module holds random-number generation and the double -> fp16
 * conversion of the drawn values, nothing of the LLM.int8() arithmetic.
 * Every value is a pure function of (seed, stream, index), so the bytes are
 * independent of the thread count.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: the i-th draw of a
 * stream is the SplitMix64 output function applied to state0 + (i+1)*gamma,
 * where state0 = mix(mix(seed) + stream) and gamma = 0x9E3779B97F4A7C15.
 * A uniform in (0,1) is ((h >> 11) + 0.5) * 2^-53.
 * Normal deviates: Box-Muller on the uniform pair (2p, 2p+1); element i takes
 * the cosine branch when i is even and the sine branch when odd.
 * Laplace(0,b): inverse CDF, -b * sgn(u - 1/2) * ln(1 - 2|u - 1/2|).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_state0(uint64_t seed, uint64_t stream) {
    return sm_mix(sm_mix(seed) + stream);
}

static inline double u01_from_state(uint64_t s0, uint64_t i) {
    uint64_t h = sm_mix(s0 + (i + 1) * SM_GAMMA);
    return ((double)(h >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal_from_state(uint64_t s0, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = u01_from_state(s0, 2 * p);
    double u2 = u01_from_state(s0, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline double laplace_from_state(uint64_t s0, uint64_t i, double b) {
    double d = u01_from_state(s0, i) - 0.5;
    double mag = -b * log(1.0 - 2.0 * fabs(d));
    return d < 0 ? -mag : mag;
}

/* IEEE binary16 from a double, round to nearest even, one rounding. */
static uint16_t f64_to_f16_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;          /* at or past the tie above 65504 */
    if (a < 0x1.0p-14) {                               /* subnormal range: step 2^-24 */
        double m = rint(ldexp(a, 24));                 /* exact scaling, RNE */
        return sign | (uint16_t)m;                     /* m == 1024 is the smallest normal */
    }
    int e;
    frexp(a, &e);                                      /* a = f * 2^e, f in [0.5,1) */
    e -= 1;                                            /* a in [2^e, 2^(e+1)) */
    double m = rint(ldexp(a, 10 - e));                 /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* ---------------------------------------------------------------- threads */

typedef struct {
    void (*fn)(void* ctx, int64_t lo, int64_t hi);
    void* ctx;
    int64_t lo, hi;
} span_job;

static void* span_run(void* p) {
    span_job* j = (span_job*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static int pick_threads(int nthreads) {
    if (nthreads > 0) return nthreads > 256 ? 256 : nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    if (n < 1) n = 1;
    return n > 64 ? 64 : (int)n;
}

static void parallel_for(int64_t n, int nthreads, void (*fn)(void*, int64_t, int64_t), void* ctx) {
    int nt = pick_threads(nthreads);
    if (n < 65536 || nt == 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    int ok[256];
    span_job jobs[256];
    for (int t = 0; t < nt; ++t) {
        jobs[t].fn = fn; jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nt; jobs[t].hi = n * (t + 1) / nt;
        ok[t] = pthread_create(&th[t], NULL, span_run, &jobs[t]) == 0;
        if (!ok[t]) span_run(&jobs[t]);
    }
    for (int t = 0; t < nt; ++t) if (ok[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------ public API */

double synth_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
    return u01_from_state(sm_state0(seed, stream), i);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t i) {
    return normal_from_state(sm_state0(seed, stream), i);
}

uint16_t synth_f64_to_f16(double x) { return f64_to_f16_rne(x); }

/* Matrix [rows, cols] with element (r, c) = fp16(dist(index r*cols+c) * param
 * * scale), where scale = factors[j] when c == dims[j] and (rowsel == NULL or
 * rowsel[j*rows + r] != 0), else 1.  dist 0 = standard normal (param = sigma),
 * dist 1 = Laplace with scale b = param. */
typedef struct {
    uint16_t* out;
    int64_t rows, cols;
    uint64_t s0;
    int dist;
    double param;
    const int32_t* slot;    /* [cols]: j or -1 */
    const double* factors;
    const uint8_t* rowsel;
} fill_ctx;

static void fill_span(void* p, int64_t lo, int64_t hi) {
    fill_ctx* c = (fill_ctx*)p;
    for (int64_t i = lo; i < hi; ++i) {
        double v = c->dist == 0 ? normal_from_state(c->s0, (uint64_t)i) * c->param
                                : laplace_from_state(c->s0, (uint64_t)i, c->param);
        if (c->slot) {
            int64_t col = i % c->cols;
            int32_t j = c->slot[col];
            if (j >= 0) {
                int64_t r = i / c->cols;
                if (!c->rowsel || c->rowsel[(int64_t)j * c->rows + r]) v *= c->factors[j];
            }
        }
        c->out[i] = f64_to_f16_rne(v);
    }
}

int synth_matrix_f16(uint16_t* out, int64_t rows, int64_t cols, uint64_t seed, uint64_t stream,
                     int dist, double param, int ndims, const int64_t* dims, const double* factors,
                     const uint8_t* rowsel, int nthreads) {
    if (!out || rows < 0 || cols <= 0 || (dist != 0 && dist != 1)) return 1;
    int32_t* slot = NULL;
    if (ndims > 0) {
        slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)cols);
        if (!slot) return 2;
        for (int64_t k = 0; k < cols; ++k) slot[k] = -1;
        for (int j = 0; j < ndims; ++j) {
            if (dims[j] < 0 || dims[j] >= cols) { free(slot); return 1; }
            slot[dims[j]] = j;
        }
    }
    fill_ctx c = {out, rows, cols, sm_state0(seed, stream), dist, param, slot, factors, rowsel};
    parallel_for(rows * cols, nthreads, fill_span, &c);
    free(slot);
    return 0;
}

/* Overwrite columns cols[0..ncols) of an fp16 matrix [rows, ld] with
 * +-(lo + (hi - lo) * u): magnitude uniform from index 2*(r*ld + c) of the
 * stream, sign negative when the uniform at 2*(r*ld + c) + 1 is below 1/2. */
int synth_set_columns_f16(uint16_t* out, int64_t rows, int64_t ld, uint64_t seed, uint64_t stream,
                          int ncols, const int64_t* cols, double lo, double hi) {
    if (!out || ld <= 0) return 1;
    uint64_t s0 = sm_state0(seed, stream);
    for (int j = 0; j < ncols; ++j) {
        if (cols[j] < 0 || cols[j] >= ld) return 1;
        for (int64_t r = 0; r < rows; ++r) {
            uint64_t e = (uint64_t)(r * ld + cols[j]);
            double mag = lo + (hi - lo) * u01_from_state(s0, 2 * e);
            double v = u01_from_state(s0, 2 * e + 1) < 0.5 ? -mag : mag;
            out[r * ld + cols[j]] = f64_to_f16_rne(v);
        }
    }
    return 0;
}

/* Partial Fisher-Yates: pick `count` distinct values from [0, pool) using the
 * uniforms at indices offset .. offset+count-1 of the stream. */
int synth_choose(uint64_t seed, uint64_t stream, int64_t pool, int64_t count, uint64_t offset,
                 int64_t* out) {
    if (count < 0 || count > pool) return 1;
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)(pool > 0 ? pool : 1));
    if (!perm) return 2;
    for (int64_t i = 0; i < pool; ++i) perm[i] = i;
    uint64_t s0 = sm_state0(seed, stream);
    for (int64_t j = 0; j < count; ++j) {
        int64_t r = j + (int64_t)(u01_from_state(s0, offset + (uint64_t)j) * (double)(pool - j));
        if (r >= pool) r = pool - 1;
        int64_t t = perm[j]; perm[j] = perm[r]; perm[r] = t;
        out[j] = perm[j];
    }
    free(perm);
    return 0;
}
