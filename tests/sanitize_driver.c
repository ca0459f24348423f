/*
 * Sanitizer driver - TEST INFRASTRUCTURE ONLY.
 *
 * Calls every function that the CPU oracle (oracle/oracle.c) and the seeded
 * input generator (synth/synth.c) export, over small, ragged and degenerate
 * shapes, so that builds with AddressSanitizer + UndefinedBehaviorSanitizer
 * and with ThreadSanitizer walk every path: both 16-bit types, the
 * memory-halved branch (no 16-bit weight), sampled rows, tau = 0 and
 * tau = +inf, all-zero rows and columns, scales small enough that 127/s
 * leaves the fp32 range, the int32-overflow count of the integer matmul, and
 * the threaded splits (more threads than rows included).
 *
 * It checks no values (the pins do that); it exits non-zero only when a
 * call reports an error that it should not, and a sanitizer report ends it
 * with the sanitizer's own status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/oracle.c */
double oracle_f16_decode(uint16_t h);
uint16_t oracle_f16_encode(double x);
float oracle_bf16_decode(uint16_t b);
uint16_t oracle_bf16_encode(double x);
int oracle_max_threads(void);
void oracle_quantize_weight_typed(const void* W, int type, int64_t K, int64_t N, int8_t* Wq,
                                  float* sw, int nthreads);
void oracle_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int8_t* Wq, float* sw,
                            int nthreads);
void oracle_detect(const uint16_t* X, int64_t T, int64_t K, float tau, uint8_t* flag, int ht);
int64_t oracle_compact(const uint8_t* flag, int64_t K, int32_t* idx);
void oracle_quantize_rows(const uint16_t* X, int64_t T, int64_t K, const uint8_t* flag,
                          const int64_t* rows, int64_t M, int8_t* Xq, float* sx, int ht);
int64_t oracle_int8_gemm(const int8_t* Xq, int64_t M, int64_t K, const int8_t* Wq, int64_t N,
                         int32_t* acc, int nthreads);
uint16_t oracle_dequant_weight_h(int8_t q, float sw, int ht);
uint16_t oracle_dequant_weight(int8_t q, float sw);
void oracle_output(const int32_t* acc, const float* sx, const float* sw, const uint16_t* X,
                   const uint16_t* W16, const int8_t* Wq, const int64_t* rows, int64_t M,
                   int64_t K, int64_t N, const int32_t* idx, int64_t o, uint16_t* Y, double* Y64,
                   int nthreads, int ht);
int64_t oracle_mixed_matmul(const uint16_t* X, int64_t T, int64_t K, const int8_t* Wq,
                            const float* sw, const uint16_t* W16, int64_t N, float tau,
                            const int64_t* rows, int64_t M, uint8_t* flag_out, int32_t* idx_out,
                            int8_t* xq_out, float* sx_out, int32_t* acc_out, uint16_t* Y,
                            double* Y64, int nthreads, int ht);

/* synth/synth.c */
double synth_uniform(uint64_t seed, uint64_t stream, uint64_t i);
double synth_normal(uint64_t seed, uint64_t stream, uint64_t i);
uint16_t synth_f64_to_f16(double x);
int synth_matrix_f16(uint16_t* out, int64_t rows, int64_t cols, uint64_t seed, uint64_t stream,
                     int dist, double param, int ndims, const int64_t* dims, const double* factors,
                     const uint8_t* rowsel, int nthreads);
int synth_set_columns_f16(uint16_t* out, int64_t rows, int64_t ld, uint64_t seed,
                          uint64_t stream, int ncols, const int64_t* cols, double lo, double hi);
int synth_choose(uint64_t seed, uint64_t stream, int64_t pool, int64_t count, uint64_t offset,
                 int64_t* out);

static volatile double sink;   /* keeps results live */

static void die(const char* what) {
    fprintf(stderr, "sanitize_driver: %s\n", what);
    exit(3);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) die("out of memory");
    return p;
}

/* fp16 bit patterns -> the nearest bf16 patterns (the bf16 cases) */
static void to_bf16(uint16_t* a, int64_t n) {
    for (int64_t i = 0; i < n; ++i) a[i] = oracle_bf16_encode(oracle_f16_decode(a[i]));
}

static void codecs(void) {
    double acc = 0.0;
    for (uint32_t h = 0; h < 65536u; ++h) {
        const double v = oracle_f16_decode((uint16_t)h);
        const float b = oracle_bf16_decode((uint16_t)h);
        if (!isnan(v)) acc += oracle_f16_encode(v);
        if (!isnan(b)) acc += oracle_bf16_encode(b);
    }
    const double specials[] = {0.0, -0.0, 1e-300, -1e-300, 65504.0, 65519.9, 65520.0, 1e300,
                               -1e300, INFINITY, -INFINITY, NAN, 3.4e38, 3.5e38, 1e-45, 5e-324};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i)
        acc += oracle_f16_encode(specials[i]) + oracle_bf16_encode(specials[i]) +
               synth_f64_to_f16(specials[i]);
    for (int q = -128; q <= 127; ++q) {
        const float scales[] = {0.0f, 1e-45f, 1e-38f, 0.02f, 1.0f, 65504.0f, 3e38f};
        for (size_t i = 0; i < sizeof scales / sizeof scales[0]; ++i)
            acc += oracle_dequant_weight_h((int8_t)q, scales[i], 0) +
                   oracle_dequant_weight_h((int8_t)q, scales[i], 1) +
                   oracle_dequant_weight((int8_t)q, scales[i]);
    }
    sink = acc + oracle_max_threads();
}

static void generator(int threads) {
    double acc = 0.0;
    for (uint64_t i = 0; i < 1000; ++i) acc += synth_uniform(3, 1, i) + synth_normal(3, 2, i);
    int64_t pick[40];
    if (synth_choose(5, 1, 40, 40, 0, pick) || synth_choose(5, 1, 40, 0, 7, pick) ||
        synth_choose(5, 1, 0, 0, 0, pick) || synth_choose(5, 1, 1, 1, 0, pick))
        die("synth_choose refused a valid call");
    if (synth_choose(5, 1, 3, 4, 0, pick) == 0) die("synth_choose took count > pool");
    uint16_t m[7 * 9];
    const int64_t dims[3] = {0, 4, 8};
    const double fac[3] = {20.0, -7.0, 0.5};
    uint8_t rowsel[3 * 7];
    for (int i = 0; i < 3 * 7; ++i) rowsel[i] = (uint8_t)(i % 2);
    if (synth_matrix_f16(m, 7, 9, 9, 1, 0, 1.0, 3, dims, fac, rowsel, threads) ||
        synth_matrix_f16(m, 7, 9, 9, 2, 1, 0.5, 3, dims, fac, NULL, threads) ||
        synth_matrix_f16(m, 7, 9, 9, 3, 0, 1.0, 0, NULL, NULL, NULL, threads) ||
        synth_matrix_f16(m, 0, 9, 9, 3, 0, 1.0, 0, NULL, NULL, NULL, threads))
        die("synth_matrix_f16 refused a valid call");
    const int64_t bad_dim[1] = {9};
    if (synth_matrix_f16(m, 7, 9, 9, 1, 0, 1.0, 1, bad_dim, fac, NULL, threads) == 0)
        die("synth_matrix_f16 took a column past the end");
    if (synth_set_columns_f16(m, 7, 9, 4, 1, 3, dims, 6.0, 60.0)) die("synth_set_columns_f16");
    if (synth_set_columns_f16(m, 7, 9, 4, 1, 1, bad_dim, 6.0, 60.0) == 0)
        die("synth_set_columns_f16 took a column past the end");
    for (int i = 0; i < 7 * 9; ++i) acc += m[i];
    sink = acc;
}

/* One whole-method call plus the step functions one by one, on seeded data
 * with two planted outlier columns, then the same call with every optional
 * output left to the oracle's own allocations. */
static void method_case(int64_t T, int64_t K, int64_t N, float tau, int ht, int with_w16,
                        int sample, int threads, uint64_t seed) {
    uint16_t* X = xmalloc(sizeof(uint16_t) * (size_t)(T * K));
    uint16_t* W = xmalloc(sizeof(uint16_t) * (size_t)(K * N));
    const int64_t dims[2] = {0, K - 1};
    const double fac[2] = {30.0, -25.0};
    if (synth_matrix_f16(X, T, K, seed, 1, 0, 1.0, K > 1 ? 2 : 1, dims, fac, NULL, threads) ||
        synth_matrix_f16(W, K, N, seed, 2, 1, 0.05, 0, NULL, NULL, NULL, threads))
        die("input generation");
    if (ht) { to_bf16(X, T * K); to_bf16(W, K * N); }
    /* an all-zero row and a row of the smallest positive pattern (in bf16,
       2^-133: 127/s then lies above the largest fp32) */
    if (T > 2)
        for (int64_t k = 0; k < K; ++k) { X[K + k] = 0; X[2 * K + k] = 1; }
    if (N > 1)   /* an all-zero weight column */
        for (int64_t k = 0; k < K; ++k) W[k * N + 1] = 0;

    int8_t* Wq = xmalloc((size_t)(N * K));
    float* sw = xmalloc(sizeof(float) * (size_t)N);
    if (ht) oracle_quantize_weight_typed(W, 1, K, N, Wq, sw, threads);
    else oracle_quantize_weight(W, K, N, Wq, sw, threads);

    const int64_t M = sample ? (T + 1) / 2 : T;
    int64_t* rows = xmalloc(sizeof(int64_t) * (size_t)M);
    for (int64_t m = 0; m < M; ++m) rows[m] = T - 1 - m;
    uint8_t* flag = xmalloc((size_t)K);
    int32_t* idx = xmalloc(sizeof(int32_t) * (size_t)K);
    int8_t* xq = xmalloc((size_t)(M * K));
    float* sx = xmalloc(sizeof(float) * (size_t)M);
    int32_t* acc = xmalloc(sizeof(int32_t) * (size_t)(M * N));
    uint16_t* Y = xmalloc(sizeof(uint16_t) * (size_t)(M * N));
    double* Y64 = xmalloc(sizeof(double) * (size_t)(M * N));
    const uint16_t* w16 = with_w16 ? W : NULL;
    const int64_t* rsel = sample ? rows : NULL;

    const int64_t o = oracle_mixed_matmul(X, T, K, Wq, sw, w16, N, tau, rsel, M, flag, idx, xq,
                                          sx, acc, Y, Y64, threads, ht);
    if (o < 0) die("oracle_mixed_matmul failed");

    oracle_detect(X, T, K, tau, flag, ht);
    const int64_t o2 = oracle_compact(flag, K, idx);
    oracle_quantize_rows(X, T, K, flag, rsel, M, xq, sx, ht);
    if (oracle_int8_gemm(xq, M, K, Wq, N, acc, threads) != 0) die("int32 overflow at small K");
    oracle_output(acc, sx, sw, X, w16, Wq, rsel, M, K, N, idx, o2, Y, NULL, threads, ht);
    if (o2 != o) die("outlier counts differ between calls");

    if (oracle_mixed_matmul(X, T, K, Wq, sw, w16, N, tau, rsel, M, NULL, NULL, NULL, NULL, NULL,
                            Y, NULL, threads, ht) != o)
        die("oracle_mixed_matmul with its own buffers");

    double s = 0.0;
    for (int64_t i = 0; i < M * N; ++i) s += Y[i] + Y64[i];
    sink = s;
    free(X); free(W); free(Wq); free(sw); free(rows); free(flag); free(idx); free(xq); free(sx);
    free(acc); free(Y); free(Y64);
}

/* fp32 and bf16 checkpoint columns with tiny, zero and mixed magnitudes */
static void typed_weights(int threads) {
    enum { K = 5, N = 6 };
    float W32[K * N];
    uint16_t W16b[K * N];
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            const float mags[N] = {1e-38f, 0.0f, 1e-45f, 2.5f, 3e38f, 1e-20f};
            W32[k * N + n] = (k % 2 ? -1.0f : 1.0f) * mags[n] * ((float)(k + 1) / (float)K);
            W16b[k * N + n] = oracle_bf16_encode(W32[k * N + n]);
        }
    int8_t Wq[N * K];
    float sw[N];
    oracle_quantize_weight_typed(W32, 2, K, N, Wq, sw, threads);
    oracle_quantize_weight_typed(W16b, 1, K, N, Wq, sw, threads);
    double s = 0.0;
    for (int i = 0; i < N * K; ++i) s += Wq[i];
    sink = s;
}

/* 127^2 * K past 2^31: the integer matmul counts the entries that do not fit */
static void gemm_overflow(void) {
    const int64_t K = 133145;
    int8_t* a = xmalloc((size_t)K);
    int8_t* b = xmalloc((size_t)(2 * K));
    memset(a, 127, (size_t)K);
    memset(b, 127, (size_t)K);
    memset(b + K, -127, (size_t)K);
    int32_t acc[2];
    if (oracle_int8_gemm(a, 1, K, b, 2, acc, 2) != 2) die("overflow count at K = 133145");
    free(a); free(b);
}

int main(void) {
    codecs();
    generator(3);
    typed_weights(1);
    typed_weights(4);
    gemm_overflow();
    const struct { int64_t T, K, N; } shapes[] = {
        {1, 1, 1}, {2, 4, 2}, {3, 17, 5}, {5, 64, 9}, {16, 130, 24}, {9, 33, 3}};
    const float taus[] = {0.0f, 6.0f, INFINITY};
    uint64_t seed = 11;
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        for (size_t j = 0; j < sizeof taus / sizeof taus[0]; ++j)
            for (int ht = 0; ht < 2; ++ht)
                for (int w16 = 0; w16 < 2; ++w16)
                    method_case(shapes[i].T, shapes[i].K, shapes[i].N, taus[j], ht, w16,
                                (int)((i + j) % 2), 1 + (int)(i % 3) * 2, ++seed);
    printf("sanitize_driver: done\n");
    return 0;
}
