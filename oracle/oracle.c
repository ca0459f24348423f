/*
 * ORACLE - TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the LLM.int8()
 * mixed-precision matrix multiplication.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section; the pages carry no equations):
 *   [A]  LLM.int8() abstract (taxoreview.com page, dblp:280/8696, second
 *        paragraph): Int8 matmul for feed-forward and attention projections;
 *        vector-wise quantization with a separate normalization constant per
 *        inner product; emergent outlier feature dimensions isolated into a
 *        16-bit matrix multiplication, with more than 99.9% of values still
 *        multiplied in 8-bit; a 16/32-bit checkpoint converted to Int8 at load.
 *   [S]  "LLM.int8(): A Procedure for Int8 Matrix Multiplication in
 *        Transformer Language Models" (summarizepaper.com, arXiv 2208.07339v1),
 *        section "The LLM.int8() Methodology" and the bullet summary: outlier
 *        features are picked out by their magnitude.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - a hidden dimension k is an outlier when |X[t,k]| >= tau for at least
 *     one row t (">=": tau = 0 makes every dimension an outlier);
 *   - symmetric absmax quantization to [-127, 127]:
 *       q = clamp(rint(x * fp32(127 / s)), -127, 127),
 *     the divide an IEEE fp32 divide, the product one fp32 multiply, rint
 *     rounding half to even; s = 0 gives q = 0; fp32(127/s) has no upper
 *     exponent limit (it would overflow for s < ~3.7e-37);
 *   - the row scale s_x[t] is the absmax of row t over non-outlier columns
 *     only; outlier columns of Xq are 0;
 *   - the column scale s_w[n] is the absmax of column n of W over all K rows;
 *   - dequantization: y8 = acc * s_x[t] * s_w[n] / 127^2 (fp64 here);
 *   - the 16-bit part multiplies the fp16 values X[t,k] and W[k,n] of the
 *     outlier dimensions exactly (fp64 here);
 *   - Y = fp16(y8 + y16), rounded once, to nearest even;
 *   - memory-halved variant (no 16-bit weight kept, [A]: inference memory
 *     "cut by half"): the outlier rows of W are recovered from the Int8
 *     weight, W^[k,n] = fp16(fp32(q[n,k] * fp32(s_w[n] / 127))) (an IEEE fp32
 *     divide, one fp32 multiply, one rounding to fp16, each to nearest even),
 *     and the 16-bit part multiplies X[t,k] by W^[k,n] instead;
 *   - bf16 variant ("16-bit" is not specified on the pages): X, W16 and Y
 *     are bfloat16 instead of fp16; every step is the same, values widen to
 *     fp32 exactly, Y is rounded once to the nearest bf16 (ties to even) and
 *     a recovered weight value is rounded to bf16.
 *
 * Parity pins: every function below is checked in tests/ against values
 * that do not come from this file (hand-derived examples, closed forms,
 * numpy library routines, invariants); see tests/test_oracle_*.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------ fp16 codec */

/* Exact value of an IEEE binary16 bit pattern. */
static double oh_decode(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                 /* subnormal or zero */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);             /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest binary16 to a double, ties to even (one rounding). */
static uint16_t oh_encode(double x) {
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* Largest finite is 65504 = 2047 * 2^5; halfway to 65536 is 65520 and the
       tie goes to the even neighbour, which is 2^16 = overflow. */
    if (a >= 65520.0) return sign | 0x7C00;
    /* Find the binade: the largest e with 2^e <= a, clamped at -14 so that
       subnormals share the 2^-24 step of the lowest binade. */
    int e = -14;
    while (e < 15 && ldexp(1.0, e + 1) <= a) ++e;
    double step = ldexp(1.0, e - 10);
    double q = a / step;                                    /* exact: power-of-two divide */
    double fl = floor(q);
    double frac = q - fl;
    double n = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    /* n * step is the rounded magnitude; re-encode it. */
    double r = n * step;
    if (r >= 65536.0) return sign | 0x7C00;
    if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
    int be = -14;
    while (ldexp(1.0, be + 1) <= r) ++be;
    int mant = (int)(r / ldexp(1.0, be - 10)) - 1024;
    return sign | (uint16_t)(((be + 15) << 10) | mant);
}

double oracle_f16_decode(uint16_t h) { return oh_decode(h); }
uint16_t oracle_f16_encode(double x) { return oh_encode(x); }

/* fp32 value of an fp16 element (exact: binary16 is a subset of binary32). */
static float oh_f32(uint16_t h) { return (float)oh_decode(h); }

/* ------------------------------------------------------------ bf16 codec */

/* bfloat16: the upper 16 bits of an IEEE binary32 (exact widening). */
float oracle_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bfloat16 to a double, ties to even (one rounding): 8 significant
 * bits, the binary32 exponent range, subnormal step 2^-133. */
uint16_t oracle_bf16_encode(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* Largest finite is (2 - 2^-7) * 2^127; halfway to 2^128 is
       (2 - 2^-8) * 2^127, and that tie goes to the even neighbour 2^128. */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7F80;
    int e = -126;                                   /* subnormals share 2^-133 */
    if (a >= ldexp(1.0, -126)) e = ilogb(a);        /* 2^e <= a < 2^(e+1) */
    double step = ldexp(1.0, e - 7);
    double q = a / step;                            /* exact: power-of-two divide */
    double fl = floor(q);
    double frac = q - fl;
    double n = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    float r = (float)(n * step);                    /* exact: a bfloat16 value */
    uint32_t u;
    memcpy(&u, &r, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* The 16-bit element types of X, W16 and Y: 0 = fp16, 1 = bf16. */
static double h_decode(int ht, uint16_t b) { return ht ? (double)oracle_bf16_decode(b) : oh_decode(b); }
static float h_f32(int ht, uint16_t b) { return (float)h_decode(ht, b); }
static uint16_t h_encode(int ht, double x) { return ht ? oracle_bf16_encode(x) : oh_encode(x); }

/* ---------------------------------------------------- the quantizer itself */

/* Symmetric absmax quantization of one value with scale s (see header).
 * fp32(127/s) is the quotient rounded to nearest even at 24 significant
 * bits, as an IEEE fp32 divide gives it; for s below about 3.7e-37 (bf16 or
 * fp32 values only, never fp16) that quotient lies above the largest fp32,
 * and it is read with an unbounded exponent instead of overflowing.  The
 * quotient is formed in double first: rounding 53 bits and then 24 is the
 * same as rounding 24 once for a quotient of 24-bit numbers. */
static int8_t quant_one(float x, float s) {
    if (s == 0.0f) return 0;
    int e;
    double m = frexp(127.0 / (double)s, &e);      /* 127/s = m * 2^e, 0.5 <= m < 1 */
    double r = ldexp((double)(float)m, e);        /* 24 significant bits, exponent unbounded */
    float p = (float)((double)x * r);             /* exact 48-bit product, rounded to fp32 once */
    float q = rintf(p);             /* round half to even */
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    return (int8_t)q;
}

/* ------------------------------------------------------------- threading */

typedef struct {
    void (*fn)(void*, int64_t, int64_t);
    void* ctx;
    int64_t lo, hi;
} o_job;

static void* o_run(void* p) {
    o_job* j = (o_job*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static int o_threads(int n) {
    if (n > 0) return n > 256 ? 256 : n;
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c < 1 ? 1 : (c > 256 ? 256 : (int)c);
}

/* Runs fn over [0, n) split into contiguous ranges; the arithmetic of each
   index does not depend on the split. */
static void o_parallel(int64_t n, int nthreads, void (*fn)(void*, int64_t, int64_t), void* ctx) {
    int nt = o_threads(nthreads);
    if (nt > n) nt = (int)(n > 0 ? n : 1);
    if (nt <= 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    int ok[256];
    o_job jobs[256];
    for (int t = 0; t < nt; ++t) {
        jobs[t] = (o_job){fn, ctx, n * t / nt, n * (t + 1) / nt};
        ok[t] = pthread_create(&th[t], NULL, o_run, &jobs[t]) == 0;
        if (!ok[t]) o_run(&jobs[t]);
    }
    for (int t = 0; t < nt; ++t) if (ok[t]) pthread_join(th[t], NULL);
}

int oracle_max_threads(void) { return o_threads(0); }

/* --------------------------------------------- step: weight quantization */

/* Column-wise ("vector-wise", one constant per inner product) absmax int8
 * conversion of a 16- or 32-bit checkpoint weight [A]: for every output
 * column n,
 *   s_w[n] = max_k |W[k,n]|,  Wq[n,k] = quant(W[k,n], s_w[n]),
 * on the checkpoint's own values (fp16 and bf16 widen to fp32 exactly).
 * W is [K,N] row-major of type 0 = fp16, 1 = bf16, 2 = fp32; Wq is stored
 * [N,K] (K contiguous). */
typedef struct { const void* W; int type; int64_t K, N; int8_t* Wq; float* sw; } qw_ctx;

static float w_value(const qw_ctx* c, int64_t i) {
    if (c->type == 1) return oracle_bf16_decode(((const uint16_t*)c->W)[i]);
    if (c->type == 2) return ((const float*)c->W)[i];
    return oh_f32(((const uint16_t*)c->W)[i]);
}

static void qw_span(void* p, int64_t lo, int64_t hi) {
    qw_ctx* c = (qw_ctx*)p;
    for (int64_t n = lo; n < hi; ++n) {
        float s = 0.0f;
        for (int64_t k = 0; k < c->K; ++k) {
            float a = fabsf(w_value(c, k * c->N + n));
            if (a > s) s = a;
        }
        c->sw[n] = s;
        for (int64_t k = 0; k < c->K; ++k)
            c->Wq[n * c->K + k] = quant_one(w_value(c, k * c->N + n), s);
    }
}

void oracle_quantize_weight_typed(const void* W, int type, int64_t K, int64_t N, int8_t* Wq,
                                  float* sw, int nthreads) {
    qw_ctx c = {W, type, K, N, Wq, sw};
    o_parallel(N, nthreads, qw_span, &c);
}

void oracle_quantize_weight(const uint16_t* W, int64_t K, int64_t N, int8_t* Wq, float* sw,
                            int nthreads) {
    oracle_quantize_weight_typed(W, 0, K, N, Wq, sw, nthreads);
}

/* ---------------------------------------------- step: outlier detection */

/* Outlier feature dimensions [A], found by magnitude [S]:
 *   flag[k] = 1 iff |X[t,k]| >= tau for some row t.
 * The 16-bit value (fp16 or bf16, type ht) is compared exactly (in fp32). */
void oracle_detect(const uint16_t* X, int64_t T, int64_t K, float tau, uint8_t* flag, int ht) {
    for (int64_t k = 0; k < K; ++k) {
        flag[k] = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (fabsf(h_f32(ht, X[t * K + k])) >= tau) { flag[k] = 1; break; }
        }
    }
}

/* Isolation of the outlier dimensions [A]: their indices in ascending order.
 * Returns the count o. */
int64_t oracle_compact(const uint8_t* flag, int64_t K, int32_t* idx) {
    int64_t o = 0;
    for (int64_t k = 0; k < K; ++k)
        if (flag[k]) idx[o++] = (int32_t)k;
    return o;
}

/* ------------------------------------------- step: row-wise quantization */

/* Vector-wise quantization of the activations [A]: one constant per row t
 * (per inner product), taken over the non-outlier columns only:
 *   s_x[t] = max_{k not outlier} |X[t,k]|  (0 when there is none),
 *   Xq[t,k] = 0 for outlier k, else quant(X[t,k], s_x[t]).
 * rows == NULL quantizes every row; otherwise row m of the output is row
 * rows[m] of X (a sample). */
void oracle_quantize_rows(const uint16_t* X, int64_t T, int64_t K, const uint8_t* flag,
                          const int64_t* rows, int64_t M, int8_t* Xq, float* sx, int ht) {
    (void)T;
    for (int64_t m = 0; m < M; ++m) {
        int64_t t = rows ? rows[m] : m;
        const uint16_t* xr = X + t * K;
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (flag[k]) continue;
            float a = fabsf(h_f32(ht, xr[k]));
            if (a > s) s = a;
        }
        sx[m] = s;
        for (int64_t k = 0; k < K; ++k)
            Xq[m * K + k] = flag[k] ? 0 : quant_one(h_f32(ht, xr[k]), s);
    }
}

/* ---------------------------------------------------- step: int8 matmul */

/* Int8 matrix multiplication [A] with exact integer accumulation:
 *   acc[m,n] = sum_k Xq[m,k] * Wq[n,k]
 * in int64, then checked to fit int32.  Returns the number of entries that
 * do not fit (0 for K <= 133144, since 127^2 * K < 2^31 there). */
typedef struct {
    const int8_t* Xq; int64_t M, K; const int8_t* Wq; int64_t N; int32_t* acc; int64_t bad;
    pthread_mutex_t lock;
} gemm_ctx;

static void gemm_span(void* p, int64_t lo, int64_t hi) {
    gemm_ctx* c = (gemm_ctx*)p;
    int64_t bad = 0;
    for (int64_t m = lo; m < hi; ++m) {
        const int8_t* a = c->Xq + m * c->K;
        for (int64_t n = 0; n < c->N; ++n) {
            const int8_t* b = c->Wq + n * c->K;
            int64_t s = 0;
            for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
            if (s > INT32_MAX || s < INT32_MIN) ++bad;
            c->acc[m * c->N + n] = (int32_t)s;
        }
    }
    pthread_mutex_lock(&c->lock);
    c->bad += bad;
    pthread_mutex_unlock(&c->lock);
}

/* Splits over n instead of m when there are fewer rows than threads. */
static void gemm_span_cols(void* p, int64_t lo, int64_t hi) {
    gemm_ctx* c = (gemm_ctx*)p;
    int64_t bad = 0;
    for (int64_t m = 0; m < c->M; ++m) {
        const int8_t* a = c->Xq + m * c->K;
        for (int64_t n = lo; n < hi; ++n) {
            const int8_t* b = c->Wq + n * c->K;
            int64_t s = 0;
            for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
            if (s > INT32_MAX || s < INT32_MIN) ++bad;
            c->acc[m * c->N + n] = (int32_t)s;
        }
    }
    pthread_mutex_lock(&c->lock);
    c->bad += bad;
    pthread_mutex_unlock(&c->lock);
}

int64_t oracle_int8_gemm(const int8_t* Xq, int64_t M, int64_t K, const int8_t* Wq, int64_t N,
                         int32_t* acc, int nthreads) {
    gemm_ctx c;
    c.Xq = Xq; c.M = M; c.K = K; c.Wq = Wq; c.N = N; c.acc = acc; c.bad = 0;
    pthread_mutex_init(&c.lock, NULL);
    if (M >= o_threads(nthreads)) o_parallel(M, nthreads, gemm_span, &c);
    else o_parallel(N, nthreads, gemm_span_cols, &c);
    pthread_mutex_destroy(&c.lock);
    return c.bad;
}

/* ------------------------------- step: dequantize, outlier part, output */

/* Dequantization by the outer product of the two scale vectors plus the
 * 16-bit matrix multiplication over the isolated outlier dimensions [A]:
 *   y8  = acc[m,n] * s_x[m] * s_w[n] / 127^2
 *   y16 = sum_{j<o} X[t,idx_j] * W[idx_j,n]       (t = rows[m] or m)
 *   Y   = fp16(y8 + y16)   (bf16 when ht = 1: the bf16 variant of the path)
 * all in fp64 (fp16 x fp16 and bf16 x bf16 products are exact there).  Y64, when given,
 * receives y8 + y16 before the final rounding.  Without W16 (NULL), the
 * memory-halved variant: W[idx_j,n] is the fp16 value recovered from the
 * Int8 weight, see oracle_dequant_weight. */
typedef struct {
    const int32_t* acc; const float* sx; const float* sw; const uint16_t* X; const uint16_t* W16;
    const int8_t* Wq; const int64_t* rows; int64_t M, K, N; const int32_t* idx; int64_t o;
    uint16_t* Y; double* Y64; int ht;
} out_ctx;

/* The 16-bit value (type ht) of weight element (k, n) recovered from its
 * Int8 code q = Wq[n,k] and column scale s_w[n]: fp16(fp32(q * fp32(s_w/127)))
 * (bf16 for ht = 1), each step rounded to nearest even (the divide an IEEE
 * fp32 divide). */
uint16_t oracle_dequant_weight_h(int8_t q, float sw, int ht) {
    const float d = sw / 127.0f;
    const float v = (float)q * d;
    return h_encode(ht, (double)v);
}

uint16_t oracle_dequant_weight(int8_t q, float sw) { return oracle_dequant_weight_h(q, sw, 0); }

static void out_span(void* p, int64_t lo, int64_t hi) {
    out_ctx* c = (out_ctx*)p;
    for (int64_t m = lo; m < hi; ++m) {
        int64_t t = c->rows ? c->rows[m] : m;
        for (int64_t n = 0; n < c->N; ++n) {
            double y8 = (double)c->acc[m * c->N + n] * (double)c->sx[m] * (double)c->sw[n] / 16129.0;
            double y16 = 0.0;
            for (int64_t j = 0; j < c->o; ++j) {
                int64_t k = c->idx[j];
                const uint16_t w = c->W16 ? c->W16[k * c->N + n]
                                          : oracle_dequant_weight_h(c->Wq[n * c->K + k], c->sw[n], c->ht);
                y16 += h_decode(c->ht, c->X[t * c->K + k]) * h_decode(c->ht, w);
            }
            double y = y8 + y16;
            if (c->Y64) c->Y64[m * c->N + n] = y;
            c->Y[m * c->N + n] = h_encode(c->ht, y);
        }
    }
}

void oracle_output(const int32_t* acc, const float* sx, const float* sw, const uint16_t* X,
                   const uint16_t* W16, const int8_t* Wq, const int64_t* rows, int64_t M,
                   int64_t K, int64_t N, const int32_t* idx, int64_t o, uint16_t* Y, double* Y64,
                   int nthreads, int ht) {
    out_ctx c = {acc, sx, sw, X, W16, Wq, rows, M, K, N, idx, o, Y, Y64, ht};
    o_parallel(M, nthreads, out_span, &c);
}

/* ----------------------------------------------------- the whole method */

/* All steps in the pages' order, on a quantized weight (Wq, s_w) and the
 * 16-bit weight W16 (NULL: the memory-halved variant), with X, W16 and Y of
 * 16-bit type ht (0 fp16, 1 bf16): detect -> isolate ->
 * quantize rows -> int8 matmul -> dequantize + 16-bit outlier matmul.  Detection always looks at all T rows
 * of X; the other steps run on the M rows listed in `rows` (all when NULL).
 * Outputs (any but Y may be NULL): flag[K], idx[K], Xq[M,K], sx[M],
 * acc[M,N], Y[M,N], Y64[M,N].  Returns o, or -1 on allocation failure,
 * or -2 when an accumulator does not fit int32. */
int64_t oracle_mixed_matmul(const uint16_t* X, int64_t T, int64_t K, const int8_t* Wq,
                            const float* sw, const uint16_t* W16, int64_t N, float tau,
                            const int64_t* rows, int64_t M,
                            uint8_t* flag_out, int32_t* idx_out, int8_t* xq_out, float* sx_out,
                            int32_t* acc_out, uint16_t* Y, double* Y64, int nthreads, int ht) {
    if (!rows) M = T;
    uint8_t* flag = flag_out ? flag_out : (uint8_t*)malloc((size_t)K);
    int32_t* idx = idx_out ? idx_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int8_t* xq = xq_out ? xq_out : (int8_t*)malloc((size_t)(M * K));
    float* sx = sx_out ? sx_out : (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc = acc_out ? acc_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * N));
    int64_t o = -1;
    if (flag && idx && xq && sx && acc) {
        oracle_detect(X, T, K, tau, flag, ht);
        o = oracle_compact(flag, K, idx);
        oracle_quantize_rows(X, T, K, flag, rows, M, xq, sx, ht);
        if (oracle_int8_gemm(xq, M, K, Wq, N, acc, nthreads) != 0) o = -2;
        else oracle_output(acc, sx, sw, X, W16, Wq, rows, M, K, N, idx, o, Y, Y64, nthreads, ht);
    }
    if (!flag_out) free(flag);
    if (!idx_out) free(idx);
    if (!xq_out) free(xq);
    if (!sx_out) free(sx);
    if (!acc_out) free(acc);
    return o;
}
