/*
 * int8mm.h - C ABI of the LLM.int8() mixed-precision matrix multiplication
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (LLM.int8() abstract, taxoreview.com page dblp:280/8696,
 * second paragraph; restated in "LLM.int8(): A Procedure for Int8 Matrix
 * Multiplication in Transformer Language Models", section "The LLM.int8()
 * Methodology"):
 *
 *   Y = LLM.int8()(X, W, tau),  X fp16 [T,K], W fp16 [K,N], Y fp16 [T,N]
 *
 *   1. outlier feature dimensions: k is an outlier when |X[t,k]| >= tau for
 *      some row t (the pages pick outliers by magnitude; ">=" and the
 *      absolute threshold are this library's reading);
 *   2. vector-wise quantization, one normalization constant per inner
 *      product: s_x[t] = absmax of row t over non-outlier k, s_w[n] = absmax
 *      of column n of W; q = clamp(rint(v * fp32(127/s)), -127, 127), round
 *      half to even, s = 0 -> q = 0; outlier columns of Xq are 0;
 *   3. int8 matmul with int32 accumulation, acc = Xq . Wq^T, dequantized by
 *      the outer product of the scales: y8 = acc * s_x[t] * s_w[n] / 127^2;
 *   4. the isolated outlier dimensions go through a 16-bit matmul,
 *      y16 = sum over outlier k of X[t,k] * W[k,n] (fp16 operands, fp32
 *      accumulation), and Y = fp16(y8 + y16), rounded once.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless noted.  All buffers are owned by
 *     the caller; the library never allocates or frees memory on any call.
 *   - Matrices are row-major and dense (leading dimension = row length),
 *     except the converted weight, whose layout int8_quantize_weight gives.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return without synchronizing; results are valid
 *     once the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-zero status nothing was enqueued, except INT8MM_E_HIP, which
 *     reports a launch failure from the HIP runtime.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified results.
 *   - Calls on different streams may run concurrently when they use
 *     different workspaces and outputs.  The library holds no mutable global
 *     state.
 *   - Shape limits: T, K, N >= 1; K % 16 == 0; N % 8 == 0; K <= 133136 (the
 *     largest multiple of 16 with 127*127*K < 2^31, so int32 accumulators
 *     cannot overflow); T <= 2^24 - 1 and T*N <= 2^38 (launch-grid limits).
 *     Every pointer must be 16-byte aligned.
 */
#ifndef INT8MM_H
#define INT8MM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    INT8MM_OK = 0,
    INT8MM_E_NULL = 1,        /* a required pointer is NULL */
    INT8MM_E_SHAPE = 2,       /* T, K or N outside the limits above */
    INT8MM_E_TAU = 3,         /* tau is NaN or negative */
    INT8MM_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    INT8MM_E_WORKSPACE = 5,   /* workspace smaller than the size query returns */
    INT8MM_E_UNSUPPORTED = 6, /* a request the library does not implement: a checkpoint
                                 type code other than the INT8MM_WEIGHT_* values */
    INT8MM_E_HIP = 7          /* the HIP runtime reported a launch error */
} int8mm_status;

#define INT8MM_MAX_K 133136
#define INT8MM_MAX_T 16777215
#define INT8MM_MAX_TN 274877906944.0 /* 2^38 */

/* Static, human-readable name of a status code (host only; never NULL). */
const char* int8mm_status_string(int status);

/* Bytes of device workspace that int8_mixed_matmul and its variants need
 * for this shape (host only, enqueues nothing).  The size covers the
 * worst case in which every hidden dimension is an outlier, and (except
 * for the decode shapes that run as a single kernel: T <= 16, K 4096 or
 * 8192, T*K <= 65536) room for min(K, 512) outlier rows of N 16-bit values
 * into which the memory-halved variant (W16 = NULL) recovers the outlier
 * rows of W once per call (with more outliers, or without that room, the
 * matmul recovers them itself, more slowly).  For long K (>= 24576, or
 * >= 8192 past 256 rows) with a partial last round of 256 x 256 output
 * tiles on the current device, the matmul splits K in two and the size
 * also covers, per
 * output tile, two 256 KB blocks of int32 partial sums and a counter; this
 * part depends on N and on the device's compute-unit count (256 when no
 * device can be queried).  For up to 256 rows with K a multiple of 128 and
 * at least 4096, whose output tiles (256 x 128 one per compute unit past
 * 128 rows when K is not split in two as above and the N / 128 column
 * tiles fit the device, 128 x 128 one per compute unit past 64 rows,
 * 64 x 64 two per compute unit below) occupy at most half (256 x 128 and
 * 128 x 128) or a quarter (64 x 64) of the slots, the matmul splits K into
 * S = min(slots / tiles, K / 2048, 8) slabs and the size covers, per tile,
 * S blocks of int32 partial sums of the tile's size and a counter.  A
 * workspace at least as large as the size without the split part is
 * accepted and runs the matmul without the split.
 * For few rows with a long K (K a multiple of 1024, T*K > 131072, and T <= 8,
 * or T <= 16 with K >= 32768)
 * the size covers, instead of the recovered rows and the split, S slabs of
 * int32 partial sums [S][T][N] (S = ceil(K / (1024 * floor(128 / T))) + 3,
 * at most K / 1024): the decode kernel then streams K in slabs; without that
 * room these shapes run through the matmul kernels.
 * bytes: host pointer, receives the size.  Errors: E_NULL, E_SHAPE. */
int int8_mixed_matmul_workspace_size(int64_t T, int64_t K, int64_t N, size_t* bytes);

/* Bytes of the converted weight Wq for a [K,N] weight (host only, enqueues
 * nothing); currently K*N.  Callers size Wq with this query: the layout is
 * the library's (see int8_quantize_weight).  Errors: E_NULL, E_SHAPE. */
int int8_quantize_weight_size(int64_t K, int64_t N, size_t* bytes);

/* Weight conversion to Int8 ("converted to Int8" at load time, LLM.int8()
 * abstract): column-wise absmax quantization, one scale per output column
 * n (one per inner product).
 *   W16: fp16 [K,N] row-major (read only)
 *   Wq:  int8, int8_quantize_weight_size() bytes (written): the transpose of
 *        W, [N,K], in a panel-blocked layout.  Rows n are grouped in panels
 *        of 256 (the last panel has N % 256 rows when that is not 0); a
 *        panel's K range is cut into k-tiles of 64 columns (the last one is
 *        K % 64 wide when that is not 0); each (panel, k-tile) block is
 *        stored row-major, blocks follow each other in k order inside a
 *        panel and panels in row order, with no padding.  Element (n, k),
 *        with p0 = n - n % 256, rows = min(256, N - p0), k0 = k - k % 64 and
 *        w = min(64, K - k0), is at byte
 *            p0*K + k0*rows + (n - p0)*w + (k - k0).
 *        (16 consecutive rows of one k-tile are one contiguous kilobyte,
 *        which is how the matmul kernels copy them.)
 *   sw:  fp32 [N] column scales s_w[n] = max_k |W[k,n]| (written)
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_HIP. */
int int8_quantize_weight(const void* W16, int64_t K, int64_t N, int8_t* Wq, float* sw,
                         void* stream);

/* Checkpoint types accepted by int8_quantize_weight_typed. */
enum {
    INT8MM_WEIGHT_F16 = 0,   /* IEEE binary16 */
    INT8MM_WEIGHT_BF16 = 1,  /* bfloat16 (upper half of binary32) */
    INT8MM_WEIGHT_F32 = 2    /* IEEE binary32 */
};

/* Weight conversion from a 16- or 32-bit checkpoint (LLM.int8() abstract: a
 * 16/32-bit checkpoint is loaded, converted to Int8 and used immediately).
 * The column scale and the codes are taken on the checkpoint's own values:
 * s_w[n] = max_k |W[k,n]|, Wq[n,k] = clamp(rint(W[k,n] * fp32(127/s_w[n]))).
 *   W:     [K,N] row-major of type wtype (read only)
 *   Wq, sw: as int8_quantize_weight (written)
 *   W16_out: NULL, or fp16 [K,N] (written): W rounded to fp16 (nearest
 *          even), the 16-bit weight of the outlier path for checkpoints that
 *          are not fp16.  With the memory-halved variant (W16 = NULL in the
 *          matmul) no 16-bit copy is needed.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_UNSUPPORTED (unknown wtype), E_HIP. */
int int8_quantize_weight_typed(const void* W, int wtype, int64_t K, int64_t N, int8_t* Wq,
                               float* sw, void* W16_out, void* stream);

/* The whole LLM.int8() matmul (steps 1-4 above) on a converted weight.
 *   X:   fp16 [T,K] activations (read only)
 *   Wq, sw: from int8_quantize_weight for the same K and N (read only)
 *   W16: fp16 [K,N], the 16-bit weight; only its outlier rows are read.
 *        NULL selects the memory-halved variant (only the Int8 weight is
 *        kept, LLM.int8() abstract: inference memory cut by half): the
 *        outlier rows are recovered from Wq as
 *        W^[k,n] = fp16(fp32(Wq[n,k] * fp32(sw[n] / 127))).
 *   tau: outlier threshold, tau >= 0 (+inf: no outliers; 0: every
 *        dimension is an outlier and Y is the fp16 matmul)
 *   Y:   fp16 [T,N] (written)
 *   workspace: device buffer of at least the size query's bytes; its
 *        contents on entry are ignored and on return are unspecified.
 * Errors: E_NULL, E_SHAPE, E_TAU, E_ALIGN, E_WORKSPACE, E_HIP. */
int int8_mixed_matmul(const void* X, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                      const void* W16, int64_t N, float tau, void* Y, void* workspace,
                      size_t workspace_bytes, void* stream);

/* int8_mixed_matmul that also writes its intermediates (for bit-exact
 * checking).  Each output may be NULL to skip it:
 *   count: int32 [1]   number of outlier dimensions o
 *   idx:   int32 [K]   outlier dimensions, ascending, in idx[0..o)
 *   xq:    int8  [T,K] quantized activations (outlier columns 0)
 *   sx:    fp32  [T]   row scales
 *   acc:   int32 [T,N] int8 matmul accumulators before dequantization
 * It runs the same kernels as int8_mixed_matmul (the single-kernel decode
 * path when the shape qualifies, the staged kernels otherwise) and adds
 * only the stores of the intermediates.
 * Errors: as int8_mixed_matmul. */
int int8_mixed_matmul_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                            const float* sw, const void* W16, int64_t N, float tau, void* Y,
                            void* workspace, size_t workspace_bytes, void* stream,
                            int32_t* count, int32_t* idx, int8_t* xq, float* sx, int32_t* acc);

/* The bf16 variant of the whole path ("16-bit" is not fixed by the pages):
 * X, W16 and Y are bfloat16 instead of fp16; every step is the same (values
 * widen to fp32 exactly, the 16-bit matmul multiplies bf16 values with fp32
 * accumulation, Y is rounded once to the nearest bf16, ties to even; a
 * recovered weight value (W16 = NULL) is rounded to bf16).  Wq and sw come
 * from int8_quantize_weight_typed on the bf16 (or any) checkpoint.
 * Arguments, workspace and errors as int8_mixed_matmul. */
int int8_mixed_matmul_bf16(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                           const float* sw, const void* W16, int64_t N, float tau, void* Y,
                           void* workspace, size_t workspace_bytes, void* stream);

/* int8_mixed_matmul_debug for the bf16 variant. */
int int8_mixed_matmul_bf16_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                 const float* sw, const void* W16, int64_t N, float tau, void* Y,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t* count, int32_t* idx, int8_t* xq, float* sx,
                                 int32_t* acc);

/* Steps 1-2 on the activation side only: finds the outlier dimensions,
 * quantizes X row-wise and gathers the outlier columns of X, all into the
 * workspace.  Lets several weights that share one X (e.g. the query, key
 * and value projections) reuse one pass, and lets a profiler time the
 * matmul by itself.  Arguments as int8_mixed_matmul; N is only used for
 * the workspace size check.
 * Errors: E_NULL, E_SHAPE, E_TAU, E_ALIGN, E_WORKSPACE, E_HIP. */
int int8mm_quantize_activations(const void* X, int64_t T, int64_t K, int64_t N, float tau,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Steps 3-4 on a workspace filled by int8mm_quantize_activations with the
 * same T and K.  The activation part of the workspace is only read here and
 * may be reused for any number of weights (any N the workspace size
 * covers); the recovered-rows, K-split and K-slab parts (see the size
 * query) are scratch of this call, so matmuls on one workspace run one after another
 * (one stream).  X is read only through the gathered copy in the
 * workspace.  Arguments as int8_mixed_matmul.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_HIP. */
int int8mm_matmul_prepared(void* workspace, size_t workspace_bytes, int64_t T, int64_t K,
                           const int8_t* Wq, const float* sw, const void* W16, int64_t N,
                           void* Y, void* stream);

/* int8_mixed_matmul without a workspace argument and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a scratch array of 128 MiB (134217728 bytes) inside the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends; the first call on a GPU (with it current) looks its address
 * up, so make that call outside graph capture.  Every call on one GPU uses
 * the same array: calls that overlap on one GPU (different streams, or
 * threads) race and give unspecified results; serialize them.  Shapes
 * whose workspace without the optional regions exceeds the scratch are
 * rejected (E_WORKSPACE): about 3*T*K bytes, e.g. T*K up to about 44
 * million; the optional regions (recovered outlier rows, K split, K slabs)
 * are used when they fit as well.  Arguments, results and the other errors
 * as int8_mixed_matmul; E_UNSUPPORTED for a device index of 256 or more. */
int int8_mixed_matmul_noalloc(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                              const float* sw, const void* W16, int64_t N, float tau, void* Y,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INT8MM_H */
