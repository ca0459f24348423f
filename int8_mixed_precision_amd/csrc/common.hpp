// Internal declarations shared by the HIP translation units of libint8mm.
// Not part of the public ABI (that is include/int8mm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint16_t v8u16 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// 16-bit element type of X, W16 and Y (and of the gathered outlier columns):
// fp16, or bf16 for the bf16 variant.  Kernels store them as raw 16-bit
// patterns and convert with these helpers.
constexpr int kHalfF16 = 0, kHalfBF16 = 1;

template <int HT>
__device__ __forceinline__ float h16_to_f32(uint16_t b) {
    if constexpr (HT == kHalfBF16) return __builtin_bit_cast(float, (uint32_t)b << 16);
    else return (float)__builtin_bit_cast(_Float16, b);
}

// Packed unsigned max of two pairs of 16-bit lanes (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// fp32 -> 16-bit, round to nearest even
template <int HT>
__device__ __forceinline__ uint16_t f32_to_h16(float f) {
    if constexpr (HT == kHalfBF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
    else return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Device workspace of one activation pass.  All regions are 256-byte aligned.
//   flags   u32 [kw]     bit k%32 of word k/32 set when dimension k is an outlier;
//           past 128 rows with K <= 49152, [kDetectParts][kwp]: one partial
//           bitmap per row group of the detection, to be ORed (kwp = kw
//           rounded up to 64 words)
//   wprefix i32 [kw]     number of outlier dimensions before word w
//   count   i32 [4]      count[0] = o, count[1] = o rounded up to 16
//   segmax  f32 [nseg][16], segcnt i32 [nseg]   per 2048-column segment, the
//           row maxima over its non-outlier columns and its outlier count
//           (activation pass for T <= 16 only; nseg = ceil(K / 2048))
//   idx     i32 [K]      outlier dimensions, ascending
//   sx      f32 [T]      row scales
//   xq      i8  [T,K]    quantized activations, outlier columns 0
//   xo      16-bit [T,opad] outlier columns of X, row stride count[1], zero padded
//   wrec    16-bit [min(K, kRecoverRows), N]  the outlier rows of W recovered from
//           Wq for the memory-halved variant, row j = outlier j (present when the
//           workspace is large enough for it)
// and, only when the matmul splits K (gemm_ksplit), after all of the above:
//   ks_count i32 [nsplit]            per split tile, parts finished (zeroed by
//                                    the call's activation pass or the matmul's launch)
//   ks_part  i32 [nsplit][2][65536]  each half's int32 sums of its 256 x 256 tile
//                                    (large-tile kernel, T > 128), or
//            i32 [tiles][S][BM*BN]   each K slab's sums of its tile (streaming
//                                    kernel up to 256 rows, stream_split)
// or, for few rows with a long K (decode_split_reserve), instead of wrec and
// the split:
//   dpart    i32 [dslabs][T][N]     each K slab's int32 sums
struct Workspace {
    uint32_t* flags;
    int32_t* wprefix;
    int32_t* count;
    float* segmax;
    int32_t* segcnt;
    int32_t* idx;
    float* sx;
    int8_t* xq;
    uint16_t* xo;
    uint16_t* wrec;      // NULL when the workspace has no room for it
    int64_t wrec_rows;
    int32_t* ks_count;   // NULL without the K split
    int32_t* ks_part;
    int32_t* dpart;      // decode K slabs: int32 partial sums [dslabs][T][N], or NULL
    int dslabs;          // slabs the dpart region holds (0 without it)
    size_t bytes;        // total bytes the layout needs
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The quantizer q = rint(x * fp32(127/s)) reads fp32(127/s) with an
// unbounded exponent: for s below about 3.7e-37 (bf16 or fp32 values only;
// an fp16 scale is at least 2^-24) the fp32 quotient would overflow.  Below
// 2^-64 both s and x are multiplied by 2^64 first: the scalings are exact,
// the quotient 127/(s * 2^64) is a normal fp32 equal to fp32(127/s) * 2^-64,
// and (x * 2^64) * that quotient is the same product x * fp32(127/s).
// Kernels take r = 127 / (s * qfactor(s)) and quantize x * qfactor(s).
__device__ __forceinline__ float qfactor(float s) { return s < 0x1p-64f ? 0x1p64f : 1.0f; }

// A weight value recovered from its Int8 code q and column scale s_w
// (memory-halved variant): fp16(fp32(q * fp32(s_w / 127))) (bf16 for the bf16
// variant).  The product is rounded to fp32 first: the empty asm keeps the
// compiler from fusing the multiply and the conversion into one
// v_fma_mixlo_f16 (a single rounding of the exact product straight to fp16).
template <int HT>
__device__ __forceinline__ uint16_t recover_weight(int8_t q, float d) {
    float v = (float)q * d;
    asm volatile("" : "+v"(v));
    return f32_to_h16<HT>(v);
}

// Panel-blocked int8 layout of an [R,K] operand of the int8 matmul (the
// converted weight, R = N, and the quantized activations in the workspace,
// R = T): rows are grouped in panels of kPanel rows (the last panel may be
// shorter), a panel's K range is cut into k-tiles of kKTile columns (the
// last may be narrower, always a multiple of 16), and each (panel, k-tile)
// block is stored row-major.  So the kKTile bytes of 16 consecutive rows of
// one k-tile are one contiguous kilobyte: a wave's 16-byte-per-lane copy of
// a tile slice touches 8 whole 128-byte lines instead of halves of 16 (the
// CU's L2 -> LDS copy rate with 64-byte row pieces is about two thirds of
// the rate with whole lines).  The blocks of a panel follow each other in k
// order, the panels in row order; nothing is padded (R*K bytes in all).
constexpr int64_t kPanel = 256;
constexpr int64_t kKTile = 64;

// Rows of the panel that holds row r.
__host__ __device__ inline int64_t blk_rows(int64_t r, int64_t R) {
    const int64_t p0 = r - r % kPanel;
    return R - p0 < kPanel ? R - p0 : kPanel;
}

// Byte offset of element (r, k) of an [R,K] operand in the panel-blocked layout.
__host__ __device__ inline int64_t blk_offset(int64_t r, int64_t k, int64_t R, int64_t K) {
    const int64_t p0 = r - r % kPanel;          // first row of the panel
    const int64_t rows = R - p0 < kPanel ? R - p0 : kPanel;
    const int64_t k0 = k - k % kKTile;          // first column of the k-tile
    const int64_t w = K - k0 < kKTile ? K - k0 : kKTile;
    return p0 * K + k0 * rows + (r - p0) * w + (k - k0);
}

// Bytes of the converted weight: int8 [N,K] in the panel-blocked layout.
inline int64_t wq_bytes(int64_t K, int64_t N) { return K * N; }

// Compute units of the current device (256 if it cannot be queried).
int device_cus();

// Bits of the smallest 16-bit value (binary16, or bfloat16 for ht = bf16)
// >= tau (tau >= 0, not NaN), or the +inf pattern when no finite value
// reaches tau: for a non-negative 16-bit value x (not NaN),
// x >= tau <=> bits(x) >= this.
uint32_t tau_to_h16_ceil(float tau, int ht);

// 2 when the large-tile matmul of (T, K, N) runs each 256 x 256 output tile
// as two halves of K on the current device, else 1.
int gemm_ksplit(int64_t T, int64_t K, int64_t N);
// K split of the streaming kernel (65..128 rows): s slabs (1: none) of
// tiles tiles with tile_bytes of int32 partial sums per slab (k_gemm.hip).
constexpr int64_t kStreamMinSlab = 16;   // k-tiles of 128 per slab, at least
constexpr int kStreamMaxSplit = 8;
struct StreamSplit {
    int s;
    int64_t tiles, tile_bytes;
};
StreamSplit stream_split(int64_t T, int64_t K, int64_t N);
// 129..256 rows that run on the streaming kernel's 256x128 tile (k_gemm.hip)
bool stream_256x128(int64_t T, int64_t K, int64_t N);
// Completes Y from int32 partial sums part [slabs][T][N] (sum of the slabs,
// dequantization, the outlier terms from W16 [K,N] or, W16 = NULL, from the
// Int8 weight; one fp16/bf16 rounding) - the decode kernel's finishing
// kernel, also used by the streaming matmul's 64x64 K split (k_decode.hip).
hipError_t launch_finish_partials(int ht, int64_t T, int64_t K, int64_t N, int slabs,
                                  const int32_t* part, const int8_t* Wq, const float* sw,
                                  const uint16_t* W16, const float* sx, const int32_t* count,
                                  const int32_t* idx, const uint16_t* xo, uint16_t* Y,
                                  int32_t* dbg_acc, hipStream_t stream);
// The large-tile matmul's K split on this device: the first `full` tiles run
// all of K, the last `nsplit` as two halves (nsplit = 0: no split).
struct KSplitPlan {
    int64_t full, nsplit;
};
KSplitPlan gemm_ksplit_plan(int64_t T, int64_t K, int64_t N);

// Partial outlier bitmaps the workspace holds (row groups of the detection).
constexpr int kDetectParts = 4;

// Words between two partial outlier bitmaps of the workspace.
inline int64_t bitmap_stride(int64_t K) { return (ceil_div(K, 32) + 63) & ~int64_t(63); }

// Outlier rows the memory-halved variant recovers into the workspace before
// the matmul (more outliers than this: the matmul recovers them itself).
constexpr int64_t kRecoverRows = 512;

// Activation pass for few rows (T <= kSmallT): one workgroup per segment of
// kSegCols columns holds every row of them, so it knows its outlier columns
// without waiting for the rest of X.
constexpr int kSmallT = 16;
constexpr int kSegCols = 2048;

// Layout of the workspace for (T, K, N) at `base` (base may be NULL to size
// it); wrec adds the recovered-rows region, ksplit = 2 the K-split regions
// (which need wrec), dslabs > 0 the decode kernel's K-slab partial sums.
Workspace carve_workspace(void* base, int64_t T, int64_t K, int64_t N, bool wrec, int ksplit,
                          int dslabs = 0);

// Recovers W^[j, n] = 16-bit(fp32(Wq[n, idx_j] * fp32(s_w[n] / 127))) for the
// outliers j < o <= rows into out [rows, N] (nothing when o > rows).
hipError_t launch_recover_rows(const int8_t* Wq, const float* sw, const int32_t* idx,
                               const int32_t* count, int64_t K, int64_t N, int ht,
                               uint16_t* out, int64_t rows, hipStream_t stream);

// ---- activation side (k_activation.hip)
// zero, nzero: int32 words the pass also sets to zero (the matmul's K-split
// tile counters, so the matmul of the same call needs no launch for them);
// only with more than 128 rows, where the column detection runs
// (hipErrorInvalidValue otherwise).
hipError_t launch_activation_pass(const uint16_t* X, int ht, int64_t T, int64_t K, float tau,
                                  const Workspace& ws, hipStream_t stream,
                                  int32_t* zero = nullptr, int64_t nzero = 0);

// ---- weight side (k_weight.hip)
// weight checkpoint types (the values of INT8MM_WEIGHT_* in include/int8mm.h)
constexpr int kWeightF16 = 0, kWeightBF16 = 1, kWeightF32 = 2;
hipError_t launch_quantize_weight(const void* W, int wtype, int64_t K, int64_t N, int8_t* Wq,
                                  float* sw, _Float16* w16, hipStream_t stream);

// ---- int8 GEMM + dequantization + 16-bit outlier GEMM (k_gemm.hip)
struct GemmArgs {
    const int8_t* xq;      // [T,K]
    const float* sx;       // [T]
    const int8_t* wq;      // [N,K]
    const float* sw;       // [N]
    const uint16_t* xo;    // [T,opad] 16-bit
    const int32_t* idx;    // [K]
    const int32_t* count;  // [2]
    const uint16_t* w16;   // [K,N] 16-bit (row idx_j), or NULL: outlier rows recovered from wq
    int64_t w16_rows;      // > 0: w16 is [w16_rows, N] with row j = outlier j, valid when
                           // o <= w16_rows (else the rows are recovered from wq)
    uint16_t* y;           // [T,N] 16-bit
    int32_t* acc_out;      // [T,N] or NULL
    int64_t T, K, N;
    int ksplit;            // 1; 2: K split in two halves (large-tile kernel); S: slabs (streaming kernel)
    int32_t* ks_count;     // [nsplit] (ksplit = 2; zero at launch_gemm or zeroed by it)
    int32_t* ks_part;      // [nsplit][2][65536] (ksplit = 2)
    int64_t ks_full;       // ksplit = 2: tiles that run all of K (set by launch_gemm)
    int ks_zeroed;         // ksplit = 2: ks_count already zero (else launch_gemm zeroes it)
};
hipError_t launch_gemm(const GemmArgs& a, int ht, hipStream_t stream);

// ---- single-kernel decode path (k_decode.hip)
bool decode_path_supported(int64_t T, int64_t K, int64_t N);
hipError_t launch_decode(const uint16_t* X, int ht, int64_t T, int64_t K, const int8_t* Wq,
                         const float* sw, const uint16_t* W16, int64_t N, float tau,
                         uint16_t* Y, int32_t* dbg_count, int32_t* dbg_idx, int8_t* dbg_xq,
                         float* dbg_sx, int32_t* dbg_acc, hipStream_t stream);

// Decode shapes the single-kernel path does not take (T <= 8, K % 1024 == 0,
// T*K <= 128 KB): the same weight stream with the activation side read from
// a workspace the activation pass has filled (k_decode.hip).
bool decode_pre_supported(int64_t T, int64_t K, int64_t N);
hipError_t launch_decode_pre(int ht, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                             const uint16_t* W16, int64_t N, uint16_t* Y, const Workspace& ws,
                             int32_t* dbg_acc, hipStream_t stream);

// Few rows whose Xq is longer than the decode kernel keeps in LDS (T <= 8,
// or T <= 16 with K >= 32768; K % 1024 == 0, T*K > 128 KB): K is cut into
// slabs, each workgroup streams
// one slab of its rows and writes int32 partial sums to ws.dpart, and a
// second kernel adds them and finishes Y.  decode_split_reserve is the
// number of slabs the workspace must hold (0: not such a shape).
int decode_split_reserve(int64_t T, int64_t K, int64_t N);
hipError_t launch_decode_split(int ht, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                               const uint16_t* W16, int64_t N, uint16_t* Y, const Workspace& ws,
                               int32_t* dbg_acc, hipStream_t stream);

// ---- debug copies (k_activation.hip)
hipError_t launch_debug_copies(const Workspace& ws, int64_t T, int64_t K, int32_t* count,
                               int32_t* idx, int8_t* xq, float* sx, hipStream_t stream);

}  // namespace i8mm
