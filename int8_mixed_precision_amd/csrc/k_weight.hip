// Weight side of LLM.int8(): a 16- or 32-bit checkpoint weight (fp16, bf16
// or fp32) is converted to Int8 once, at load time (LLM.int8() abstract,
// taxoreview.com page dblp:280/8696, second paragraph), with one absmax
// scale per output column n - the column is one operand of the inner
// products that produce column n of Y.  The scale and the codes are taken
// on the checkpoint's own values.
//
//   s_w[n] = max_k |W[k,n]|,  Wq[n,k] = clamp(rint(W[k,n] * fp32(127/s_w[n])), -127, 127)
// (fp32(127/s) with an unbounded exponent: see qfactor in common.hpp)
//
// Wq is written transposed, [N,K] with K contiguous inside the panel-blocked
// layout (panels of 256 rows, k-tiles of 64 columns), so that the int8 GEMM
// reads both of its operands along K with 16-byte loads, a kilobyte of 16
// rows at a time.
//
// Two HBM-bound passes: a column-absmax reduction (16-byte loads along rows,
// one atomicMax per column per workgroup) and a tiled quantize + transpose
// through LDS (coalesced reads along N, coalesced int8 writes along K).
#include "common.hpp"

// Quantization must round x * r and any following add separately, exactly
// like the definition; no multiply-add contraction in this file.
#pragma clang fp contract(off)

namespace i8mm {

namespace {

constexpr int kColThreads = 256;
constexpr int kColCols = kColThreads * 8;   // columns per workgroup
constexpr int kColRows = 256;               // rows per workgroup

constexpr int kTrThreads = 256;
constexpr int kTrK = 128;                   // k extent of a tile
constexpr int kTrN = 64;                    // n extent of a tile

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline float bf2f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// Eight consecutive weight values starting at element `off` (a multiple of
// 8) of a [K,N] checkpoint of type WT, widened to fp32 (exact for fp16 and
// bf16): one 16-byte load for the 16-bit types, two for fp32.
template <int WT>
__device__ inline void load8(const void* W, int64_t off, float (&v)[8]) {
    if (WT == kWeightF32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + off);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t b = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
            v[e] = WT == kWeightBF16 ? bf2f(b) : h2f(b);
        }
    }
}

__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Column absmax over the workgroup's rows; merged into sw with an unsigned
// atomicMax on the float bits (valid because every value is >= +0).
template <int WT>
__global__ __launch_bounds__(kColThreads) void k_colmax(const void* __restrict__ W, int64_t K,
                                                        int64_t N, float* __restrict__ sw) {
    const int64_t c0 = ((int64_t)blockIdx.x * kColThreads + threadIdx.x) * 8;
    if (c0 >= N) return;
    const int64_t k0 = (int64_t)blockIdx.y * kColRows;
    const int64_t k1 = k0 + kColRows < K ? k0 + kColRows : K;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // 8 rows' loads in flight per lane (measured 4% faster than 4 on a
    // 12288 x 49152 fp16 weight; 16 was slower again)
    int64_t k = k0;
    for (; k + 8 <= k1; k += 8) {
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) load8<WT>(W, (k + u) * N + c0, v[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(v[u][e]));
    }
    for (; k < k1; ++k) {
        float v[8];
        load8<WT>(W, k * N + c0, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(v[e]));
    }
    unsigned int* swu = reinterpret_cast<unsigned int*>(sw);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (m[e] > 0.0f) atomicMax(&swu[c0 + e], __builtin_bit_cast(unsigned int, m[e]));
}

__device__ inline int8_t quant(float x, float r) {
    float q = __builtin_rintf(x * r);
    q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
    return (int8_t)(int)q;
}

// One tile of kTrK rows (k) by kTrN columns (n): read W[k0.., n0..] along n,
// quantize with the column's scale, transpose through LDS, write Wq[n0.., k0..]
// along k (each 16-byte piece at its place in the blocked layout).  With
// w16 given, the fp16 copy of the values (round to nearest even) is written
// to w16[k, n] on the way (the 16-bit weight of the outlier path, for
// checkpoints that are not fp16).
template <int WT>
__global__ __launch_bounds__(kTrThreads) void k_quant_transpose(const void* __restrict__ W,
                                                                int64_t K, int64_t N,
                                                                const float* __restrict__ sw,
                                                                int8_t* __restrict__ Wq,
                                                                _Float16* __restrict__ w16) {
    // +16 bytes per row spreads the transposed byte stores over banks
    __shared__ __attribute__((aligned(16))) int8_t tile[kTrN][kTrK + 16];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kTrN;
    const int64_t k0 = (int64_t)blockIdx.y * kTrK;
    // read phase: 8 lanes cover one 64-column row segment (8 values each)
    const int cn = (tid & 7) * 8;           // column inside the tile
    const int64_t n = n0 + cn;
    // (fp16 scales are at least 2^-24: the tiny-scale factor is 1 for them)
    float r[8], qk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float s = (n + e < N) ? sw[n + e] : 0.0f;
        qk[e] = WT == kWeightF16 ? 1.0f : qfactor(s);
        r[e] = s > 0.0f ? 127.0f / (s * qk[e]) : 0.0f;
    }
    for (int kr = tid >> 3; kr < kTrK; kr += kTrThreads / 8) {
        const int64_t k = k0 + kr;
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (k < K && n < N) {
            load8<WT>(W, k * N + n, v);
            if (w16) {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * e]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * e + 1]) << 16);
                *reinterpret_cast<uint4*>(w16 + k * N + n) = make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[cn + e][kr] = quant(v[e] * qk[e], r[e]);
    }
    __syncthreads();
    // write phase: 8 lanes cover one 128-byte row of Wq
    const int ck = (tid & 7) * 16;
    for (int nr = tid >> 3; nr < kTrN; nr += kTrThreads / 8) {
        const int64_t nn = n0 + nr;
        const int64_t k = k0 + ck;
        if (nn < N && k < K)
            *reinterpret_cast<uint4*>(Wq + blk_offset(nn, k, N, K)) =
                *reinterpret_cast<const uint4*>(&tile[nr][ck]);
    }
}

template <int WT>
hipError_t launch_typed(const void* W, int64_t K, int64_t N, int8_t* Wq, float* sw,
                        _Float16* w16, hipStream_t stream) {
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, stream, sw, N);
    hipLaunchKernelGGL(k_colmax<WT>, dim3((unsigned)ceil_div(N, kColCols), (unsigned)ceil_div(K, kColRows)),
                       dim3(kColThreads), 0, stream, W, K, N, sw);
    hipLaunchKernelGGL(k_quant_transpose<WT>, dim3((unsigned)ceil_div(N, kTrN), (unsigned)ceil_div(K, kTrK)),
                       dim3(kTrThreads), 0, stream, W, K, N, sw, Wq, w16);
    return hipGetLastError();
}

// Memory-halved variant: the outlier rows of W recovered from the Int8
// weight once per call, out[j, n] = 16-bit(fp32(Wq[n, idx_j] * fp32(s_w[n] /
// 127))) (HT: fp16 or bf16), so that the matmul reads them as contiguous rows
// like a caller's W16.  Thread -> column n (stores coalesced along n); the
// y dimension of the grid strides over the outliers.  Each thread reads one
// byte per outlier from its row of Wq.  Nothing is written when o > rows: the
// matmul then recovers the values itself.
template <int HT>
__global__ __launch_bounds__(256) void k_recover_rows(const int8_t* __restrict__ Wq,
                                                      const float* __restrict__ sw,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ count,
                                                      int64_t K, int64_t N,
                                                      uint16_t* __restrict__ out, int64_t rows) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t o = count[0];
    if (n >= N || o > rows) return;
    const float d = sw[n] / 127.0f;
    for (int64_t j = blockIdx.y; j < o; j += gridDim.y)
        out[j * N + n] = recover_weight<HT>(Wq[blk_offset(n, idx[j], N, K)], d);
}

}  // namespace

hipError_t launch_recover_rows(const int8_t* Wq, const float* sw, const int32_t* idx,
                               const int32_t* count, int64_t K, int64_t N, int ht,
                               uint16_t* out, int64_t rows, hipStream_t stream) {
    // enough workgroups to fill the chip for any N; each strides over o
    const dim3 grid((unsigned)ceil_div(N, 256), 16);
    if (ht == kHalfBF16)
        hipLaunchKernelGGL(k_recover_rows<kHalfBF16>, grid, dim3(256), 0, stream, Wq, sw, idx,
                           count, K, N, out, rows);
    else
        hipLaunchKernelGGL(k_recover_rows<kHalfF16>, grid, dim3(256), 0, stream, Wq, sw, idx,
                           count, K, N, out, rows);
    return hipGetLastError();
}

hipError_t launch_quantize_weight(const void* W, int wtype, int64_t K, int64_t N, int8_t* Wq,
                                  float* sw, _Float16* w16, hipStream_t stream) {
    switch (wtype) {
        case kWeightF16: return launch_typed<kWeightF16>(W, K, N, Wq, sw, w16, stream);
        case kWeightBF16: return launch_typed<kWeightBF16>(W, K, N, Wq, sw, w16, stream);
        case kWeightF32: return launch_typed<kWeightF32>(W, K, N, Wq, sw, w16, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace i8mm
