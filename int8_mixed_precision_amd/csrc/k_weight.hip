// Weight side of LLM.int8(): a 16-bit weight is converted to Int8 once, at
// load time (LLM.int8() abstract, taxoreview.com page dblp:280/8696, second
// paragraph), with one absmax scale per output column n - the column is one
// operand of the inner products that produce column n of Y.
//
//   s_w[n] = max_k |W[k,n]|,  Wq[n,k] = clamp(rint(W[k,n] * fp32(127/s_w[n])), -127, 127)
//
// Wq is written transposed, [N,K] with K contiguous, so that the int8 GEMM
// reads both of its operands along K with 16-byte loads.
//
// Two HBM-bound passes: a column-absmax reduction (16-byte loads along rows,
// one atomicMax per column per workgroup) and a tiled quantize + transpose
// through LDS (coalesced fp16 reads along N, coalesced int8 writes along K).
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

__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Column absmax over the workgroup's rows; merged into sw with an unsigned
// atomicMax on the float bits (valid because every value is >= +0).
__global__ __launch_bounds__(kColThreads) void k_colmax(const uint16_t* __restrict__ W, int64_t K,
                                                        int64_t N, float* __restrict__ sw) {
    const int64_t c0 = ((int64_t)blockIdx.x * kColThreads + threadIdx.x) * 8;
    if (c0 >= N) return;
    const int64_t k0 = (int64_t)blockIdx.y * kColRows;
    const int64_t k1 = k0 + kColRows < K ? k0 + kColRows : K;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* p = W + k0 * N + c0;
    int64_t k = k0;
    for (; k + 4 <= k1; k += 4, p += 4 * N) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(p + u * N);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(h2f((uint16_t)(w[e >> 1] >> ((e & 1) * 16)))));
        }
    }
    for (; k < k1; ++k, p += N) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(h2f((uint16_t)(w[e >> 1] >> ((e & 1) * 16)))));
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
// along k.
__global__ __launch_bounds__(kTrThreads) void k_quant_transpose(const uint16_t* __restrict__ W,
                                                                int64_t K, int64_t N,
                                                                const float* __restrict__ sw,
                                                                int8_t* __restrict__ Wq) {
    // +16 bytes per row spreads the transposed byte stores over banks
    __shared__ __attribute__((aligned(16))) int8_t tile[kTrN][kTrK + 16];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kTrN;
    const int64_t k0 = (int64_t)blockIdx.y * kTrK;
    // read phase: 8 lanes cover one 64-column row segment (8 halves each)
    const int cn = (tid & 7) * 8;           // column inside the tile
    const int64_t n = n0 + cn;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float s = (n + e < N) ? sw[n + e] : 0.0f;
        r[e] = s > 0.0f ? 127.0f / s : 0.0f;
    }
    for (int kr = tid >> 3; kr < kTrK; kr += kTrThreads / 8) {
        const int64_t k = k0 + kr;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (k < K && n < N) {
            uint4 v = *reinterpret_cast<const uint4*>(W + k * N + n);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            tile[cn + e][kr] = quant(h2f((uint16_t)(w[e >> 1] >> ((e & 1) * 16))), r[e]);
    }
    __syncthreads();
    // write phase: 8 lanes cover one 128-byte row of Wq
    const int ck = (tid & 7) * 16;
    for (int nr = tid >> 3; nr < kTrN; nr += kTrThreads / 8) {
        const int64_t nn = n0 + nr;
        const int64_t k = k0 + ck;
        if (nn < N && k < K)
            *reinterpret_cast<uint4*>(Wq + nn * K + k) = *reinterpret_cast<const uint4*>(&tile[nr][ck]);
    }
}

}  // namespace

hipError_t launch_quantize_weight(const _Float16* W, int64_t K, int64_t N, int8_t* Wq, float* sw,
                                  hipStream_t stream) {
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(W);
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, stream, sw, N);
    hipLaunchKernelGGL(k_colmax, dim3((unsigned)ceil_div(N, kColCols), (unsigned)ceil_div(K, kColRows)),
                       dim3(kColThreads), 0, stream, wb, K, N, sw);
    hipLaunchKernelGGL(k_quant_transpose, dim3((unsigned)ceil_div(N, kTrN), (unsigned)ceil_div(K, kTrK)),
                       dim3(kTrThreads), 0, stream, wb, K, N, sw, Wq);
    return hipGetLastError();
}

}  // namespace i8mm
