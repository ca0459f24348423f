// Measured ceilings of one MI355X, for reporting the matmul kernels against
// what the chip delivers as well as against its published peaks.  Not part
// of the LLM.int8() library: bench.py loads this separately built library
// (libceiling.so) only to time these two kernels.
//
//   k_mfma_i8:   back-to-back v_mfma_i32_32x32x32_i8 on independent
//                accumulators, no memory traffic: the int8 MFMA rate the
//                part sustains when nothing else draws power;
//   k_stream:    a coalesced 16-byte-per-lane read of a large buffer with
//                16 loads in flight per lane, the HBM read rate a plain
//                stream reaches.
// Both record each workgroup's shader-clock cycles (s_memtime) and elapsed
// constant-clock ticks (s_memrealtime, 100 MHz) so the clock they ran at
// can be reported.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace {

constexpr int kAcc = 8;   // independent 32x32 accumulators per wave

__global__ __launch_bounds__(256) void k_mfma_i8(int iters, int* sink, unsigned long long* clk) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane + 1, lane + 2, lane + 3};
    v4i b = {lane * 3, lane ^ 5, lane + 7, 11};
    v16i acc[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    if (s == 0x7fffffff) sink[0] = s;   // keeps the work
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

// Grid-stride 16-byte loads, kStreamLoads of them in flight per lane; XOR
// of everything read keeps the loads.
constexpr int kStreamLoads = 16;
__global__ __launch_bounds__(256) void k_stream(const uint4* __restrict__ p, int64_t n16, int* sink,
                                                unsigned long long* clk) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kStreamLoads - 1) * stride < n16; i += kStreamLoads * stride) {
        uint4 v[kStreamLoads];
#pragma unroll
        for (int u = 0; u < kStreamLoads; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kStreamLoads; ++u) {
            x.x ^= v[u].x; x.y ^= v[u].y; x.z ^= v[u].z; x.w ^= v[u].w;
        }
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        x.x ^= a.x; x.y ^= a.y; x.z ^= a.z; x.w ^= a.w;
    }
    if ((x.x ^ x.y ^ x.z ^ x.w) == 0x7fffffffu) sink[0] = 1;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

}  // namespace

// int8 ops of one k_mfma_i8 launch: grid * 4 waves * iters * kAcc * 65536.
extern "C" int ceiling_mfma_i8(int grid, int iters, void* sink, void* clk, void* stream) {
    hipLaunchKernelGGL(k_mfma_i8, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                       (int*)sink, (unsigned long long*)clk);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int ceiling_mfma_acc(void) { return kAcc; }

extern "C" int ceiling_stream(const void* buf, int64_t bytes, int grid, void* sink, void* clk,
                              void* stream) {
    hipLaunchKernelGGL(k_stream, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)buf, bytes / 16, (int*)sink, (unsigned long long*)clk);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
