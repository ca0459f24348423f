// Measured ceilings of one MI355X, for reporting the matmul kernels against
// what the chip delivers as well as against its published peaks.  Not part
// of the LLM.int8() library: bench.py loads this separately built library
// (libceiling.so) only to time these two kernels.
//
//   k_mfma_i8:   back-to-back int8 MFMAs (v_mfma_i32_32x32x32_i8 or
//                v_mfma_i32_16x16x64_i8) on independent accumulators, with
//                pseudo-random operands that change from one instruction to
//                the next and no memory traffic: the int8 MFMA rate the
//                part sustains on matmul-like data when nothing else draws
//                power (the part is power limited, so the rate depends on
//                the instruction and on how many operand bits toggle);
//   k_stream:    coalesced 16-byte-per-lane reads of a large buffer with
//                16 or 32 loads in flight per lane, in a few orders and
//                launch shapes: the HBM read rate a plain stream reaches.
// Both record each workgroup's shader-clock cycles (s_memtime) and elapsed
// constant-clock ticks (s_memrealtime, 100 MHz) so the clock they ran at
// can be reported.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace {

constexpr int kOpsPerIter = 16 * 65536;   // int8 ops per wave per loop iteration

__device__ __forceinline__ int mix(uint32_t x) {   // integer hash (operand bits only)
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return (int)x;
}

// FORM 0: 8 accumulators of 32x32x32, 16 instructions per iteration; FORM 1:
// 32 accumulators of 16x16x64, 32 instructions per iteration (the same ops).
// Four A and four B operand registers per lane, combined differently by
// consecutive instructions.
template <int FORM>
__global__ __launch_bounds__(512) void k_mfma_i8(int iters, int* sink, unsigned long long* clk) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const uint32_t l = threadIdx.x + 977u * blockIdx.x;
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = v4i{mix(l * 16 + i * 4), mix(l * 16 + i * 4 + 1), mix(l * 16 + i * 4 + 2), mix(l * 16 + i * 4 + 3)};
        b[i] = v4i{mix(~l * 16 + i * 4), mix(~l * 16 + i * 4 + 1), mix(~l * 16 + i * 4 + 2),
                   mix(~l * 16 + i * 4 + 3)};
    }
    int s = 0;
    if constexpr (FORM == 0) {
        v16i acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i & 3], b[(i >> 1) & 3], acc[i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(i + 1) & 3], b[((i >> 1) ^ 1) & 3], acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][r];
    } else {
        v4i acc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = v4i{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i & 3], b[i >> 3], acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += acc[i][r];
    }
    if (s == 0x7fffffff) sink[0] = s;   // keeps the work
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

// Streams of 16-byte loads, L of them in flight per lane, B lanes per
// workgroup, in one of two orders: grid-stride (every workgroup walks the
// whole buffer, one 16-byte piece per lane per step) or partitioned (each
// workgroup reads one contiguous range).  The rate depends on the order,
// the launch shape and the run (6.0 to 6.5 TB/s for the good shapes on
// 2 GiB), so the host times a few and reports the best.  XOR of everything
// read keeps the loads.  The host makes the element count a multiple of
// grid * B * L, so no lane reads past the buffer.
template <int L, int B, bool PART>
__global__ __launch_bounds__(B) void k_stream(const uint4* __restrict__ p, int64_t n16, int* sink,
                                              unsigned long long* clk) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    const int64_t per = PART ? n16 / gridDim.x : n16;             // elements this workgroup walks
    const int64_t step = PART ? B : (int64_t)gridDim.x * B;       // between a lane's loads
    const uint4* q = p + (PART ? (int64_t)blockIdx.x * per : (int64_t)blockIdx.x * B) + threadIdx.x;
    const int64_t span = PART ? per : n16 - (int64_t)blockIdx.x * B;
    for (int64_t i = 0; i + (L - 1) * step < span; i += L * step) {
        uint4 v[L];
#pragma unroll
        for (int u = 0; u < L; ++u) v[u] = q[i + u * step];
#pragma unroll
        for (int u = 0; u < L; ++u) {
            x.x ^= v[u].x; x.y ^= v[u].y; x.z ^= v[u].z; x.w ^= v[u].w;
        }
    }
    if ((x.x ^ x.y ^ x.z ^ x.w) == 0x7fffffffu) sink[0] = 1;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
        clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

}  // namespace

// int8 ops of one k_mfma_i8 launch: grid * 8 waves * iters * ceiling_mfma_ops_per_iter().
// form 0: v_mfma_i32_32x32x32_i8, form 1: v_mfma_i32_16x16x64_i8; returns 2
// for an unknown form.
extern "C" int ceiling_mfma_i8(int form, int grid, int iters, void* sink, void* clk, void* stream) {
    if (form == 0)
        hipLaunchKernelGGL(k_mfma_i8<0>, dim3(grid), dim3(512), 0, (hipStream_t)stream, iters,
                           (int*)sink, (unsigned long long*)clk);
    else if (form == 1)
        hipLaunchKernelGGL(k_mfma_i8<1>, dim3(grid), dim3(512), 0, (hipStream_t)stream, iters,
                           (int*)sink, (unsigned long long*)clk);
    else
        return 2;
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int ceiling_mfma_ops_per_iter(void) { return kOpsPerIter; }

// Stream variants: 0 = grid-stride, 16 loads, 256 lanes; 1 = grid-stride,
// 32 loads, 256 lanes; 2 = partitioned, 16 loads, 512 lanes; 3 =
// partitioned, 16 loads, 256 lanes.  Returns 2 for an unknown variant or a
// size that is not a multiple of grid * lanes * loads * 16 bytes.
extern "C" int ceiling_stream(const void* buf, int64_t bytes, int grid, int variant, void* sink,
                              void* clk, void* stream) {
    static const int lanes[4] = {256, 256, 512, 256}, loads[4] = {16, 32, 16, 16};
    if (variant < 0 || variant > 3 || grid <= 0 || bytes <= 0) return 2;
    const int64_t n16 = bytes / 16;
    if (bytes % 16 != 0 || n16 % ((int64_t)grid * lanes[variant] * loads[variant]) != 0) return 2;
    const hipStream_t s = (hipStream_t)stream;
    const uint4* p = (const uint4*)buf;
    int* k = (int*)sink;
    unsigned long long* c = (unsigned long long*)clk;
    switch (variant) {
        case 0: hipLaunchKernelGGL((k_stream<16, 256, false>), dim3(grid), dim3(256), 0, s, p, n16, k, c); break;
        case 1: hipLaunchKernelGGL((k_stream<32, 256, false>), dim3(grid), dim3(256), 0, s, p, n16, k, c); break;
        case 2: hipLaunchKernelGGL((k_stream<16, 512, true>), dim3(grid), dim3(512), 0, s, p, n16, k, c); break;
        default: hipLaunchKernelGGL((k_stream<16, 256, true>), dim3(grid), dim3(256), 0, s, p, n16, k, c); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
