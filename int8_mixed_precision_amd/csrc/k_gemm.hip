// Int8 matrix multiplication of LLM.int8() with its fused epilogue.
//
// Method (LLM.int8() abstract, taxoreview.com page dblp:280/8696, second
// paragraph): the non-outlier part is an Int8 matrix multiplication with one
// normalization constant per inner product, and the isolated outlier
// dimensions go through a 16-bit matrix multiplication whose result is added.
// Per output element (t, n):
//   acc = sum_k Xq[t,k] * Wq[n,k]                   int8 x int8 -> int32 (MFMA)
//   y   = acc * s_x[t] * s_w[n] / 127^2              dequantization, fp32
//   y  += sum_{j<o} X[t,idx_j] * W16[idx_j,n]        fp16 MFMA, fp32 accumulation
//   Y   = fp16(y)                                    one rounding
//
// gfx950 design: both operands are K-contiguous (Xq [T,K], Wq [N,K]), so a
// lane's 16 int8 of an MFMA operand are one 16-byte load.  Tiles are staged
// through LDS, double-buffered, with an XOR swizzle of the 16-byte chunks so
// the ds_read_b128 of the operand fragments avoid bank conflicts.  The
// 16-bit outlier product reuses the dequantized fp32 accumulators as the C
// operand of v_mfma_f32_32x32x16_f16, so it needs no extra registers and the
// sum is rounded to fp16 once.  Workgroups are renumbered so that the tiles
// sharing a weight panel run on the same XCD (one L2).
#include "common.hpp"

namespace i8mm {

namespace {

constexpr int kThreads = 256;   // 4 waves

template <int BM, int BN, int BK, int WAVES_M>
struct Cfg {
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int WM = BM / WAVES_M;   // wave tile rows
    static constexpr int WN = BN / WAVES_N;   // wave tile cols
    static constexpr int TM = WM / 32;        // 32x32 MFMA tiles per wave, rows
    static constexpr int TN = WN / 32;        //                            cols
    static constexpr int CPR = BK / 16;       // 16-byte chunks per LDS row
    static constexpr int LA = BM * CPR / kThreads;   // A chunks per thread per stage
    static constexpr int LB = BN * CPR / kThreads;   // B chunks per thread per stage
    static constexpr int ROWS_PER_WINDOW = 128 / BK > 0 ? 128 / BK : 1;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BK % 32 == 0, "BK must be a multiple of 32");
    static_assert(LA >= 1 && LB >= 1 && (BM * CPR) % kThreads == 0 && (BN * CPR) % kThreads == 0,
                  "tile must split evenly over the workgroup");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row`.
template <int CPR, int RPW>
__device__ inline int swz(int row, int c) {
    return c ^ ((row / RPW) & (CPR - 1));
}

template <int BM, int BN, int BK, int WAVES_M, bool WRITE_ACC>
__global__ __launch_bounds__(kThreads) void k_gemm_i8(GemmArgs a) {
    using C = Cfg<BM, BN, BK, WAVES_M>;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t T = a.T, K = a.K, N = a.N;
    const int64_t MT = ceil_div(T, BM);

    // XCD-aware renumbering: hardware deals workgroups round-robin over the
    // 8 XCDs; give each XCD a contiguous range of logical tiles (M fastest),
    // so the M-tiles that share one weight panel hit the same L2.
    int64_t bid = blockIdx.x;
    const int64_t nb = gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int64_t m0 = (bid % MT) * BM;
    const int64_t n0 = (bid / MT) * BN;

    const int wm0 = (wave % WAVES_M) * C::WM;
    const int wn0 = (wave / WAVES_M) * C::WN;

    v16i acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    v4i ra[C::LA], rb[C::LB];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < C::LA; ++i) {
            const int id = i * kThreads + tid;
            const int row = id / C::CPR, c = id % C::CPR;
            const int64_t gm = m0 + row, gk = k0 + c * 16;
            ra[i] = (gm < T && gk < K) ? *reinterpret_cast<const v4i*>(a.xq + gm * K + gk)
                                       : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::LB; ++i) {
            const int id = i * kThreads + tid;
            const int row = id / C::CPR, c = id % C::CPR;
            const int64_t gn = n0 + row, gk = k0 + c * 16;
            rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const v4i*>(a.wq + gn * K + gk)
                                       : v4i{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::LA; ++i) {
            const int id = i * kThreads + tid;
            const int row = id / C::CPR, c = id % C::CPR;
            *reinterpret_cast<v4i*>(&As[buf][row * BK + swz<C::CPR, C::ROWS_PER_WINDOW>(row, c) * 16]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < C::LB; ++i) {
            const int id = i * kThreads + tid;
            const int row = id / C::CPR, c = id % C::CPR;
            *reinterpret_cast<v4i*>(&Bs[buf][row * BK + swz<C::CPR, C::ROWS_PER_WINDOW>(row, c) * 16]) = rb[i];
        }
    };

    const int64_t KT = ceil_div(K, BK);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            v4i af[C::TM], bf[C::TN];
            const int c = s * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const int row = wm0 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const v4i*>(&As[cur][row * BK + swz<C::CPR, C::ROWS_PER_WINDOW>(row, c) * 16]);
            }
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int row = wn0 + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const v4i*>(&Bs[cur][row * BK + swz<C::CPR, C::ROWS_PER_WINDOW>(row, c) * 16]);
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---------------- epilogue
    // 32x32 accumulator layout: lane holds column (lane & 31) and, in register
    // r, row 8*(r/4) + 4*(lane/32) + (r%4) of the tile.
    const int col_l = lane & 31;
    const int row_l = (lane >> 5) * 4;
    if (WRITE_ACC && a.acc_out) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int64_t n = n0 + wn0 + j * 32 + col_l;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm0 + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                    if (m < T && n < N) a.acc_out[m * N + n] = acc[i][j][r];
                }
            }
    }
    float swn[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        const int64_t n = n0 + wn0 + j * 32 + col_l;
        swn[j] = n < N ? a.sw[n] * (1.0f / 16129.0f) : 0.0f;
    }
    v16f y[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        float sxm[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm0 + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
            sxm[r] = m < T ? a.sx[m] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) y[i][j][r] = (float)acc[i][j][r] * sxm[r] * swn[j];
    }

    // 16-bit matmul over the isolated outlier dimensions, 16 at a time.
    const int o = a.count[0];
    const int opad = a.count[1];
    for (int jc = 0; jc < opad; jc += 16) {
        const int jl = jc + (lane >> 5) * 8;   // first of this lane's 8 outlier slots
        v8h xa[C::TM], wb[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int64_t m = m0 + wm0 + i * 32 + (lane & 31);
            xa[i] = m < T ? *reinterpret_cast<const v8h*>(a.xo + m * opad + jl)
                          : v8h{0, 0, 0, 0, 0, 0, 0, 0};
        }
        int64_t rowoff[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rowoff[e] = (jl + e < o) ? (int64_t)a.idx[jl + e] * N : -1;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int64_t n = n0 + wn0 + j * 32 + col_l;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wb[j][e] = (rowoff[e] >= 0 && n < N) ? a.w16[rowoff[e] + n] : (_Float16)0.0f;
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[i], wb[j], y[i][j], 0, 0, 0);
    }

#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int64_t n = n0 + wn0 + j * 32 + col_l;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm0 + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                if (m < T && n < N) a.y[m * N + n] = (_Float16)y[i][j][r];
            }
        }
}

template <int BM, int BN, int BK, int WAVES_M>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    const int64_t tiles = ceil_div(a.T, BM) * ceil_div(a.N, BN);
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, WAVES_M, true>), dim3((unsigned)tiles), dim3(kThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, WAVES_M, false>), dim3((unsigned)tiles), dim3(kThreads),
                           0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
    if (a.T <= 32) return launch_cfg<32, 256, 128, 1>(a, stream);
    return launch_cfg<128, 128, 64, 2>(a, stream);
}

}  // namespace i8mm
