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
// gfx950 design: both operands are K-contiguous (Xq [T,K], Wq [N,K], each
// in the panel-blocked layout of common.hpp: 256-row panels cut into
// 64-column k-tiles, every (panel, k-tile) block row-major), so a lane's 16
// int8 of an MFMA operand are one 16-byte load and a wave's copy of 16 rows
// of a k-tile is one contiguous kilobyte.  Tiles are staged
// through LDS, double-buffered, with an XOR swizzle of the 16-byte chunks so
// the ds_read_b128 of the operand fragments avoid bank conflicts.  The
// 16-bit outlier product reuses the dequantized fp32 accumulators as the C
// operand of the fp16 (bf16) MFMA of the same tile shape as the int8 one
// (v_mfma_f32_16x16x32_f16 in the large-tile kernel, 32x32x16 in the
// others), so it needs no extra registers and the sum is rounded to fp16
// once.  Workgroups are renumbered so that the tiles
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

// What the large-tile kernel hands its epilogue for staging the outlier
// operands through LDS (the streaming kernel passes lds, tid and n0 only).
struct StageCtx {
    int8_t* lds;         // at least kStageBytes and kYBytes, free once the main loop is done
    int tid;             // 0 .. 511
    int64_t m0, n0;      // the workgroup's 256 x 256 output tile
    float* sxs;          // 256 floats of LDS outside the above for the tile's row scales
    float sx_pre;        // s_x of tile row tid (tid < 256; the last row past T)
    const float* sw_pre; // s_w of the lane's TN columns (0 past N)
    int o, opad;         // outlier count and its padded value
    int k_first;         // outlier slot tid % 32's dimension (or -1), read before the main loop
    // the first chunk's 16-bit W values and X columns of this thread, loaded
    // by the kernel before the dequantization (valid when pre_loaded)
    bool pre_loaded;
    uint4 pre_w[2], pre_x[2];
};
constexpr int kOC = 32;                       // outliers per staged chunk
constexpr int kOS = kOC * 2 + 16;             // bytes per staged row / column (padded)
constexpr int kStageHalf = 256 * kOS;         // X part (rows) or W part (columns)
constexpr int kStageBytes = 4 * kStageHalf;   // two buffers of X and W
// The staged Y tile of the large-tile kernel: 64 groups of 4 rows; in a
// group, column c's 4 values are 8 contiguous bytes at 8 c (so a lane
// stores the 4 rows of one column that it holds as one 8-byte write),
// groups kYG bytes apart (padded so that groups g and g+1 lie half a bank
// period apart).
constexpr int kYG = 256 * 8 + 128;
constexpr int kYBytes = 64 * kYG;             // the 256 x 256 tile of 16-bit Y values

// Epilogue of the register-staged and streaming kernels, for one wave's
// TM x TN grid of 32x32 accumulator tiles whose top-left output element is
// (mb, nb).  32x32 accumulator layout: lane holds column (lane & 31) and, in
// register r, row 8*(r/4) + 4*(lane/32) + (r%4) of the tile.
// SBN > 0 (streaming kernel, STH threads, n-tile of SBN columns): with more
// than 16 outliers the outlier W rows go through LDS like the large-tile
// kernel's (sc.lds, sc.tid and sc.n0 used).
template <int TM, int TN, bool WRITE_ACC, int HT, int SBN = 0, int STH = 256>
__device__ __forceinline__ void epilogue(v16i (&acc)[TM][TN], const GemmArgs& a, int64_t mb,
                                         int64_t nb, int lane, const StageCtx& sc = StageCtx{}) {
    const int64_t T = a.T, N = a.N;
    const int col_l = lane & 31;
    const int row_l = (lane >> 5) * 4;
    if (WRITE_ACC && a.acc_out) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = nb + j * 32 + col_l;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = mb + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                    if (m < T && n < N) a.acc_out[m * N + n] = acc[i][j][r];
                }
            }
    }
    // dequantization by the outer product of the scales (1/127^2 folded
    // into the column scale)
    float swn[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = nb + j * 32 + col_l;
        swn[j] = n < N ? a.sw[n] * (1.0f / 16129.0f) : 0.0f;
    }
    const int o = a.count[0];
    const int opad = a.count[1];
    // 16-bit outlier rows: the caller's W16 (row idx_j), the rows recovered
    // before the matmul (row j, when o fits), or - memory-halved variant
    // without room for those - recovered here from the Int8 weight,
    // W^[k,n] = fp16(q[n,k] * fp32(s_w[n] / 127))
    const bool recover = a.w16 == nullptr || (a.w16_rows > 0 && o > a.w16_rows);
    const bool by_pos = !recover && a.w16_rows > 0;   // W16 row = outlier position
    float dn[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = nb + j * 32 + col_l;
        dn[j] = recover && n < N ? a.sw[n] / 127.0f : 0.0f;
    }
    // dequantize every tile (the integer accumulators die here, so the fp32
    // values take their registers; keeping the fp32 values in the integer
    // array through bit casts instead was compiled wrongly - the four rows of
    // a lane's row group were stored from one register)
    v16f y[TM][TN];
    // rows as 32-bit values (T < 2^24); rows past T read the last row's
    // scale (those outputs are never stored), so the loads are unconditional
    const int Ti = (int)T;
    int mrow0 = (int)mb + row_l;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // registers r = 4g .. 4g+3 hold four consecutive rows starting at a
        // multiple of 4 (sx is 256-byte aligned): one 16-byte load when all
        // four are below T
        float sxm[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int m = mrow0 + i * 32 + g * 8;
            if (m + 3 < Ti) {
                const float4 v = *reinterpret_cast<const float4*>(a.sx + m);
                sxm[4 * g] = v.x; sxm[4 * g + 1] = v.y; sxm[4 * g + 2] = v.z; sxm[4 * g + 3] = v.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) sxm[4 * g + q] = a.sx[m + q < Ti ? m + q : Ti - 1];
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) y[i][j][r] = (float)acc[i][j][r] * sxm[r] * swn[j];
    }
    int jstart = 0;   // outliers done through LDS
    if constexpr (SBN > 0) {
        if (opad > 16) {
            // the W rows of 32 outliers at a time: thread (slot e, column
            // block cb) loads its outlier's row segment (16-byte loads
            // along n) and writes it transposed into LDS, so that a lane's
            // 8 outliers of one column are one 16-byte read; double
            // buffered, the next chunk's loads in flight during this
            // chunk's MFMAs.  X values come straight from the gathered
            // columns (16 contiguous bytes per lane).
            constexpr int CPB = SBN / (STH / 32);     // columns per block (STH / 32 blocks)
            constexpr int NV = CPB / 8;               // 16-byte loads per thread
            constexpr int kWS = SBN * kOS;            // bytes of one buffer
            static_assert(NV >= 1 && NV * 8 * (STH / 32) == SBN, "whole 8-column pieces per thread");
            __syncthreads();   // the main loop's LDS reads are complete
            const int e = sc.tid & 31, cb = sc.tid >> 5;
            float dcol[CPB];
            if (recover) {
#pragma unroll
                for (int c = 0; c < CPB; ++c) {
                    const int64_t n = sc.n0 + cb * CPB + c;
                    dcol[c] = n < N ? a.sw[n] / 127.0f : 0.0f;
                }
            }
            // Wq byte (n, k) of this tile's panel (K % 64 == 0 here):
            // wbase + the k part + 64 (n - wp0)
            const int64_t wp0 = sc.n0 - sc.n0 % kPanel;
            const int64_t wrows = N - wp0 < kPanel ? N - wp0 : kPanel;
            int k_next = e < o ? (by_pos ? e : a.idx[e]) : -1;
            uint4 wv[NV];
            auto load_chunk = [&](int jc) {
                const int k = k_next;
                k_next = jc + kOC + e < o ? (by_pos ? jc + kOC + e : a.idx[jc + kOC + e]) : -1;
                const int kc = k < 0 ? 0 : k;   // (k < 0: nothing is read)
                const int8_t* wk = a.wq + wp0 * a.K + (int64_t)(kc & ~(int)(kKTile - 1)) * wrows +
                                   (kc & (int)(kKTile - 1)) - wp0 * kKTile;
#pragma unroll
                for (int h = 0; h < NV; ++h) {
                    const int64_t n = sc.n0 + cb * CPB + h * 8;
                    if (!recover) {
                        wv[h] = (k >= 0 && n < N)
                                    ? *reinterpret_cast<const uint4*>(a.w16 + (int64_t)k * N + n)
                                    : make_uint4(0u, 0u, 0u, 0u);
                    } else {
                        uint32_t p[4];
#pragma unroll
                        for (int c = 0; c < 8; c += 2) {
                            const int64_t nc = n + c;
                            const uint16_t lo = (k >= 0 && nc < N)
                                                    ? recover_weight<HT>(wk[nc * kKTile], dcol[h * 8 + c])
                                                    : (uint16_t)0;
                            const uint16_t hi = (k >= 0 && nc + 1 < N)
                                                    ? recover_weight<HT>(wk[(nc + 1) * kKTile],
                                                                         dcol[h * 8 + c + 1])
                                                    : (uint16_t)0;
                            p[c >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
                        }
                        wv[h] = make_uint4(p[0], p[1], p[2], p[3]);
                    }
                }
            };
            auto store_chunk = [&](int buf) {
                int8_t* ws = sc.lds + buf * kWS;
#pragma unroll
                for (int h = 0; h < NV; ++h) {
                    const uint32_t w4[4] = {wv[h].x, wv[h].y, wv[h].z, wv[h].w};
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        *reinterpret_cast<uint16_t*>(ws + (cb * CPB + h * 8 + c) * kOS + e * 2) =
                            (uint16_t)(w4[c >> 1] >> ((c & 1) * 16));
                }
            };
            load_chunk(0);
            for (int jc = 0; jc < opad; jc += kOC) {
                const int buf = (jc / kOC) & 1;
                store_chunk(buf);
                __syncthreads();
                if (jc + kOC < opad) load_chunk(jc + kOC);
                const int8_t* ws = sc.lds + buf * kWS;
                const int wn0 = (int)(nb - sc.n0);
#pragma unroll
                for (int ks = 0; ks < kOC / 16; ++ks) {
                    if (jc + ks * 16 >= opad) break;
                    const int ko = ks * 32 + (lane >> 5) * 16;
                    const int jl = jc + ks * 16 + (lane >> 5) * 8;
                    v8u16 wb[TN];
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        wb[j] = *reinterpret_cast<const v8u16*>(ws + (wn0 + j * 32 + col_l) * kOS + ko);
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const int64_t mrow = mb + i * 32 + (lane & 31);
                        const v8u16 xa = mrow < T ? *reinterpret_cast<const v8u16*>(a.xo + mrow * opad + jl)
                                                  : v8u16{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            if constexpr (HT == kHalfBF16)
                                y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    __builtin_bit_cast(v8bf, xa), __builtin_bit_cast(v8bf, wb[j]),
                                    y[i][j], 0, 0, 0);
                            else
                                y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    __builtin_bit_cast(v8h, xa), __builtin_bit_cast(v8h, wb[j]),
                                    y[i][j], 0, 0, 0);
                        }
                    }
                }
            }
            jstart = opad;
        }
    }
    // 16-bit matmul over the isolated outlier dimensions, 16 at a time, with
    // the dequantized values as the fp32 C operand.  A group's weight
    // fragments (8 gathered values of one column per lane) are loaded once
    // and serve all TM row strips.
    for (int jc = jstart; jc < opad; jc += 16) {
        const int jl = jc + (lane >> 5) * 8;   // first of this lane's 8 outlier slots
        int kk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kk[e] = (jl + e < o) ? (by_pos ? jl + e : a.idx[jl + e]) : -1;
        v8u16 wb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = nb + j * 32 + col_l;
            if (!recover) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wb[j][e] = (kk[e] >= 0 && n < N) ? a.w16[(int64_t)kk[e] * N + n] : (uint16_t)0;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wb[j][e] = (kk[e] >= 0 && n < N)
                                   ? recover_weight<HT>(a.wq[blk_offset(n, kk[e], N, a.K)], dn[j])
                                   : (uint16_t)0;
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t mrow = mb + i * 32 + (lane & 31);
            const v8u16 xa = mrow < T ? *reinterpret_cast<const v8u16*>(a.xo + mrow * opad + jl)
                                      : v8u16{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (HT == kHalfBF16)
                    y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(v8bf, xa), __builtin_bit_cast(v8bf, wb[j]), y[i][j],
                        0, 0, 0);
                else
                    y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(v8h, xa), __builtin_bit_cast(v8h, wb[j]), y[i][j],
                        0, 0, 0);
            }
        }
    }
    // the row indices are recomputed here rather than kept live through the
    // outlier loop (an empty asm hides the earlier values from the compiler)
    asm volatile("" : "+v"(mrow0));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = nb + j * 32 + col_l;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = mrow0 + i * 32 + (r >> 2) * 8 + (r & 3);
                if (m < Ti && n < N)
                    a.y[(int64_t)m * N + n] = f32_to_h16<HT>(y[i][j][r]);
            }
        }
}

// XCD-aware renumbering: hardware deals workgroups round-robin over the 8
// XCDs; give each XCD a contiguous range of logical tiles, M fastest, so the
// M-tiles that share one weight panel run under the same L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t nb) {
    return (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
}

template <int BM, int BN, int BK, int WAVES_M, bool WRITE_ACC, int HT>
__global__ __launch_bounds__(kThreads) void k_gemm_i8(GemmArgs a) {
    using C = Cfg<BM, BN, BK, WAVES_M>;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t T = a.T, K = a.K, N = a.N;
    const int64_t MT = ceil_div(T, BM);

    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x);
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
            ra[i] = (gm < T && gk < K) ? *reinterpret_cast<const v4i*>(a.xq + blk_offset(gm, gk, T, K))
                                       : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < C::LB; ++i) {
            const int id = i * kThreads + tid;
            const int row = id / C::CPR, c = id % C::CPR;
            const int64_t gn = n0 + row, gk = k0 + c * 16;
            rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const v4i*>(a.wq + blk_offset(gn, gk, N, K))
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

    epilogue<C::TM, C::TN, WRITE_ACC, HT>(acc, a, m0 + wm0, n0 + wn0, lane);
}

// 16-byte copy global -> LDS without VGPR staging (global_load_lds_dwordx4,
// address = wave-uniform base + 32-bit lane offset).  The wave's 64 lanes
// land contiguously at lds_dst + 16 * lane; lds_dst must be wave-uniform.  Written as inline asm so that the compiler's wait-count
// insertion, which cannot tell which LDS bytes such a copy writes, does not
// add a full vmcnt(0) before every LDS read; the kernels below wait for the
// copies themselves (s_waitcnt vmcnt + barrier) before reading the stage.
// The instruction has no register result.  m0 carries the LDS address; no
// other instruction in these kernels uses m0.
__device__ __forceinline__ void copy_to_lds16(const void* gbase, uint32_t goff, const void* lds_dst) {
    const uint32_t la =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_dst;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(goff), "s"(gbase), "s"(la)
                 : "memory");
}

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// are outstanding (expcnt and lgkmcnt left at their no-wait maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0xF70; }

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row (physical
// chunk = logical chunk ^ big_swz(row)).  A fragment read has lane l on row
// 16 g + l % 16 at logical chunk l / 16.  Chosen by measurement (a probe
// timing ds_read_b128 of this fragment pattern, 16 waves per CU): with
// (row / 2) % 4 the read runs at the rate of a contiguous 1 KB read; with
// (row / 4) % 4, row % 4, no swizzle, or ((row / 2) % 4) ^ ((row / 8) % 2)
// (conflict-free for 32 consecutive rows at one chunk) it takes 1.6-1.8
// times as long.
__device__ __forceinline__ int big_swz(int row) { return (row >> 1) & 3; }

// Epilogue of the large-tile kernel for one wave's 8 x 4 grid of 16x16
// accumulator tiles (128 rows x 64 columns, top-left element (mb, nb)).
// 16x16 accumulator layout: lane holds column lane % 16 and, in register v,
// row 4 (lane / 16) + v of the tile - four consecutive rows of one column.
// Dequantization by the outer product of the scales, the 16-bit outlier
// product through LDS (v_mfma_f32_16x16x32_f16 / _bf16 with the dequantized
// values as C, one 32-outlier chunk per instruction), then Y through LDS to
// whole 16-byte row pieces.

template <bool WRITE_ACC, int HT>
__device__ __forceinline__ void epilogue_big(v4i (&acc)[8][4], const GemmArgs& a, int64_t mb,
                                             int64_t nb, int lane, const StageCtx& sc) {
    constexpr int TM = 8, TN = 4;
    const int64_t T = a.T, N = a.N;
    const int col_l = lane & 15;
    const int row_l = (lane >> 4) * 4;
    if (WRITE_ACC && a.acc_out) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = nb + j * 16 + col_l;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t m = mb + i * 16 + row_l + v;
                    if (m < T && n < N) a.acc_out[m * N + n] = acc[i][j][v];
                }
            }
    }
    // dequantization by the outer product of the scales (1/127^2 folded
    // into the column scale); s_w, s_x and the counts were read before the
    // main loop, s_x reaches every lane through LDS
    float swn[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) swn[j] = sc.sw_pre[j] * (1.0f / 16129.0f);
    const int o = sc.o, opad = sc.opad;
    // 16-bit outlier rows: the caller's W16 (row idx_j), the rows recovered
    // before the matmul (row j, when o fits), or - memory-halved variant
    // without room for those - recovered here from the Int8 weight,
    // W^[k,n] = fp16(q[n,k] * fp32(s_w[n] / 127))
    const bool recover = a.w16 == nullptr || (a.w16_rows > 0 && o > a.w16_rows);
    const bool by_pos = !recover && a.w16_rows > 0;   // W16 row = outlier position
    if (sc.tid < 256) sc.sxs[sc.tid] = sc.sx_pre;
    __syncthreads();
    const int wm0 = (int)(mb - sc.m0), wn0 = (int)(nb - sc.n0);
    // the integer accumulators die here; the fp32 values take their registers
    v4f y[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // the lane's four rows of strip i: one 16-byte LDS read (rows past T
        // hold the last row's scale; those outputs are never stored)
        const float4 s = *reinterpret_cast<const float4*>(sc.sxs + wm0 + i * 16 + row_l);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            y[i][j][0] = (float)acc[i][j][0] * s.x * swn[j];
            y[i][j][1] = (float)acc[i][j][1] * s.y * swn[j];
            y[i][j][2] = (float)acc[i][j][2] * s.z * swn[j];
            y[i][j][3] = (float)acc[i][j][3] * s.w * swn[j];
        }
    }
    if (opad > 0) {
        // Staged through LDS, kOC outliers per chunk, double buffered: the
        // 512 threads load the chunk's X columns (256 rows x kOC, coalesced
        // along the compacted outliers) and W rows (kOC x 256 columns,
        // transposed on the way into LDS so that a lane's 8 outliers of one
        // column are contiguous), then every wave reads its MFMA fragments
        // from LDS.  The next chunk's loads fly during this chunk's MFMAs;
        // the outlier indices are fetched one chunk ahead of their use.  A
        // chunk's slots past o hold zeros on both sides.
        __syncthreads();   // the main loop's LDS reads are complete
        const int t = sc.tid;
        const int e = t & 31, cb = t >> 5;        // W: outlier slot, 16-column block
        const int xr = t >> 1, xh = t & 1;        // X: tile row, 16-outlier half
        const int64_t xrow = sc.m0 + xr;
        float dcol[16];
        if (recover) {
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int64_t n = sc.n0 + cb * 16 + c;
                dcol[c] = n < N ? a.sw[n] / 127.0f : 0.0f;
            }
        }
        // k: the W16 row of slot e (the outlier's dimension, or its position
        // for recovered rows), or the dimension whose Wq bytes are recovered
        // (the tile's columns are one panel of the blocked Wq and K % 64 ==
        // 0: byte (n, k) is at wk[64 (n - n0)] for the k part wk)
        const int64_t wrows = N - sc.n0 < kPanel ? N - sc.n0 : kPanel;
        int k_next = e < o ? (by_pos ? e : sc.k_first) : -1;
        uint4 wv[2], xv[2];
        auto load_chunk = [&](int jc) {
            const int k = k_next;
            k_next = jc + kOC + e < o ? (by_pos ? jc + kOC + e : a.idx[jc + kOC + e]) : -1;
            const int kc = k < 0 ? 0 : k;   // (k < 0: nothing is read)
            const int8_t* wk = a.wq + sc.n0 * a.K + (int64_t)(kc & ~(int)(kKTile - 1)) * wrows +
                               (kc & (int)(kKTile - 1));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t n = sc.n0 + cb * 16 + h * 8;
                if (!recover) {
                    wv[h] = (k >= 0 && n < N)
                                ? *reinterpret_cast<const uint4*>(a.w16 + (int64_t)k * N + n)
                                : make_uint4(0u, 0u, 0u, 0u);
                } else {
                    uint32_t p[4];
#pragma unroll
                    for (int c = 0; c < 8; c += 2) {
                        const int nl = cb * 16 + h * 8 + c;   // column inside the tile
                        const uint16_t lo = (k >= 0 && n + c < N)
                                                ? recover_weight<HT>(wk[nl * kKTile], dcol[h * 8 + c])
                                                : (uint16_t)0;
                        const uint16_t hi = (k >= 0 && n + c + 1 < N)
                                                ? recover_weight<HT>(wk[(nl + 1) * kKTile],
                                                                     dcol[h * 8 + c + 1])
                                                : (uint16_t)0;
                        p[c >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
                    }
                    wv[h] = make_uint4(p[0], p[1], p[2], p[3]);
                }
                const int jx = jc + xh * 16 + h * 8;
                xv[h] = (xrow < T && jx < opad)
                            ? *reinterpret_cast<const uint4*>(a.xo + xrow * opad + jx)
                            : make_uint4(0u, 0u, 0u, 0u);
            }
        };
        auto store_chunk = [&](int buf) {
            int8_t* xs = sc.lds + buf * 2 * kStageHalf;
            int8_t* ws = xs + kStageHalf;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                *reinterpret_cast<uint4*>(xs + xr * kOS + xh * 32 + h * 16) = xv[h];
                const uint32_t w4[4] = {wv[h].x, wv[h].y, wv[h].z, wv[h].w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    *reinterpret_cast<uint16_t*>(ws + (cb * 16 + h * 8 + c) * kOS + e * 2) =
                        (uint16_t)(w4[c >> 1] >> ((c & 1) * 16));
            }
        };
        if (sc.pre_loaded && !recover) {
            // chunk 0 was loaded before the dequantization
            k_next = kOC + e < o ? (by_pos ? kOC + e : a.idx[kOC + e]) : -1;
            wv[0] = sc.pre_w[0]; wv[1] = sc.pre_w[1];
            xv[0] = sc.pre_x[0]; xv[1] = sc.pre_x[1];
        } else {
            load_chunk(0);
        }
        // fragments: lane reads row (column) lane % 16 of its strip, outlier
        // slots 8 (lane / 16) .. +7 of the chunk
        const int ko = (lane >> 4) * 16;
        for (int jc = 0; jc < opad; jc += kOC) {
            const int buf = (jc / kOC) & 1;
            store_chunk(buf);
            __syncthreads();
            if (jc + kOC < opad) load_chunk(jc + kOC);
            const int8_t* xs = sc.lds + buf * 2 * kStageHalf;
            const int8_t* ws = xs + kStageHalf;
            v8u16 wb[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j)
                wb[j] = *reinterpret_cast<const v8u16*>(ws + (wn0 + j * 16 + col_l) * kOS + ko);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const v8u16 xa = *reinterpret_cast<const v8u16*>(xs + (wm0 + i * 16 + col_l) * kOS + ko);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (HT == kHalfBF16)
                        y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(v8bf, xa), __builtin_bit_cast(v8bf, wb[j]), y[i][j], 0, 0, 0);
                    else
                        y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, xa), __builtin_bit_cast(v8h, wb[j]), y[i][j], 0, 0, 0);
                }
            }
        }
    }
    // Y through LDS, then out as whole 16-byte pieces of rows (1 KB per wave
    // store instruction).  The tile is kept in LDS as groups of 4 rows with
    // each column's 4 values contiguous, so a lane writes the 4 rows of one
    // column it holds as one 8-byte write (16 lanes: 128 contiguous bytes of
    // one group, the next 16 lanes the next group half a bank period away).
    // The store phase reads, per thread, 8 columns of a group (64 contiguous
    // bytes) and regroups the 16-bit values into the group's 4 row pieces
    // with byte permutes.
    __syncthreads();   // every LDS read of the main loop and the outlier stage is done
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int grp = (wm0 + i * 16 + row_l) >> 2;
            const int nl = wn0 + j * 16 + col_l;
            const uint32_t lo = (uint32_t)f32_to_h16<HT>(y[i][j][0]) | ((uint32_t)f32_to_h16<HT>(y[i][j][1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_h16<HT>(y[i][j][2]) | ((uint32_t)f32_to_h16<HT>(y[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(sc.lds + grp * kYG + nl * 8) = make_uint2(lo, hi);
        }
    __syncthreads();
    const int c = sc.tid & 31;           // columns 8 c .. 8 c + 7 of the tile
    const int64_t n = sc.n0 + c * 8;     // N % 8 == 0: a piece is all in or all out
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int grp = (sc.tid >> 5) + 16 * q;
        const uint4* src = reinterpret_cast<const uint4*>(sc.lds + grp * kYG + c * 64);
        // d[4 j2 + r/2 ...]: column pairs; d[2 j] = rows 0, 1 of column j;
        // d[2 j + 1] = rows 2, 3
        uint32_t d[16];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint4 v = src[h];
            d[4 * h] = v.x; d[4 * h + 1] = v.y; d[4 * h + 2] = v.z; d[4 * h + 3] = v.w;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t m = sc.m0 + grp * 4 + k;
            uint32_t w[4];
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                // columns 2 j2 and 2 j2 + 1 of row k
                const uint32_t a0 = d[4 * j2 + (k >> 1)], a1 = d[4 * j2 + 2 + (k >> 1)];
                w[j2] = (k & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
            }
            if (m < T && n < N)
                *reinterpret_cast<uint4*>(a.y + m * N + n) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Large-tile kernel for prefill shapes: a 256x256 workgroup tile over 8
// waves of 128 x 64 (two waves share each SIMD: while one waits to issue,
// the other keeps the MFMA pipe busy), each a grid of 8 x 4 16x16 tiles of
// v_mfma_i32_16x16x64_i8 (128 int32 accumulators per lane; a 64-deep
// k-tile is one instruction deep).  The int8 products run on the 16x16x64
// instruction rather than 32x32x32 because the part's clock is power
// limited: back-to-back on random operands the 32x32x32 form held 1.62 GHz
// and the 16x16x64 form 1.92 GHz for the same work per cycle.
// Operands go from global memory straight into LDS (global_load_lds_dwordx4:
// no VGPR staging, no LDS store instructions) through a ring of 4 buffers of
// 32 KB (BK = 64).  A wave instruction fills 1 KB of LDS, lane l landing at
// byte 16*l, so the swizzle is applied by choosing which global chunk each
// lane fetches.
//
// Per k-tile a wave issues 32 MFMAs on fragment set P (the 12 fragments of
// tile kt, read during the previous k-tile) while it reads tile kt+1 into
// set Q and copies tile kt+4 into tile kt's buffer; the sets alternate
// between k-tiles.  One barrier per k-tile, after the first 4 MFMAs: after
// it every wave's reads of tile kt are complete (each waited for them) and
// every wave's copies of tile kt+1 have landed.  The reads then go out over
// 16 MFMAs and the copies over the rest (all 8 waves leave the barrier
// together, and issuing the 12 reads back to back queued them behind each
// other in the LDS: 4% slower).  Requires K % 64 == 0; rows
// past T or N are clamped to the last valid row (they only feed outputs
// that are never stored).
template <bool WRITE_ACC, int HT>
__global__ __launch_bounds__(512) void k_gemm_i8_big(GemmArgs a) {
    constexpr int BM = 256, BN = 256, BK = 64, STAGES = 4;
    constexpr int WAVES = 8;
    constexpr int TM = 8, TN = 4;                    // 16x16 tiles per wave
    constexpr int NF = TM + TN;                      // fragments per k-tile
    constexpr int NM = TM * TN;                      // MFMAs per k-tile
    constexpr int STAGE_BYTES = (BM + BN) * BK;
    constexpr int GPW = 16 / WAVES;                  // 1 KB groups of A (and of B) per wave
    constexpr int LOADS = 2 * GPW;                   // copies per lane per tile
    static_assert(NF <= NM && LOADS <= NM, "interleave needs one MFMA per read and copy");
    constexpr int LDS_BYTES = STAGES * STAGE_BYTES > kYBytes ? STAGES * STAGE_BYTES : kYBytes;
    static_assert(LDS_BYTES >= kStageBytes, "outlier stage fits");
    __shared__ __attribute__((aligned(1024))) int8_t lds[LDS_BYTES];
    __shared__ __attribute__((aligned(16))) float sxs[BM];
    __shared__ int ks_first;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t T = a.T, K = a.K, N = a.N;
    const int64_t MT = ceil_div(T, BM);
    // K split: whole tiles first, then the split tiles' first and second halves
    // With the K split (ksplit = 2) the first ks_full tiles run all of K
    // (whole rounds of the CUs) and the rest as two halves: the grid holds
    // the whole tiles, then the split tiles' first halves, then their second
    // halves, so a unit never waits for another (half = -1: a whole tile).
    // Split tile si = tix - full keeps its partial sums and counter at si.
    const int64_t tiles = ceil_div(T, (int64_t)BM) * ceil_div(N, (int64_t)BN);
    const int64_t full = a.ksplit == 2 ? a.ks_full : tiles;
    int half = -1;
    int64_t tix = blockIdx.x;
    if (tix >= full) {
        const int64_t v = tix - full, nsplit = tiles - full;
        half = (int)(v / nsplit);
        tix = full + v - half * nsplit;
    }
    const int64_t si = tix - full;   // split tile index (half >= 0)
    const int64_t bid = xcd_tile(tix, tiles);
    const int64_t m0 = (bid % MT) * BM;
    const int64_t n0 = (bid / MT) * BN;
    const int wm0 = (wave & 1) * 128;
    const int wn0 = (wave >> 1) * 64;
    // what the epilogue needs, read now (the main loop hides the latency)
    const float sx_pre = a.sx[m0 + (tid & (BM - 1)) < T ? m0 + (tid & (BM - 1)) : T - 1];
    float sw_pre[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn0 + j * 16 + (lane & 15);
        sw_pre[j] = n < N ? a.sw[n] : 0.0f;
    }
    const int o_pre = a.count[0], opad_pre = a.count[1];
    const int k_first = (tid & 31) < o_pre ? a.idx[tid & 31] : -1;

    // copy assignment: wave w fills the 1 KB groups GPW*w .. GPW*w+GPW-1 of A
    // and of B; in a group, lane l writes row 16g + l/4, physical chunk l%4.
    // Copy u < GPW is an A group, u >= GPW a B group.  The tile's rows are
    // one panel of the blocked layout (m0 and n0 are multiples of 256), whose
    // k-tile kt is a block of rows x 64 bytes, row r at 64 r: an address is a
    // per-workgroup scalar base plus a 32-bit lane offset inside the block,
    // and a group's 16 rows are one contiguous kilobyte.
    static_assert(BK == kKTile && BM == kPanel && BN == kPanel, "tile = panel x k-tile");
    const int64_t arows = T - m0 < BM ? T - m0 : BM, brows = N - n0 < BN ? N - n0 : BN;
    const int8_t* abase = a.xq + m0 * K;
    const int8_t* bbase = a.wq + n0 * K;
    uint32_t goff[LOADS];
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
        const int row = (wave * GPW + u) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ big_swz(row);
        const int64_t ra = row < arows ? row : arows - 1;
        const int64_t rb = row < brows ? row : brows - 1;
        goff[u] = (uint32_t)(ra * BK + c * 16);
        goff[GPW + u] = (uint32_t)(rb * BK + c * 16);
    }
    auto copy = [&](int u, int kt, int stage) {
        const bool isa = u < GPW;
        const int8_t* base = isa ? abase + (int64_t)kt * BK * arows : bbase + (int64_t)kt * BK * brows;
        const int8_t* dst = lds + stage * STAGE_BYTES + (isa ? 0 : BM * BK) +
                            (wave * GPW + (isa ? u : u - GPW)) * 1024;
        copy_to_lds16(base, goff[u], dst);
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // fragment q < TM: A rows wm0 + 16 q + lane % 16, q >= TM: B rows
    // wn0 + 16 (q - TM) + lane % 16; k bytes 16 (lane / 16) .. +16 (logical
    // chunk lane / 16).  The swizzle depends on row bits 1..2 only, i.e. on
    // lane % 16, so fragment q is a fixed 1 KB step from the first.
    const int l15 = lane & 15;
    const int csw = ((lane >> 4) ^ big_swz(l15)) * 16;
    const int fa = (wm0 + l15) * BK + csw;
    const int fb = BM * BK + (wn0 + l15) * BK + csw;
    auto foff = [&](int q) { return q < TM ? fa + q * 1024 : fb + (q - TM) * 1024; };
    v4i f0[NF], f1[NF];

    const int nkt = (int)(K / BK);
    const int KT0 = half < 0 ? 0 : half * (nkt / 2);
    const int KT = half < 0 ? nkt : KT0 + nkt / 2;
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int u = 0; u < LOADS; ++u) copy(u, KT0 + st < KT ? KT0 + st : KT - 1, st);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 1)));
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NF; ++q) f0[q] = *reinterpret_cast<const v4i*>(lds + foff(q));

    int s_cur = 0;
    // one k-tile: MFMAs on P (tile kt), reads of tile kt+1 into Q, copies of
    // tile kt+4 (past the last tile: tile KT-1 again, into a buffer that is
    // never read again) into tile kt's buffer.  At the last k-tile the reads
    // of Q fetch a buffer nobody uses.
    auto ktile = [&](int kt, const v4i (&P)[NF], v4i (&Q)[NF]) {
        const int s_next = (s_cur + 1) & (STAGES - 1);
        const int8_t* nxt = lds + s_next * STAGE_BYTES;
        const int kcopy = kt + STAGES < KT ? kt + STAGES : KT - 1;
        // The first BPOS MFMAs need only P, which is in registers: they go
        // out before the barrier, so the pipe has work while the waves meet
        // (whole calls, alternated: up-projection -1.2 to -1.5%, down -0.4
        // to -0.9%, QKV -0.4%; after 2 or 8 MFMAs within noise of 4).  At
        // the barrier P has arrived (this wave's reads of tile kt are done:
        // no wave reads tile kt's buffer again, which the copies below
        // overwrite) and this wave's copies of tile kt+1 have landed.
        // The next tile's 12 fragment reads follow over 16 MFMAs, so they
        // have landed when the wave reaches the next barrier (whose wait
        // includes them); spread over all 32 the last read left with 3
        // MFMAs to go (whole calls -0.6 to -1.2%; over 24, 20 or 12 MFMAs,
        // or with the copies moved, level or slower).  The 4 copies are
        // spread over the rest.
        constexpr int BPOS = 4;
        constexpr int RSPAN = NM / 2;
        static_assert(BPOS + RSPAN <= NM && BPOS + LOADS * ((NM - BPOS) / LOADS) <= NM, "schedule");
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m == BPOS) {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 2)) & ~0xF00);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < NF; ++r) {
                const int q = r < TN ? TM + r : r - TN;   // B fragments first
                if (BPOS + (r * RSPAN) / NF == m) Q[q] = *reinterpret_cast<const v4i*>(nxt + foff(q));
            }
#pragma unroll
            for (int u = 0; u < LOADS; ++u)
                if (BPOS + u * ((NM - BPOS) / LOADS) + 1 == m) copy(u, kcopy, s_cur);
            const int i = m / TN, j = m % TN;
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(P[i], P[TM + j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_cur = s_next;
    };
    for (int kt = KT0; kt < KT; kt += 2) {
        ktile(kt, f0, f1);
        if (kt + 1 < KT) ktile(kt + 1, f1, f0);
    }
    // no LDS copy or read may still be in flight when the LDS is reused or
    // the workgroup retires
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~0xF00);
    if (half >= 0) {
        // K split: each half publishes its int32 sums, and the half that
        // finishes second adds the other's (exact, order independent) and
        // runs the epilogue.  The tile counters were zeroed at launch.
        // The sums travel through agent-scope atomic stores and loads (the
        // other half may run on another XCD, whose L2 is not this one's);
        // the ordering is the memory model's: every wave's stores, then a
        // workgroup barrier, then thread 0's counter increment with
        // release semantics at agent scope; in the other half the same
        // increment acquires, and a barrier orders it before every wave's
        // loads.  A half that finds the other one already done skips
        // publishing its own sums.
        uint64_t* mine = reinterpret_cast<uint64_t*>(a.ks_part) +
                         ((si * 2 + half) * WAVES + wave) * (TM * TN * 2 * 64);
        const uint64_t* other = reinterpret_cast<const uint64_t*>(a.ks_part) +
                                ((si * 2 + (1 - half)) * WAVES + wave) * (TM * TN * 2 * 64);
        if (tid == 0)
            ks_first = __hip_atomic_load(&a.ks_count[si], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const bool other_done = ks_first != 0;
        if (!other_done) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const uint64_t v = (uint64_t)(uint32_t)acc[i][j][2 * q] |
                                           ((uint64_t)(uint32_t)acc[i][j][2 * q + 1] << 32);
                        __hip_atomic_store(mine + ((i * TN + j) * 2 + q) * 64 + lane, v,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();   // every wave's sums are out (and ks_first is read)
        if (tid == 0)
            ks_first = __hip_atomic_fetch_add(&a.ks_count[si], 1, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT) == 0;
        __syncthreads();
        if (ks_first) return;   // the other half finishes the tile
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint64_t v = __hip_atomic_load(other + ((i * TN + j) * 2 + q) * 64 + lane,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    acc[i][j][2 * q] += (int32_t)(uint32_t)v;
                    acc[i][j][2 * q + 1] += (int32_t)(uint32_t)(v >> 32);
                }
    }
    // the first outlier chunk's operands (as the epilogue's staging assigns
    // them), loaded now so that they arrive during the dequantization
    StageCtx sc{lds, tid, m0, n0, sxs, sx_pre, sw_pre, o_pre, opad_pre, k_first, false, {}, {}};
    if (opad_pre > 0 && a.w16 && !(a.w16_rows > 0 && o_pre > a.w16_rows)) {
        const int e = tid & 31, cb = tid >> 5, xr = tid >> 1, xh = tid & 1;
        const int k = e < o_pre ? (a.w16_rows > 0 ? e : k_first) : -1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t n = n0 + cb * 16 + h * 8;
            sc.pre_w[h] = (k >= 0 && n < N) ? *reinterpret_cast<const uint4*>(a.w16 + (int64_t)k * N + n)
                                            : make_uint4(0u, 0u, 0u, 0u);
            const int jx = xh * 16 + h * 8;
            sc.pre_x[h] = (m0 + xr < T && jx < opad_pre)
                              ? *reinterpret_cast<const uint4*>(a.xo + (m0 + xr) * opad_pre + jx)
                              : make_uint4(0u, 0u, 0u, 0u);
        }
        sc.pre_loaded = true;
    }
    epilogue_big<WRITE_ACC, HT>(acc, a, m0 + wm0, n0 + wn0, lane, sc);
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row (streaming
// kernel): 8 consecutive rows land on 8 distinct chunks, and rows r and r+8
// on different chunks too, so a fragment read (lanes on consecutive rows at
// one logical chunk) is free of bank conflicts for 8- and 16-lane service.
__device__ __forceinline__ int stream_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Streaming kernel for 9..256 rows with K % 128 == 0: the matmul is bound by
// the weight stream, so both operands go from global memory straight into
// LDS (global_load_lds_dwordx4, no VGPR staging) through a ring of STAGES
// k-tiles of 128, STAGES - 1 of them in flight.  One barrier per k-tile:
// after it every wave's copies of tile kt have landed and tile kt-1 is no
// longer read, so its buffer takes tile kt+STAGES-1.  BM x BN tile over
// WAVES_M x WAVES_N waves of (BM/WAVES_M) x (BN/WAVES_N); rows past T or N
// are clamped to the last row (never stored).
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool WRITE_ACC, int HT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm_i8_stream(GemmArgs a) {
    constexpr int BK = 128;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int STAGE_BYTES = (BM + BN) * BK;
    constexpr int GA = BM * BK / 1024, GB = BN * BK / 1024;   // 1 KB groups of A and B
    constexpr int LOADS = (GA + GB) / NW;                     // copies per lane per tile
    static_assert(TM >= 1 && TN >= 1 && (GA + GB) % NW == 0, "tile shape");
    static_assert((STAGES - 2) * LOADS <= 63 && STAGES >= 3, "wait count range");
    __shared__ __attribute__((aligned(1024))) int8_t lds[STAGES * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t T = a.T, K = a.K, N = a.N;
    const int64_t MT = ceil_div(T, BM);
    // K split (ksplit = S > 1): unit u is slab u / tiles of tile u % tiles
    // (every tile's first slab is dispatched before any second one)
    const int64_t tiles = MT * ceil_div(N, (int64_t)BN);
    const int S = a.ksplit > 1 ? a.ksplit : 1;
    const int64_t tix = S > 1 ? (int64_t)blockIdx.x % tiles : (int64_t)blockIdx.x;
    const int slab = S > 1 ? (int)((int64_t)blockIdx.x / tiles) : 0;
    const int64_t bid = xcd_tile(tix, tiles);
    const int64_t m0 = (bid % MT) * BM;
    const int64_t n0 = (bid / MT) * BN;
    const int wm0 = (wave % WAVES_M) * WM;
    const int wn0 = (wave / WAVES_M) * WN;

    // copy u of this wave fills 1 KB group g = LOADS * wave + u of the tile
    // (g < GA: rows 8g .. 8g+7 of A, else rows 8(g - GA) .. of B); lane l
    // writes row 8g + l/8 at physical chunk l%8, so it fetches the logical
    // chunk c = (l%8) ^ stream_swz(row).  In the blocked layout the tile's
    // rows lie in one panel (BM and BN divide 256); k-tile kt of 128 is the
    // panel's 64-column k-tiles 2 kt and 2 kt + 1, so chunk c of row r sits
    // in block 2 kt + c/4 at 64 r + 16 (c%4): a scalar base per k-tile plus
    // a 32-bit lane offset, and a group's copy touches 8 whole lines.
    static_assert(BK == 2 * kKTile && kPanel % BM == 0 && kPanel % BN == 0, "tile inside a panel");
    const int64_t pa = m0 - m0 % kPanel, pb = n0 - n0 % kPanel;      // panel starts
    const int64_t arows = T - pa < kPanel ? T - pa : kPanel;
    const int64_t brows = N - pb < kPanel ? N - pb : kPanel;
    const int8_t* abase = a.xq + pa * K;
    const int8_t* bbase = a.wq + pb * K;
    uint32_t goff[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int g = LOADS * wave + u;
        const bool isa = g < GA;
        const int row = (isa ? g : g - GA) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ stream_swz(row);
        // row inside the panel (rows past T or N read the last one)
        const int64_t r = isa ? (m0 + row < T ? m0 - pa + row : T - 1 - pa)
                              : (n0 + row < N ? n0 - pb + row : N - 1 - pb);
        const int64_t rows = isa ? arows : brows;
        goff[u] = (uint32_t)((c >> 2) * kKTile * rows + r * kKTile + (c & 3) * 16);
    }
    auto copy = [&](int u, int kt, int stage) {
        const int g = LOADS * wave + u;
        const bool isa = g < GA;
        const int8_t* base = isa ? abase + (int64_t)kt * BK * arows : bbase + (int64_t)kt * BK * brows;
        const int8_t* dst = lds + stage * STAGE_BYTES + (isa ? g * 1024 : BM * BK + (g - GA) * 1024);
        copy_to_lds16(base, goff[u], dst);
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // fragment offsets inside a tile for k-step 0; k-step s adds 32 s bytes
    // of logical k, i.e. logical chunk 2 s + lane / 32
    // k-tiles KT0 .. KT-1 of 128 (all of K without the split)
    const int KTA = (int)(K / BK);
    const int kps = (KTA + S - 1) / S;
    const int KT0 = slab * kps;
    const int KT = KT0 + kps < KTA ? KT0 + kps : KTA;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
#pragma unroll
        for (int u = 0; u < LOADS; ++u) copy(u, KT0 + st < KT ? KT0 + st : KT - 1, st);

    int s_cur = 0;
    for (int kt = KT0; kt < KT; ++kt) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 2) * LOADS));   // this wave's part of tile kt
        __syncthreads();                                                 // everyone's part; tile kt-1 read
        const int s_fill = s_cur == 0 ? STAGES - 1 : s_cur - 1;
        const int kf = kt + STAGES - 1 < KT ? kt + STAGES - 1 : KT - 1;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) copy(u, kf, s_fill);
        const int8_t* cur = lds + s_cur * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            const int c = s * 2 + (lane >> 5);
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm0 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const v4i*>(cur + row * BK + ((c ^ stream_swz(row)) * 16));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn0 + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const v4i*>(cur + BM * BK + row * BK + ((c ^ stream_swz(row)) * 16));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        s_cur = s_cur == STAGES - 1 ? 0 : s_cur + 1;
    }
    // the copies past the last tile went to buffers no one reads; let them
    // land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (BM == 64 && S > 1) {
        // 64x64 tiles: the slab's int32 sums go to part [S][T][N] with plain
        // stores and a second kernel (launch_finish_partials) adds the slabs
        // and completes Y; the kernel boundary orders the two.  32x32
        // accumulator layout: lane holds column lane % 32 and, in register
        // r, row 8 (r / 4) + 4 (lane / 32) + r % 4 of the 32x32 tile.
        int32_t* part = a.ks_part + (int64_t)slab * T * N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t n = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (m < T && n < N) part[m * N + n] = acc[i][j][r];
                }
            }
        return;
    }
    if (S > 1) {
        // Every slab publishes its int32 sums, then counts itself done on the
        // tile's counter (zeroed before the launch); the slab that counts
        // last adds the others' sums (exact, in any order) and runs the
        // epilogue.  Ordering as in the large-tile kernel's K split: agent-
        // scope atomic stores (the slabs may run on different XCDs, whose L2
        // caches are not shared), a workgroup barrier, thread 0's acq_rel
        // increment at agent scope, a barrier, agent-scope atomic loads.  No
        // unit waits for another.
        __shared__ int last;
        constexpr int PER = TM * TN * 8 * 64;                 // 64-bit words per wave
        uint64_t* part = reinterpret_cast<uint64_t*>(a.ks_part) + (tix * S) * NW * PER;
        uint64_t* mine = part + (slab * NW + wave) * PER;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint64_t v = (uint64_t)(uint32_t)acc[i][j][2 * q] |
                                       ((uint64_t)(uint32_t)acc[i][j][2 * q + 1] << 32);
                    __hip_atomic_store(mine + ((i * TN + j) * 8 + q) * 64 + lane, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();   // every wave's sums are out
        if (tid == 0)
            last = __hip_atomic_fetch_add(&a.ks_count[tix], 1, __ATOMIC_ACQ_REL,
                                          __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!last) return;   // the last slab finishes the tile
        for (int o = 0; o < S; ++o) {
            if (o == slab) continue;
            const uint64_t* other = part + (o * NW + wave) * PER;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint64_t v = __hip_atomic_load(other + ((i * TN + j) * 8 + q) * 64 + lane,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        acc[i][j][2 * q] += (int32_t)(uint32_t)v;
                        acc[i][j][2 * q + 1] += (int32_t)(uint32_t)(v >> 32);
                    }
        }
    }
    epilogue<TM, TN, WRITE_ACC, HT, BN, 64 * NW>(acc, a, m0 + wm0, n0 + wn0, lane,
                                                 StageCtx{lds, tid, m0, n0, nullptr, 0.0f, nullptr, 0, 0, -1,
                                                          false, {}, {}});
}

__global__ void k_zero_i32(int32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int HT>
hipError_t launch_stream(const GemmArgs& a, hipStream_t stream) {
    const int64_t tiles = ceil_div(a.T, BM) * ceil_div(a.N, BN);
    constexpr int threads = 64 * WAVES_M * WAVES_N;
    GemmArgs b = a;
    if (b.ksplit > 1 && BM == 64) {
        if (!b.ks_part) return hipErrorInvalidValue;   // partial sums, finished by a second kernel
    } else if (b.ksplit > 1) {
        // the K split's tile counters start at zero (a kernel, not a memset,
        // so the call can be captured in a graph)
        if (!b.ks_count || !b.ks_part) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)ceil_div(tiles, 256)), dim3(256), 0, stream,
                           b.ks_count, tiles);
    } else {
        b.ksplit = 1;
    }
    const int64_t units = tiles * b.ksplit;
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8_stream<BM, BN, WAVES_M, WAVES_N, STAGES, true, HT>),
                           dim3((unsigned)units), dim3(threads), 0, stream, b);
    else
        hipLaunchKernelGGL((k_gemm_i8_stream<BM, BN, WAVES_M, WAVES_N, STAGES, false, HT>),
                           dim3((unsigned)units), dim3(threads), 0, stream, b);
    if (b.ksplit > 1 && BM == 64) {
        // the recovered rows of the memory-halved variant are indexed by
        // outlier position; the finishing kernel takes W16 [K,N] or recovers
        // from Wq itself
        const uint16_t* w16 = b.w16_rows > 0 ? nullptr : b.w16;
        return launch_finish_partials(HT, b.T, b.K, b.N, b.ksplit, b.ks_part, b.wq, b.sw, w16, b.sx,
                                      b.count, b.idx, b.xo, b.y, b.acc_out, stream);
    }
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WAVES_M, int HT>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    const int64_t tiles = ceil_div(a.T, BM) * ceil_div(a.N, BN);
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, WAVES_M, true, HT>), dim3((unsigned)tiles),
                           dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, WAVES_M, false, HT>), dim3((unsigned)tiles),
                           dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int HT>
hipError_t launch_big(const GemmArgs& a, hipStream_t stream) {
    const int64_t tiles = ceil_div(a.T, 256) * ceil_div(a.N, 256);
    GemmArgs b = a;
    b.ks_full = tiles;
    if (a.ksplit == 2) {
        const KSplitPlan p = gemm_ksplit_plan(a.T, a.K, a.N);
        if (p.nsplit <= 0) return hipErrorInvalidValue;
        // the split tiles' counters start at zero: set by the activation pass
        // of the same call, or here (a kernel rather than a memset, so the
        // call can be captured in a graph)
        if (!a.ks_zeroed)
            hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)ceil_div(p.nsplit, 256)), dim3(256), 0, stream,
                               a.ks_count, p.nsplit);
        b.ks_full = p.full;
    }
    const int64_t units = b.ks_full + 2 * (tiles - b.ks_full);
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8_big<true, HT>), dim3((unsigned)units), dim3(512), 0, stream, b);
    else
        hipLaunchKernelGGL((k_gemm_i8_big<false, HT>), dim3((unsigned)units), dim3(512), 0, stream, b);
    return hipGetLastError();
}

// Below the large-tile kernel's range the matmul streams the weight past
// few rows of X, and the time goes to keeping enough of that stream in
// flight.  Measured at K=8192, N=28672 with the weight not cache resident
// (GEMM kernel alone): T=32 streaming 64x64 (4 stages: 64 KB of LDS, two
// workgroups per CU, 448 tiles all resident at once) 48-51 us, register-
// staged 32x128x256 55 us, 32x256x128 88 us; T=64 streaming 64x64 54 us,
// register-staged 64x128x256 60 us, 128x128x64 98 us; T=128 streaming
// 128x128 (4 stages) 61-63 us, register-staged 64x128x128 81-87 us,
// 128x128x64 98 us; with 256 outliers (their W rows staged through LDS)
// T=64 62.5 us and T=128 71 us against 114 and 128 us.  The register-staged
// kernels keep the shapes with K % 128 != 0.
// 129..256 rows: a 256x128 streaming tile (4 waves of 64x128) while its
// tiles fit the chip in one round and the large-tile kernel would not split
// K - whole calls, T=160/256: K=8192 N=28672 109 -> 94 / 120 -> 101 us,
// K=12288 N=12288 166 -> 130 us, K=4096 N=14336 66 -> 55 us; with 288 or
// more tiles (N >= 36864) or a split K the large-tile kernel stays ahead.
template <int HT>
hipError_t launch_gemm_typed(const GemmArgs& a, hipStream_t stream) {
    if (stream_256x128(a.T, a.K, a.N)) return launch_stream<256, 128, 4, 1, 3, HT>(a, stream);
    if (a.T > 128 && a.K % 64 == 0) return launch_big<HT>(a, stream);
    if (a.K % 128 == 0) {
        if (a.T <= 64) return launch_stream<64, 64, 2, 2, 4, HT>(a, stream);
        return launch_stream<128, 128, 2, 2, 4, HT>(a, stream);
    }
    if (a.T <= 32) return launch_cfg<32, 128, 256, 1, HT>(a, stream);
    if (a.T <= 64) return launch_cfg<64, 128, 256, 2, HT>(a, stream);
    if (a.T <= 128) return launch_cfg<64, 128, 128, 2, HT>(a, stream);
    return launch_cfg<128, 128, 64, 2, HT>(a, stream);
}

}  // namespace

// The large-tile kernel runs one workgroup per CU at a time, so a grid of
// `tiles` takes ceil(tiles / CUs) rounds.  Splitting K in two doubles the
// units and halves their length; it pays where that removes at least a
// quarter of the rounds (e.g. 384 tiles on 256 CUs: 2 rounds -> 1.5) and K
// is long enough that publishing and adding the 256 KB of partial sums per
// tile is small against the half tile.  Measured, whole calls: down
// projection T=2048, K=49152, N=12288 13% faster; T=512, K=12288: N=36864
// 344 -> 304 us, N=49152 347 -> 342 us (T=384, N=49152 1% slower).  Up to
// 256 rows the 256x128 streaming tile takes the shapes with K below 24576.
// Only the split tiles hold partial sums (workspace: 128 split tiles of the
// down projection's 384, 32 of 288 at T=512, N=36864).  Staggering whole
// rounds with a split half-round dispatched first (so that half the CUs
// store their Y tiles half a tile apart from the other half) measured
// level on the up, QKV, out and down projections.
KSplitPlan gemm_ksplit_plan(int64_t T, int64_t K, int64_t N) {
    const int64_t tiles = ceil_div(T, 256) * ceil_div(N, 256);
    const int64_t cus = device_cus();
    const KSplitPlan none{tiles, 0};
    if (!(T > 128 && K % 128 == 0)) return none;
    const int64_t kmin = T > 256 ? 8192 : 24576;
    if (K >= kmin) {
        const int64_t r1 = ceil_div(tiles, cus);          // rounds of whole tiles
        const int64_t r2 = ceil_div(2 * tiles, cus);      // rounds of half tiles
        if (2 * r2 <= 3 * r1) {                           // half-rounds r2/2 <= 3/4 of r1
            // whole tiles fill whole rounds of the CUs; only the rest is split
            // (T=2048, N=12288: 384 tiles on 256 CUs run as 256 whole tiles and
            // 128 split ones, 1.5 tile times either way, a third of the partial
            // sums of splitting all 384)
            const int64_t full = tiles > cus && tiles % cus != 0 ? cus * (tiles / cus) : 0;
            return {full, tiles - full};
        }
    }
    return none;
}

// K split of the streaming kernel (K % 128 == 0), when its tiles leave
// workgroup slots idle: S slabs so that tiles x S fill the slots once, each
// slab at least 16 k-tiles of 128, at most 8 slabs.
//  - 128x128 tiles (65..128 rows, one per CU) and 256x128 tiles (129..256
//    rows, one per CU), at most half of the CUs busy: the last slab to
//    finish adds the others' sums (published with
//    agent-scope atomics) and runs the epilogue.  Whole calls: T = 128,
//    N = 12288: K = 12288 -9%, K = 49152 -26%; T = 80, K = 49152 -28%.
//  - 64x64 tiles (up to 64 rows, two per CU), at most a quarter of the
//    slots busy (128 tiles on 256 CUs): every slab writes plain partial
//    sums [S][T][N] and a finishing kernel completes Y (the same scheme
//    with the release/acquire handoff ran 15-49% slower: each of the many
//    small units pays an L2 write-back and invalidate).  Whole calls:
//    T = 64, K = 12288: N = 2048 -39%, 4096 -23%, 8192 -10%; T = 64,
//    K = 49152, N = 4096 -45%; T = 32, K = 4096, N = 4096 -4%; with 192
//    tiles (N = 12288) it was 8-19% slower, hence the quarter.
StreamSplit stream_split(int64_t T, int64_t K, int64_t N) {
    StreamSplit p{1, 0, 0};
    const bool wide = stream_256x128(T, K, N);   // 129..256 rows: 256x128 tiles, one per CU
    if ((T > 128 && !wide) || K % 128 != 0) return p;
    const int64_t bm = T <= 64 ? 64 : T <= 128 ? 128 : 256;
    const int64_t bn = wide ? 128 : bm;
    const int64_t per_cu = T <= 64 ? 2 : 1;
    p.tiles = ceil_div(T, bm) * ceil_div(N, bn);
    p.tile_bytes = bm * bn * 4;
    const int64_t slots = device_cus() * per_cu;
    const int64_t s = std::min<int64_t>(slots / p.tiles, (K / 128) / kStreamMinSlab);
    const int64_t fill = T <= 64 ? 4 : 2;   // tiles may occupy at most 1/fill of the slots
    if (fill * p.tiles <= slots && s >= 2) p.s = (int)std::min<int64_t>(s, kStreamMaxSplit);
    return p;
}

int gemm_ksplit(int64_t T, int64_t K, int64_t N) {
    if (T <= 128 || stream_256x128(T, K, N)) return stream_split(T, K, N).s;
    return gemm_ksplit_plan(T, K, N).nsplit > 0 ? 2 : 1;
}

// 129..256 rows on the 256x128 streaming tile while its tiles fit the CUs
// in one round and the large-tile kernel would not split K
bool stream_256x128(int64_t T, int64_t K, int64_t N) {
    return T > 128 && T <= 256 && K % 128 == 0 && ceil_div(N, 128) <= device_cus() &&
           gemm_ksplit_plan(T, K, N).nsplit == 0;
}

hipError_t launch_gemm(const GemmArgs& a, int ht, hipStream_t stream) {
    const bool wide = stream_256x128(a.T, a.K, a.N);
    const bool big_split = a.ksplit == 2 && a.T > 128 && !wide;
    const bool stream_split_ok = a.ksplit >= 2 && (a.T <= 128 || wide) &&
                                 a.ksplit == stream_split(a.T, a.K, a.N).s;
    if (a.ksplit != 1 &&
        !((big_split || stream_split_ok) && a.ks_count && a.ks_part && a.K % 128 == 0))
        return hipErrorInvalidValue;
    return ht == kHalfBF16 ? launch_gemm_typed<kHalfBF16>(a, stream)
                           : launch_gemm_typed<kHalfF16>(a, stream);
}

}  // namespace i8mm
