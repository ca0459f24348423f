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

// Epilogue shared by the matmul kernels, for one wave's TM x TN grid of
// 32x32 accumulator tiles whose top-left output element is (mb, nb).
// 32x32 accumulator layout: lane holds column (lane & 31) and, in register
// r, row 8*(r/4) + 4*(lane/32) + (r%4) of the tile.
// What the large-tile kernel hands its epilogue for staging the outlier
// operands through LDS (the other kernels pass an empty one).
struct StageCtx {
    int8_t* lds;         // at least kStageBytes and kYBytes, free once the main loop is done
    int tid;             // 0 .. 511
    int64_t m0, n0;      // the workgroup's 256 x 256 output tile
    float* sxs;          // 256 floats of LDS outside the above for the tile's row scales
    float sx_pre;        // s_x of tile row tid (tid < 256; the last row past T)
    const float* sw_pre; // s_w of the lane's TN columns (0 past N)
    int o, opad;         // outlier count and its padded value
};
constexpr int kOC = 32;                       // outliers per staged chunk
constexpr int kOS = kOC * 2 + 16;             // bytes per staged row / column (padded)
constexpr int kStageHalf = 256 * kOS;         // X part (rows) or W part (columns)
constexpr int kStageBytes = 4 * kStageHalf;   // two buffers of X and W
constexpr int kYS = 256 * 2 + 16;             // bytes per row of the staged Y tile (padded)
constexpr int kYBytes = 256 * kYS;            // the 256 x 256 tile of 16-bit Y values

// SBN > 0 (streaming kernel, STH threads, n-tile of SBN columns): with more
// than 16 outliers the outlier W rows go through LDS like the large-tile
// kernel's (sc.lds, sc.tid and sc.n0 used).
template <int TM, int TN, bool WRITE_ACC, int HT, bool STAGED = false, int SBN = 0, int STH = 256>
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
    // (the large-tile kernel read s_w, s_x and the counts before its main
    // loop, so their latency is hidden; s_x reaches every lane through LDS)
    float swn[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = nb + j * 32 + col_l;
        if constexpr (STAGED) swn[j] = sc.sw_pre[j] * (1.0f / 16129.0f);
        else swn[j] = n < N ? a.sw[n] * (1.0f / 16129.0f) : 0.0f;
    }
    const int o = STAGED ? sc.o : a.count[0];
    const int opad = STAGED ? sc.opad : a.count[1];
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
        if constexpr (STAGED) dn[j] = recover ? sc.sw_pre[j] / 127.0f : 0.0f;
        else dn[j] = recover && n < N ? a.sw[n] / 127.0f : 0.0f;
    }
    if constexpr (STAGED) {
        if (sc.tid < 256) sc.sxs[sc.tid] = sc.sx_pre;
        __syncthreads();
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
            if constexpr (STAGED) {
                const float4 v = *reinterpret_cast<const float4*>(sc.sxs + (m - (int)sc.m0));
                sxm[4 * g] = v.x; sxm[4 * g + 1] = v.y; sxm[4 * g + 2] = v.z; sxm[4 * g + 3] = v.w;
            } else {
                if (m + 3 < Ti) {
                    const float4 v = *reinterpret_cast<const float4*>(a.sx + m);
                    sxm[4 * g] = v.x; sxm[4 * g + 1] = v.y; sxm[4 * g + 2] = v.z; sxm[4 * g + 3] = v.w;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) sxm[4 * g + q] = a.sx[m + q < Ti ? m + q : Ti - 1];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) y[i][j][r] = (float)acc[i][j][r] * sxm[r] * swn[j];
    }
    if constexpr (!STAGED) {
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
                int k_next = e < o ? (by_pos ? e : a.idx[e]) : -1;
                uint4 wv[NV];
                auto load_chunk = [&](int jc) {
                    const int k = k_next;
                    k_next = jc + kOC + e < o ? (by_pos ? jc + kOC + e : a.idx[jc + kOC + e]) : -1;
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
                                                        ? recover_weight<HT>(a.wq[nc * a.K + k], dcol[h * 8 + c])
                                                        : (uint16_t)0;
                                const uint16_t hi = (k >= 0 && nc + 1 < N)
                                                        ? recover_weight<HT>(a.wq[(nc + 1) * a.K + k],
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
                                       ? recover_weight<HT>(a.wq[n * a.K + kk[e]], dn[j])
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
    } else if (opad > 0) {
        // Staged through LDS, kOC outliers per chunk, double buffered: the
        // 512 threads load the chunk's X columns (256 rows x kOC, coalesced
        // along the compacted outliers) and W rows (kOC x 256 columns,
        // transposed on the way into LDS so that a lane's 8 outliers of one
        // column are contiguous), then every wave reads its MFMA fragments
        // from LDS.  The next chunk's loads fly during this chunk's MFMAs;
        // the outlier indices are fetched one chunk ahead of their use.
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
        int k_next = e < o ? (by_pos ? e : a.idx[e]) : -1;
        uint4 wv[2], xv[2];
        auto load_chunk = [&](int jc) {
            const int k = k_next;
            k_next = jc + kOC + e < o ? (by_pos ? jc + kOC + e : a.idx[jc + kOC + e]) : -1;
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
                        const int64_t n0c = n + c;
                        const uint16_t lo = (k >= 0 && n0c < N)
                                                ? recover_weight<HT>(a.wq[n0c * a.K + k], dcol[h * 8 + c])
                                                : (uint16_t)0;
                        const uint16_t hi = (k >= 0 && n0c + 1 < N)
                                                ? recover_weight<HT>(a.wq[(n0c + 1) * a.K + k],
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
        load_chunk(0);
        for (int jc = 0; jc < opad; jc += kOC) {
            const int buf = (jc / kOC) & 1;
            store_chunk(buf);
            __syncthreads();
            if (jc + kOC < opad) load_chunk(jc + kOC);
            const int8_t* xs = sc.lds + buf * 2 * kStageHalf;
            const int8_t* ws = xs + kStageHalf;
            const int wm0 = (int)(mb - sc.m0), wn0 = (int)(nb - sc.n0);
#pragma unroll
            for (int ks = 0; ks < kOC / 16; ++ks) {
                if (jc + ks * 16 >= opad) break;
                const int ko = ks * 32 + (lane >> 5) * 16;
                v8u16 wb[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    wb[j] = *reinterpret_cast<const v8u16*>(ws + (wn0 + j * 32 + col_l) * kOS + ko);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const v8u16 xa =
                        *reinterpret_cast<const v8u16*>(xs + (wm0 + i * 32 + col_l) * kOS + ko);
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
    }
    if constexpr (STAGED) {
        // Y through LDS: every wave writes its 16-bit values into a row-major
        // 256 x 256 tile, then the workgroup stores whole 16-byte pieces of
        // rows (1 KB per wave instruction) instead of 2-byte scattered
        // stores.  Rows are padded by 16 bytes, so the two row groups of a
        // lane write (rows 4 apart) fall on different banks.
        __syncthreads();   // every LDS read of the main loop and the outlier stage is done
        const int wm0 = (int)(mb - sc.m0), wn0 = (int)(nb - sc.n0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = wm0 + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                    const int nl = wn0 + j * 32 + col_l;
                    *reinterpret_cast<uint16_t*>(sc.lds + ml * kYS + nl * 2) =
                        f32_to_h16<HT>(y[i][j][r]);
                }
        __syncthreads();
        const int c = sc.tid & 31;
        const int64_t n = sc.n0 + c * 8;   // N % 8 == 0: a piece is all in or all out
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int row = (sc.tid >> 5) + 16 * p;
            const int64_t m = sc.m0 + row;
            const uint4 v = *reinterpret_cast<const uint4*>(sc.lds + row * kYS + c * 16);
            if (m < T && n < N) *reinterpret_cast<uint4*>(a.y + m * N + n) = v;
        }
        return;
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
// s_waitcnt immediate for lgkmcnt(0) only (vmcnt 63, expcnt 7 = no wait)
constexpr int kLgkm0 = 0xC07F;

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row.  A fragment
// read has lanes 0..31 on 32 consecutive rows at one logical chunk; with this
// swizzle any 8 consecutive rows land on 8 distinct 16-byte slots of a
// 128-byte window and any 16 consecutive rows on 16 distinct slots of a
// 256-byte window, so the read is free of bank conflicts whether the LDS
// serves 8 or 16 lanes of a ds_read_b128 per cycle.
__device__ __forceinline__ int big_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// Large-tile kernel for prefill shapes: a 256x256 workgroup tile split over
// 2 x WN waves; each wave owns a 128 x (256/WN) grid of 32x32 MFMA tiles.
// Operands go from global memory straight into LDS (global_load_lds_dwordx4:
// no VGPR staging, no LDS store instructions) through a ring of 4 buffers of
// 32 KB (BK = 64).  A wave instruction fills 1 KB of LDS, lane l landing at
// byte 16*l, so the swizzle is applied by choosing which global chunk each
// lane fetches.
//
// With WN = 4 (8 waves, 128 int32 accumulators per lane) two waves share
// each SIMD: while one waits to issue its copies the other keeps the MFMA
// pipe busy.  WN = 2 (4 waves, 256 accumulators) maximizes fragment reuse
// instead.
//
// Per k-tile kt (two 32-deep sub-steps with fragments F0/F1):
//   first half:  ds_read F1 of tile kt          under the MFMAs on F0
//   wait until tile kt+1 has landed, barrier    (tile kt is now fully read)
//   second half: copy tile kt+4 into kt's buffer, ds_read F0 of tile kt+1,
//                under the MFMAs on F1
// Each half is hand-ordered so that reads come early and every MFMA is
// preceded by at most one read and one copy.  Requires K % 64 == 0; rows past
// T or N are clamped to the last valid row (they only feed outputs that are
// never stored).
template <int WN, bool WRITE_ACC, int HT>
__global__ __launch_bounds__(128 * WN) void k_gemm_i8_big(GemmArgs a) {
    constexpr int BM = 256, BN = 256, BK = 64, STAGES = 4;
    constexpr int WAVES = 2 * WN, THREADS = 64 * WAVES;
    constexpr int TM = 4, TN = BN / WN / 32;
    constexpr int NF = TM + TN;                      // fragments per sub-step
    constexpr int NM = TM * TN;                      // MFMAs per sub-step
    constexpr int STAGE_BYTES = (BM + BN) * BK;
    constexpr int GPW = 16 / WAVES;                  // 1 KB groups of A (and of B) per wave
    constexpr int LOADS = 2 * GPW;                   // copies per lane per tile
    static_assert(NF <= NM && LOADS <= NM, "interleave needs one MFMA per read and copy");
    // the operand ring, reused after the main loop by the epilogue (outlier
    // stage, then the Y tile)
    constexpr int LDS_BYTES = STAGES * STAGE_BYTES > kYBytes ? STAGES * STAGE_BYTES : kYBytes;
    __shared__ __attribute__((aligned(1024))) int8_t lds[LDS_BYTES];
    __shared__ __attribute__((aligned(16))) float sxs[BM];
    __shared__ int ks_first;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t T = a.T, K = a.K, N = a.N;
    const int64_t MT = ceil_div(T, BM);
    // With the K split (S = 2) the grid holds every tile's first half, then
    // every tile's second half: a unit never waits for another.
    const int S = a.ksplit;
    const int64_t tiles = (int64_t)gridDim.x / S;
    const int half = (int)(blockIdx.x / tiles);
    const int64_t tix = (int64_t)blockIdx.x - half * tiles;
    const int64_t bid = xcd_tile(tix, tiles);
    const int64_t m0 = (bid % MT) * BM;
    const int64_t n0 = (bid / MT) * BN;
    const int wm0 = (wave & 1) * 128;
    const int wn0 = (wave >> 1) * (BN / WN);
    // what the epilogue needs, read now (the main loop hides the latency)
    const float sx_pre = a.sx[m0 + (tid & (BM - 1)) < T ? m0 + (tid & (BM - 1)) : T - 1];
    float sw_pre[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn0 + j * 32 + (lane & 31);
        sw_pre[j] = n < N ? a.sw[n] : 0.0f;
    }
    const int o_pre = a.count[0], opad_pre = a.count[1];

    // copy assignment: wave w fills the 1 KB groups GPW*w .. GPW*w+GPW-1 of A
    // and of B; in a group, lane l writes row 16g + l/4, physical chunk l%4.
    // Copy u < GPW is an A group, u >= GPW a B group.  Addresses are a
    // per-workgroup scalar base plus a 32-bit lane offset (a 256-row panel
    // spans at most 256 * 133136 bytes).
    const int8_t* abase = a.xq + m0 * K;
    const int8_t* bbase = a.wq + n0 * K;
    uint32_t goff[LOADS];
#pragma unroll
    for (int u = 0; u < GPW; ++u) {
        const int row = (wave * GPW + u) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ big_swz(row);
        const int64_t ra = m0 + row < T ? row : T - 1 - m0;
        const int64_t rb = n0 + row < N ? row : N - 1 - n0;
        goff[u] = (uint32_t)(ra * K + c * 16);
        goff[GPW + u] = (uint32_t)(rb * K + c * 16);
    }
    auto copy = [&](int u, int kt, int stage) {
        const bool isa = u < GPW;
        const int8_t* base = (isa ? abase : bbase) + (int64_t)kt * BK;
        const int8_t* dst = lds + stage * STAGE_BYTES + (isa ? 0 : BM * BK) +
                            (wave * GPW + (isa ? u : u - GPW)) * 1024;
        copy_to_lds16(base, goff[u], dst);
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // fragment offsets inside a stage (identical for every stage): fragment
    // q < TM is A tile q, q >= TM is B tile q-TM, for sub-step ss
    int foff[2][NF];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
        const int c = ss * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm0 + i * 32 + (lane & 31);
            foff[ss][i] = row * BK + ((c ^ big_swz(row)) * 16);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn0 + j * 32 + (lane & 31);
            foff[ss][TM + j] = BM * BK + col * BK + ((c ^ big_swz(col)) * 16);
        }
    }
    v4i f0[NF], f1[NF];
    auto mfma = [&](const v4i (&f)[NF], int m) {
        const int i = m / TN, j = m % TN;
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[i], f[TM + j], acc[i][j], 0, 0, 0);
    };

    // Prologue: tiles 0..3 in flight, wait for tile 0, first F0.  Past the
    // last tile, copies re-fetch tile KT-1 into a buffer that is never read
    // again, which keeps the loop free of branches and the wait count fixed.
    // this unit's k-tiles KT0 .. KT-1 (K / BK is even when S = 2)
    const int KT0 = half * (int)(K / BK / S);
    const int KT = KT0 + (int)(K / BK / S);
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int u = 0; u < LOADS; ++u) copy(u, KT0 + st < KT ? KT0 + st : KT - 1, st);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 1)));
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NF; ++q) f0[q] = *reinterpret_cast<const v4i*>(lds + foff[0][q]);

    int s_cur = 0;
    for (int kt = KT0; kt < KT; ++kt) {
        const int s_next = (s_cur + 1) & (STAGES - 1);
        const int8_t* cur = lds + s_cur * STAGE_BYTES;
        const int8_t* nxt = lds + s_next * STAGE_BYTES;
        const int kcopy = kt + STAGES < KT ? kt + STAGES : KT - 1;
        __builtin_amdgcn_s_waitcnt(kLgkm0);   // F0 has arrived
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m < NF) f1[m] = *reinterpret_cast<const v4i*>(cur + foff[1][m]);
            mfma(f0, m);
            __builtin_amdgcn_sched_barrier(0);
        }
        // tile kt+1 has landed (tiles kt+2, kt+3 may still fly) and this
        // wave's F1 reads are complete; after the barrier nobody reads tile kt
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 2)) & ~0xF00);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m < NF) f0[m] = *reinterpret_cast<const v4i*>(nxt + foff[0][m]);
            if (m < LOADS) copy(m, kcopy, s_cur);
            mfma(f1, m);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_cur = s_next;
    }
    // no LDS copy may still be in flight when the LDS is reused or the
    // workgroup retires
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (S > 1) {
        // K split: each half publishes its int32 sums, and the half that
        // finishes second adds the other's (exact, order independent) and
        // runs the epilogue.  The tile counters were zeroed at launch.
        // The sums travel through device-coherent accesses (agent-scope
        // atomic loads and stores: the other half may run on another XCD,
        // whose L2 is not this one's), so no cache flush or invalidate is
        // needed: a half's stores are complete (vmcnt 0) before its counter
        // increment, and the second half reads only after its increment has
        // returned the first's.  A half that finds the other one already
        // done skips publishing its own sums.
        uint64_t* mine = reinterpret_cast<uint64_t*>(a.ks_part) +
                         ((tix * 2 + half) * WAVES + wave) * (TM * TN * 8 * 64);
        const uint64_t* other = reinterpret_cast<const uint64_t*>(a.ks_part) +
                                ((tix * 2 + (1 - half)) * WAVES + wave) * (TM * TN * 8 * 64);
        if (tid == 0)
            ks_first = __hip_atomic_load(&a.ks_count[tix], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const bool other_done = ks_first != 0;
        if (!other_done) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint64_t v = (uint64_t)(uint32_t)acc[i][j][2 * q] |
                                           ((uint64_t)(uint32_t)acc[i][j][2 * q + 1] << 32);
                        __hip_atomic_store(mine + ((i * TN + j) * 8 + q) * 64 + lane, v,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();   // every wave's sums are out (and ks_first is read)
        if (tid == 0)
            ks_first = __hip_atomic_fetch_add(&a.ks_count[tix], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == 0;
        __syncthreads();
        if (ks_first) return;   // the other half finishes the tile
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
    static_assert(THREADS == 512 && BM == 256 && BN == 256 && LDS_BYTES >= kStageBytes,
                  "staged epilogue: 512 threads, 256 x 256 tile");
    epilogue<TM, TN, WRITE_ACC, HT, true>(
        acc, a, m0 + wm0, n0 + wn0, lane,
        StageCtx{lds, tid, m0, n0, sxs, sx_pre, sw_pre, o_pre, opad_pre});
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
    const int64_t bid = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t m0 = (bid % MT) * BM;
    const int64_t n0 = (bid / MT) * BN;
    const int wm0 = (wave % WAVES_M) * WM;
    const int wn0 = (wave / WAVES_M) * WN;

    // copy u of this wave fills 1 KB group g = LOADS * wave + u of the tile
    // (g < GA: rows 8g .. 8g+7 of A, else rows 8(g - GA) .. of B); lane l
    // writes row 8g + l/8 at physical chunk l%8, so it fetches the logical
    // chunk (l%8) ^ stream_swz(row).  32-bit lane offsets (a 128-row panel
    // spans at most 128 * 133144 bytes).
    const int8_t* abase = a.xq + m0 * K;
    const int8_t* bbase = a.wq + n0 * K;
    uint32_t goff[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int g = LOADS * wave + u;
        const bool isa = g < GA;
        const int row = (isa ? g : g - GA) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ stream_swz(row);
        const int64_t r = isa ? (m0 + row < T ? row : T - 1 - m0) : (n0 + row < N ? row : N - 1 - n0);
        goff[u] = (uint32_t)(r * K + c * 16);
    }
    auto copy = [&](int u, int kt, int stage) {
        const int g = LOADS * wave + u;
        const bool isa = g < GA;
        const int8_t* base = (isa ? abase : bbase) + (int64_t)kt * BK;
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
    const int KT = (int)(K / BK);
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
#pragma unroll
        for (int u = 0; u < LOADS; ++u) copy(u, st < KT ? st : KT - 1, st);

    int s_cur = 0;
    for (int kt = 0; kt < KT; ++kt) {
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
    epilogue<TM, TN, WRITE_ACC, HT, false, BN, 64 * NW>(acc, a, m0 + wm0, n0 + wn0, lane,
                                                        StageCtx{lds, tid, m0, n0, nullptr, 0.0f, nullptr, 0, 0});
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int HT>
hipError_t launch_stream(const GemmArgs& a, hipStream_t stream) {
    const int64_t tiles = ceil_div(a.T, BM) * ceil_div(a.N, BN);
    constexpr int threads = 64 * WAVES_M * WAVES_N;
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8_stream<BM, BN, WAVES_M, WAVES_N, STAGES, true, HT>),
                           dim3((unsigned)tiles), dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_gemm_i8_stream<BM, BN, WAVES_M, WAVES_N, STAGES, false, HT>),
                           dim3((unsigned)tiles), dim3(threads), 0, stream, a);
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

__global__ void k_zero_i32(int32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int WN, int HT>
hipError_t launch_big(const GemmArgs& a, hipStream_t stream) {
    if (a.ksplit == 2) {
        // the tile counters start at zero (a kernel rather than a memset, so
        // the call can be captured in a graph); a split matmul is long enough
        // that one more launch does not show
        const int64_t n = ceil_div(a.T, 256) * ceil_div(a.N, 256);
        hipLaunchKernelGGL(k_zero_i32, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream,
                           a.ks_count, n);
    }
    const int64_t tiles = ceil_div(a.T, 256) * ceil_div(a.N, 256) * a.ksplit;
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_i8_big<WN, true, HT>), dim3((unsigned)tiles), dim3(128 * WN), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((k_gemm_i8_big<WN, false, HT>), dim3((unsigned)tiles), dim3(128 * WN), 0,
                           stream, a);
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
    if (a.T > 128 && a.T <= 256 && a.K % 128 == 0 && ceil_div(a.N, 128) <= device_cus() &&
        gemm_ksplit(a.T, a.K, a.N) == 1)
        return launch_stream<256, 128, 4, 1, 3, HT>(a, stream);
    if (a.T > 128 && a.K % 64 == 0) return launch_big<4, HT>(a, stream);
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
int gemm_ksplit(int64_t T, int64_t K, int64_t N) {
    const int64_t kmin = T > 256 ? 8192 : 24576;
    if (!(T > 128 && K % 128 == 0 && K >= kmin)) return 1;
    const int64_t tiles = ceil_div(T, 256) * ceil_div(N, 256);
    const int64_t cus = device_cus();
    const int64_t r1 = ceil_div(tiles, cus);          // rounds of whole tiles
    const int64_t r2 = ceil_div(2 * tiles, cus);      // rounds of half tiles
    return 2 * r2 <= 3 * r1 ? 2 : 1;                  // half-rounds r2/2 <= 3/4 of r1
}

hipError_t launch_gemm(const GemmArgs& a, int ht, hipStream_t stream) {
    if (a.ksplit != 1 && !(a.ksplit == 2 && a.ks_count && a.ks_part && a.T > 128 && a.K % 128 == 0))
        return hipErrorInvalidValue;
    return ht == kHalfBF16 ? launch_gemm_typed<kHalfBF16>(a, stream)
                           : launch_gemm_typed<kHalfF16>(a, stream);
}

}  // namespace i8mm
