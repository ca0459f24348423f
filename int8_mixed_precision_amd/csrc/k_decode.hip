// Single-kernel LLM.int8() matmul for decode shapes (few rows T).
//
// Method (LLM.int8() abstract, taxoreview.com page dblp:280/8696, second
// paragraph): outlier feature dimensions of X are isolated into a 16-bit
// matmul, everything else goes through an Int8 matmul with one absmax
// constant per row of X and per column of W.  Readings as in the rest of the
// library: k is an outlier when |X[t,k]| >= tau in some row; the row scale is
// the absmax over non-outlier columns; q = clamp(rint(x * fp32(127/s))).
//
// At decode sizes the work is a stream of the int8 weight (K*N bytes) past
// a tiny activation, so the kernel is bound by HBM bandwidth; the design
// keeps that stream going from the first instruction to the last:
//   - each wave owns whole 16-row blocks of Wq over all of K (one block per
//     wave at the projection sizes), so the streaming loop has no barrier
//     and no cross-wave reduction; waves drift apart and overlap freely;
//   - every wave first issues the loads of its first 16 KB weight chunk,
//     then its workgroup recomputes the activation side from X
//     (T*K fp16, cache resident): a thread owns whole 8-column chunks across
//     all T rows, so the outlier flags of its columns need no exchange; row
//     absmax by wave shuffles and LDS; ascending outlier indices by a
//     popcount prefix scan; Xq to LDS;
//   - Wq goes from global memory straight into registers as the A operand of
//     v_mfma_i32_16x16x64_i8 (16 weight rows x 64 k), through a ring of three
//     chunks of 16 loads; the B operand (the T activation rows as columns,
//     zero padded) is read from LDS per k-step;
//   - at the end of a block the wave dequantizes its int32 sums, adds the
//     fp16 outlier product in fp32 and rounds Y to fp16 once.
// Limits (host checks them; other shapes use the general kernels):
// T <= 16, K in {4096, 8192}, T*K <= 65536.
#include "common.hpp"

// Quantization must round x * r and any following add separately, exactly
// like the definition; no multiply-add contraction in this file.
#pragma clang fp contract(off)

namespace i8mm {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kRows = 16;              // weight rows per block (MFMA M)
constexpr int kMaxT = 16;
constexpr int kMaxK = 8192;
constexpr int kMaxXK = 65536;          // T*K bytes of Xq kept in LDS
constexpr int kMaxOutliersLds = 256;   // outlier values cached in LDS

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

struct DecodeArgs {
    const uint16_t* x;      // [T,K] fp16 bits
    const int8_t* wq;       // [N,K]
    const float* sw;        // [N]
    const _Float16* w16;    // [K,N]
    _Float16* y;            // [T,N]
    float tau;
    uint32_t tau16;         // bits of the smallest fp16 >= tau (0x7C00 if none finite)
    int T, K, N;
    // optional debug outputs (NULL to skip); workgroup 0 writes all but acc
    int32_t* dbg_count;
    int32_t* dbg_idx;
    int8_t* dbg_xq;
    float* dbg_sx;
    int32_t* dbg_acc;
};

// Xq rows carry a 16-byte pad: the B-operand read has 16 lanes on 16
// different rows, which then fall on distinct banks.
struct Smem {
    int8_t xq[kMaxXK + kMaxT * 16];
    int32_t idx[kMaxK];                        // outlier dims, ascending
    float xo[kMaxT * kMaxOutliersLds];         // X values of the first outliers
    float wmax[kWaves][kMaxT];
    float sx[kMaxT];
    float rx[kMaxT];                           // 127 / s_x (0 when s_x = 0)
    int32_t wtot[kWaves * 2];
};

// Packed unsigned max of two pairs of 16-bit lanes.
__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    const uint32_t lo = (a & 0xFFFFu) > (b & 0xFFFFu) ? (a & 0xFFFFu) : (b & 0xFFFFu);
    const uint32_t hi = (a >> 16) > (b >> 16) ? (a >> 16) : (b >> 16);
    return lo | (hi << 16);
}

__device__ inline float chunk_val(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return h2f((uint16_t)(w >> ((e & 1) * 16)));
}

constexpr int kLoads = 16;                    // 16-byte loads per lane per chunk (16 KB/wave)
constexpr int kChunkK = kLoads * 64;          // k covered by one chunk


// CPB = K / 1024 chunks per 16-row block; a thread owns CPT = K / 4096
// chunks of 8 columns (c = tid + 512 j) in the activation prologue, for all
// T <= TMAX = 64 / CPB rows (so T * CPT <= 16 chunks of X per thread).
template <int CPB>
__global__ __launch_bounds__(kThreads) void k_decode(DecodeArgs a) {
    constexpr int CPT = CPB / 4;
    constexpr int TMAX = 64 / CPB;
    __shared__ __attribute__((aligned(16))) Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int T = a.T, K = a.K, N = a.N;
    const int ldx = K + 16;                    // LDS row stride of Xq
    const int nblocks = (N + kRows - 1) / kRows;
    const int gwave = blockIdx.x * kWaves + wave;   // this wave's blocks: gwave, +nwaves, ...
    const int nwaves = gridDim.x * kWaves;

    // Load i of chunk c of block blk: lane l holds weight row blk*16 + l%16
    // and bytes c*1024 + 64 i + 16*(l/16) .. +16.
    const int kl = (lane >> 4) * 16;
    // Rows past N re-read row N-1 (their outputs are never stored); loads
    // are unconditional so the wait counts stay exact.
    auto issue = [&](int blk, int c, v4i (&buf)[kLoads]) {
        const int n = blk * kRows + (lane & 15);
        const int8_t* p = a.wq + (int64_t)(n < N ? n : N - 1) * K + c * kChunkK + kl;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) buf[i] = *reinterpret_cast<const v4i*>(p + i * 64);
    };

    // The prologue's X loads go out first and their first use (the column
    // maxima) comes before any weight load is issued: vector-memory counters
    // retire in order, so a later wait on X would also wait for weight data.
    // Rows t >= T re-read row T-1: a repeated row changes neither the
    // column maxima nor anything used later (rows >= T of Xq and xo are never
    // read), and unconditional loads keep the wait counts exact.
    uint4 xr[CPT][TMAX];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            xr[j][t] = *reinterpret_cast<const uint4*>(a.x + (int64_t)(t < T ? t : T - 1) * K +
                                                       (tid + kThreads * j) * 8);
    // Magnitudes as fp16 bit patterns: for non-negative halves the unsigned
    // order is the numeric order, so |x| >= tau <=> bits(|x|) >= tau16, with
    // tau16 the bits of the smallest fp16 >= tau (0x7C00 when none is finite).
    // Column maxima over the T rows by packed unsigned 16-bit max.
    uint32_t fm[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            const uint32_t w[4] = {xr[j][t].x, xr[j][t].y, xr[j][t].z, xr[j][t].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], w[d] & 0x7FFF7FFFu);
        }
        fm[j] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            fm[j] |= (((cm[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) >= a.tau16 ? 1u : 0u) << e;
    }
    // the flags must be final (so X has arrived) before the first weight
    // load is issued: an empty asm that consumes them and orders memory
#pragma unroll
    for (int j = 0; j < CPT; ++j) asm volatile("" ::"v"(fm[j]) : "memory");
    // Ring loads are unconditional (a wave without a block re-reads the
    // clamped last row; nothing uses it) so the wait analysis sees one path.
    v4i ring[3][kLoads];
    int blk = gwave;
    issue(blk, 0, ring[0]);

    // ---- activation side, recomputed per workgroup, from registers.
    // Row absmax over the non-outlier columns: mask the outlier halves, then
    // a packed max tree, one conversion to float per row.
    float rmax[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t w[4] = {xr[j][t].x, xr[j][t].y, xr[j][t].z, xr[j][t].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t keep = (((fm[j] >> (2 * d)) & 1u) ? 0u : 0x0000FFFFu) |
                                      (((fm[j] >> (2 * d + 1)) & 1u) ? 0u : 0xFFFF0000u);
                m = pk_max_u16(m, w[d] & 0x7FFF7FFFu & keep);
            }
        }
        const uint32_t mh = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
        rmax[t] = h2f((uint16_t)mh);
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
            float v = rmax[t];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, d));
            if (lane == 0) sm.wmax[wave][t] = v;
        }
    }
    // positions of the outliers: prefix count over the chunk order
    int pc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int cnt = __builtin_popcount(fm[j]);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == 63) sm.wtot[j * kWaves + wave] = incl;
        pc[j] = incl - cnt;
    }
    __syncthreads();
    if (tid < T) {
        float v = sm.wmax[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v = __builtin_fmaxf(v, sm.wmax[w][tid]);
        sm.sx[tid] = v;
    }
    int o = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        int before = o;
        for (int w = 0; w < kWaves; ++w) {
            const int tot = sm.wtot[j * kWaves + w];
            if (w < wave) before += tot;
            o += tot;
        }
        pc[j] += before;
    }
    __syncthreads();   // sx ready
    if (tid < T) {
        const float sxt = sm.sx[tid];
        sm.rx[tid] = sxt > 0.0f ? 127.0f / sxt : 0.0f;   // IEEE fp32 divide
    }
    __syncthreads();   // rx ready
    // Quantize the owned columns into LDS and gather the outliers.
    // q = rint(x * r) by the 1.5 * 2^23 addition: for |p| < 2^22, p + 1.5*2^23
    // rounds p to the nearest integer (ties to even) and the low byte of the
    // result's bit pattern is that integer as int8.  |x| <= s_x makes
    // |p| <= 127 * (1 + 2^-23), so q is within [-127, 127] without a clamp.
    // The multiply and the add stay separate roundings (no contraction).
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kThreads * j;
        // byte mask that zeroes the outlier columns of the chunk
        uint32_t keep[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            keep[h] = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                keep[h] |= ((fm[j] >> (4 * h + e)) & 1u) ? 0u : (0xFFu << (8 * e));
        }
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            {
                const float rr = t < T ? sm.rx[t] : 0.0f;
                uint32_t packed[2] = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __fmul_rn(chunk_val(xr[j][t], e), rr);
                    const uint32_t bits = __builtin_bit_cast(uint32_t, __fadd_rn(p, 12582912.0f));
                    packed[e >> 2] |= (bits & 0xFFu) << ((e & 3) * 8);
                }
                packed[0] &= keep[0];
                packed[1] &= keep[1];
                *reinterpret_cast<uint2*>(&sm.xq[t * ldx + c * 8]) = make_uint2(packed[0], packed[1]);
                if (blockIdx.x == 0 && a.dbg_xq && t < T)
                    *reinterpret_cast<uint2*>(a.dbg_xq + (int64_t)t * K + c * 8) =
                        make_uint2(packed[0], packed[1]);
                if (fm[j]) {
                    int pos = pc[j];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if ((fm[j] >> e) & 1u) {
                            if (pos < kMaxOutliersLds)
                                sm.xo[t * kMaxOutliersLds + pos] = chunk_val(xr[j][t], e);
                            ++pos;
                        }
                    }
                }
            }
        }
        if (fm[j]) {
            int pos = pc[j];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if ((fm[j] >> e) & 1u) {
                    sm.idx[pos] = c * 8 + e;
                    if (blockIdx.x == 0 && a.dbg_idx) a.dbg_idx[pos] = c * 8 + e;
                    ++pos;
                }
            }
        }
    }
    if (blockIdx.x == 0 && tid == 0 && a.dbg_count) a.dbg_count[0] = o;
    if (blockIdx.x == 0 && a.dbg_sx && tid < T) a.dbg_sx[tid] = sm.sx[tid];
    issue(blk, 1, ring[1]);
    issue(blk, 2, ring[2]);
    __syncthreads();   // Xq, idx, xo ready

    // ---- stream this wave's blocks.  Per block the chunk loop is fully
    // unrolled with a compile-time ring slot, so the wait before each chunk
    // leaves the two younger chunks in flight; the next block's first chunks
    // go out after the epilogue (at the projection sizes a wave has exactly
    // one block).
    const int tcol = lane & 15;                         // B column = activation row t
    const int8_t* xrow = &sm.xq[(tcol < T ? tcol : 0) * ldx + kl];
    auto process_block = [&](int b) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            v4i(&buf)[kLoads] = ring[c % 3];
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const v4i xb = tcol < T ? *reinterpret_cast<const v4i*>(xrow + c * kChunkK + i * 64)
                                        : v4i{0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(buf[i], xb, acc, 0, 0, 0);
            }
            if (c + 3 < CPB) issue(b, c + 3, buf);
        }
        // 16x16 accumulator layout: lane holds column lane%16 (t) and, in
        // register v, row 4*(lane/16) + v of the block
        if (tcol < T) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = b * kRows + 4 * (lane >> 4) + v;
                if (n < N) {
                    if (a.dbg_acc) a.dbg_acc[(int64_t)tcol * N + n] = acc[v];
                    float y = (float)acc[v] * sm.sx[tcol] * (a.sw[n] * (1.0f / 16129.0f));
                    for (int jj = 0; jj < o; ++jj) {
                        const int k = sm.idx[jj];
                        const float xv = jj < kMaxOutliersLds ? sm.xo[tcol * kMaxOutliersLds + jj]
                                                              : h2f(a.x[(int64_t)tcol * K + k]);
                        y += xv * (float)a.w16[(int64_t)k * N + n];
                    }
                    a.y[(int64_t)tcol * N + n] = (_Float16)y;
                }
            }
        }
    };
    // first block in straight-line code (at the projection sizes the only one)
    if (blk < nblocks) process_block(blk);
    for (blk += nwaves; blk < nblocks; blk += nwaves) {
        issue(blk, 0, ring[0]);
        issue(blk, 1, ring[1]);
        issue(blk, 2, ring[2]);
        process_block(blk);
    }
}

}  // namespace

// Bits of the smallest binary16 value >= tau (tau >= 0 and not NaN), or
// 0x7C00 (+inf) when no finite binary16 value reaches tau.  Found by a binary
// search over the non-negative bit patterns, whose unsigned order is the
// numeric order; the fp16 -> fp32 conversion is exact.
static uint32_t tau_to_f16_ceil(float tau) {
    uint32_t lo = 0, hi = 0x7C00;   // answer in [lo, hi]
    while (lo < hi) {
        const uint32_t mid = (lo + hi) / 2;
        if ((float)__builtin_bit_cast(_Float16, (uint16_t)mid) >= tau) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

bool decode_path_supported(int64_t T, int64_t K, int64_t N) {
    (void)N;
    return T >= 1 && T <= kMaxT && (K == 4096 || K == 8192) && T * K <= kMaxXK;
}

hipError_t launch_decode(const _Float16* X, int64_t T, int64_t K, const int8_t* Wq,
                         const float* sw, const _Float16* W16, int64_t N, float tau,
                         _Float16* Y, int32_t* dbg_count, int32_t* dbg_idx, int8_t* dbg_xq,
                         float* dbg_sx, int32_t* dbg_acc, hipStream_t stream) {
    DecodeArgs a{reinterpret_cast<const uint16_t*>(X), Wq, sw, W16, Y, tau, tau_to_f16_ceil(tau),
                 (int)T, (int)K, (int)N, dbg_count, dbg_idx, dbg_xq, dbg_sx, dbg_acc};
    const int64_t nblocks = ceil_div(N, kRows);
    const unsigned grid = (unsigned)ceil_div(nblocks, kWaves);   // one 16-row block per wave
    if (K == 4096)
        hipLaunchKernelGGL(k_decode<4>, dim3(grid), dim3(kThreads), 0, stream, a);
    else if (K == 8192)
        hipLaunchKernelGGL(k_decode<8>, dim3(grid), dim3(kThreads), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace i8mm
