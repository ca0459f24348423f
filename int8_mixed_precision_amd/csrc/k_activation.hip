// Activation side of LLM.int8(): outlier-dimension detection, isolation
// (compaction of the outlier indices) and vector-wise (row-wise) int8
// quantization of the remaining activations.
//
// Method: LLM.int8() abstract (taxoreview.com page dblp:280/8696, second
// paragraph) - outlier feature dimensions are isolated and everything else is
// quantized with one normalization constant per inner product, i.e. per row
// of X; "LLM.int8(): A Procedure for Int8 Matrix Multiplication in
// Transformer Language Models" (summarizepaper.com), bullet summary -
// outliers are picked by magnitude.
//
// Readings of the pages: k is an outlier when |X[t,k]| >= tau in some row;
// the row scale is the absmax over non-outlier columns;
// q = clamp(rint(x * fp32(127 / s)), -127, 127) with an IEEE fp32 divide
// (with an unbounded exponent: see qfactor in common.hpp).
//
// The kernels stream X with 16-byte loads (8 halves per lane) and are bound
// by HBM bandwidth; the X re-read of the quantize pass is served from cache
// for the row a workgroup is working on.
#include "common.hpp"

#include <algorithm>



// Quantization must round x * r and any following add separately, exactly
// like the definition; no multiply-add contraction in this file.
#pragma clang fp contract(off)

namespace i8mm {

namespace {

constexpr int kCompactThreads = 1024;
constexpr int kQuantThreads = 256;
constexpr int kRowThreads = 512;            // k_rowquant_cached

// Outlier flags for up to kOwnedMaxT rows without atomics: a workgroup owns
// kOwnedCols columns (8 per lane, whole 32-bit words per 4 lanes) and reads
// every row of them, its kOwnedWaves waves taking rows 16 at a time (rows
// past T re-read row T-1, so all 16 loads of a batch are in flight
// together); the waves' flags are merged through LDS and every word of the
// bitmap is stored, so no clearing kernel has to run first.
// Whole calls against the clearing kernel + atomic detection: T=17-64 on
// K=8192, N=28672 up to 2.9 us faster, T=128 0.9 us; 129-256 rows within
// +-1 us either way, so they keep the other path.
constexpr int kOwnedCols = 512;
constexpr int kOwnedWaves = 16;
constexpr int kOwnedMaxT = 128;
template <int HT>
__global__ __launch_bounds__(kOwnedWaves * kWave) void k_detect_owned(const uint16_t* __restrict__ X,
                                                                      int64_t T, int64_t K, float tau,
                                                                      uint32_t* __restrict__ flags) {
    __shared__ uint32_t wfm[kOwnedWaves][kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * kOwnedCols + lane * 8;
    const bool in = c0 < K;
    const uint16_t* xc = X + (in ? c0 : 0);
    uint32_t m = 0;
    for (int64_t t0 = wv * 16; t0 < T; t0 += 16 * kOwnedWaves) {
        uint4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t t = t0 + u < T ? t0 + u : T - 1;
            v[u] = *reinterpret_cast<const uint4*>(xc + t * K);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
                m |= (__builtin_fabsf(x) >= tau ? 1u : 0u) << e;
            }
        }
    }
    wfm[wv][lane] = in ? m : 0u;   // lanes past K (which read column 0) flag nothing
    __syncthreads();
    if (wv == 0) {
        uint32_t f = 0;
#pragma unroll
        for (int w = 0; w < kOwnedWaves; ++w) f |= wfm[w][lane];
        uint32_t word = f << ((lane & 3) * 8);
        word |= __shfl_xor(word, 1);
        word |= __shfl_xor(word, 2);
        if ((lane & 3) == 0 && in) flags[c0 >> 5] = word;
    }
}

// Outlier flags for any number of rows without atomics or a clearing
// kernel: a workgroup owns kColBlock = 64 columns (two bitmap words) of one
// group of rows (blockIdx.y; gridDim.y groups of consecutive rows) and
// stores the flags of its rows whole into that group's partial bitmap
// (flags + group * kwp words); the consumers OR the partial bitmaps.  The
// row groups give the launch enough workgroups to fill the chip (one group:
// K / 64 = 192 workgroups at K = 12288).  A row's 64 columns are one
// 128-byte line, and a wave's load instruction covers 8 rows (8 lanes per
// row, 16 bytes each), so every request is a whole line; each lane keeps
// kColLoads rows' loads in flight.  The lanes holding one column group
// merge their flags by shuffles, the waves through LDS.
// Columns per workgroup: 64 (a 128-byte line per row) up to K = 16384,
// 256 (512 bytes per row) above: a longer piece of each row per DRAM page
// opened (rows are 2K bytes apart); whole calls, down projection T=2048,
// K=49152 -0.5%, up projection (K=12288) +0.2% with 256.
constexpr int kColBlockShort = 64;
constexpr int kColBlockLong = 256;
constexpr int kColWaves = 8;
constexpr int kColLoads = 8;
constexpr int kColRowsPerPass = 8 * kColWaves * kColLoads;   // 512 (row groups)
template <int HT, int CB>
__global__ __launch_bounds__(kColWaves * kWave) void k_detect_cols(const uint16_t* __restrict__ X,
                                                                   int64_t T, int64_t K, float tau,
                                                                   uint32_t* __restrict__ flags,
                                                                   int64_t kwp, int32_t* __restrict__ zero,
                                                                   int64_t nzero) {
    constexpr int LPR = CB / 8;                        // lanes per row
    constexpr int RPL = kWave / LPR;                   // rows per wave load
    constexpr int RPP = RPL * kColWaves * kColLoads;   // rows per pass
    static_assert(CB % 32 == 0 && kWave % LPR == 0, "whole bitmap words, whole rows per wave");
    __shared__ uint32_t wfm[kColWaves][LPR];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int64_t i = tid; i < nzero; i += kColWaves * kWave) zero[i] = 0;
    const int cg = lane % LPR;                         // 8-column group of the lane
    const int64_t c0 = (int64_t)blockIdx.x * CB + cg * 8;
    const bool in = c0 < K;
    const uint16_t* xc = X + (in ? c0 : 0);
    // rows r0 .. r1-1 of this group
    const int64_t per = ceil_div(T, (int64_t)gridDim.y);
    const int64_t r0 = (int64_t)blockIdx.y * per;
    const int64_t r1 = r0 + per < T ? r0 + per : T;
    uint32_t m = 0;
    for (int64_t t0 = r0 + lane / LPR + RPL * wv; t0 < r1; t0 += RPP) {
        uint4 v[kColLoads];
#pragma unroll
        for (int u = 0; u < kColLoads; ++u) {
            const int64_t t = t0 + (int64_t)u * RPL * kColWaves;
            v[u] = *reinterpret_cast<const uint4*>(xc + (t < r1 ? t : r1 - 1) * K);
        }
#pragma unroll
        for (int u = 0; u < kColLoads; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
                m |= (__builtin_fabsf(x) >= tau ? 1u : 0u) << e;
            }
        }
    }
    // rows past the group re-read its last row (no flag changes); lanes past
    // K flag nothing
    if (!in) m = 0;
#pragma unroll
    for (int d = LPR; d < kWave; d <<= 1) m |= __shfl_xor(m, d);
    if (lane < LPR) wfm[wv][lane] = m;
    __syncthreads();
    if (wv == 0 && lane < LPR) {
        uint32_t f = 0;
#pragma unroll
        for (int w = 0; w < kColWaves; ++w) f |= wfm[w][lane];
        uint32_t word = f << ((lane & 3) * 8);
        word |= __shfl_xor(word, 1);
        word |= __shfl_xor(word, 2);
        if ((lane & 3) == 0 && in) flags[(int64_t)blockIdx.y * kwp + (c0 >> 5)] = word;
    }
}

// Isolation of the outlier dimensions: one workgroup turns the bitmap into
// the ascending index list idx[0..o), per-word prefix counts and o.
// Popcounts are scanned across the workgroup (wave prefix by shuffles, wave
// totals through LDS).
__global__ __launch_bounds__(kCompactThreads) void k_compact(const uint32_t* __restrict__ flags,
                                                             int64_t kw,
                                                             int32_t* __restrict__ wprefix,
                                                             int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ count) {
    __shared__ int wave_tot[kCompactThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const int64_t per = (kw + kCompactThreads - 1) / kCompactThreads;
    const int64_t w0 = tid * per;
    const int64_t w1 = w0 + per < kw ? w0 + per : kw;
    int local = 0;
    for (int64_t w = w0; w < w1; ++w) local += __builtin_popcount(flags[w]);
    // inclusive scan inside the wave
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wave_tot[i];
    int run = before + incl - local;   // exclusive prefix of this thread
    for (int64_t w = w0; w < w1; ++w) {
        wprefix[w] = run;
        uint32_t f = flags[w];
        while (f) {
            int b = __builtin_ctz(f);
            idx[run++] = (int32_t)(w * 32 + b);
            f &= f - 1u;
        }
    }
    if (tid == kCompactThreads - 1) {
        count[0] = run;
        count[1] = (run + 15) & ~15;
    }
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, d));
    return v;
}

__device__ inline int8_t quant(float x, float r) {
    float q = __builtin_rintf(x * r);
    q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
    return (int8_t)(int)q;
}

// Row-wise quantization of one row t per workgroup, over the non-outlier
// columns, plus the gather of the row's outlier values (16-bit patterns,
// unchanged) into xo.
template <int HT>
__global__ __launch_bounds__(kQuantThreads) void k_rowquant(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ flags,
    const int32_t* __restrict__ wprefix, const int32_t* __restrict__ count,
    int8_t* __restrict__ xq, float* __restrict__ sx, uint16_t* __restrict__ xo) {
    __shared__ float red[kQuantThreads / kWave];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const uint16_t* row = X + t * K;
    const int64_t nch = K / 8;
    float mx = 0.0f;
    for (int64_t c = tid; c < nch; c += kQuantThreads) {
        uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
        uint32_t fm = (flags[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = __builtin_fabsf(h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
            mx = ((fm >> e) & 1u) ? mx : __builtin_fmaxf(mx, a);
        }
    }
    mx = wave_max(mx);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / kWave; ++i) mx = __builtin_fmaxf(mx, red[i]);
    const float qk = HT == kHalfF16 ? 1.0f : qfactor(mx);   // fp16 scales are >= 2^-24
    const float r = mx > 0.0f ? 127.0f / (mx * qk) : 0.0f;
    const int64_t opad = count[1];
    const int64_t o = count[0];
    uint16_t* xo_row = xo + t * opad;
    for (int64_t c = tid; c < nch; c += kQuantThreads) {
        uint4 v = *reinterpret_cast<const uint4*>(row + c * 8);
        const uint32_t word = flags[c >> 2];
        uint32_t fm = (word >> ((c & 3) * 8)) & 0xFFu;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t hb = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
            float x = h16_to_f32<HT>(hb);
            uint32_t q = ((fm >> e) & 1u) ? 0u : (uint32_t)(uint8_t)quant(x * qk, r);
            packed[e >> 2] |= q << ((e & 3) * 8);
        }
        *reinterpret_cast<uint2*>(xq + blk_offset(t, c * 8, T, K)) = make_uint2(packed[0], packed[1]);
        if (fm) {
            const int base_bit = (int)(c & 3) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if ((fm >> e) & 1u) {
                    int bit = base_bit + e;
                    int pos = wprefix[c >> 2] + __builtin_popcount(word & ((1u << bit) - 1u));
                    xo_row[pos] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
    for (int64_t j = o + tid; j < opad; j += kQuantThreads) xo_row[j] = 0;   // +0 in both types
    if (tid == 0) sx[t] = mx;
}

// Exclusive prefix sum over the workgroup (wave scan by shuffles, wave
// totals through LDS); total receives the workgroup's sum.
template <int NT = kQuantThreads>
__device__ inline int block_excl_scan(int v, int* wtot, int& total) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
    }
    if (lane == kWave - 1) wtot[wv] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        before += w < wv ? wtot[w] : 0;
        total += wtot[w];
    }
    return before + incl - v;
}

// k_rowquant for rows of at most kQuantThreads * kRowCache * 8 values: the
// row is read from HBM once into registers (one pass instead of two), the
// outlier bitmap once into LDS, and every load is issued before the first
// use (chunks past the row re-read chunk 0; nothing uses them).  It also
// isolates the outlier dimensions itself: every workgroup scans the bitmap
// words it holds in LDS for their prefix counts (a few words per lane), and
// workgroup 0 writes the ascending index list and the count, so no separate
// compaction kernel runs.
// kRowCache = 16-byte chunks per thread, NT threads: K <= 16384 (4 x 512)
// or K <= 49152 (12 x 512).  Fewer chunks per thread and more threads per
// row than 8 x 256 and 24 x 256 raised the occupancy: K = 49152, T = 2048
// activation pass 124 -> 103 us; T = 4096 264 -> 222 us; K = 8192, T = 256
// 11.1 -> 10.1 us; K = 12288 within 2% either way (6 x 1024 and 8 x 768
// were no faster than 24 x 256).
template <int HT, int kRowCache, int NT>
__global__ __launch_bounds__(NT) void k_rowquant_cached(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ flags,
    int32_t* __restrict__ idx, int32_t* __restrict__ count,
    int8_t* __restrict__ xq, float* __restrict__ sx, uint16_t* __restrict__ xo) {
    constexpr int KW = NT * kRowCache / 4;                  // bitmap words held
    constexpr int WPT = (KW + NT - 1) / NT;      // words per lane
    __shared__ float red[NT / kWave];
    __shared__ uint32_t fl[KW];
    __shared__ int pf[KW];
    __shared__ int wtot[NT / kWave];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const uint16_t* row = X + t * K;
    const int nch = (int)(K / 8);
    uint4 v[kRowCache];
#pragma unroll
    for (int i = 0; i < kRowCache; ++i) {
        const int c = tid + NT * i;
        v[i] = *reinterpret_cast<const uint4*>(row + (c < nch ? c : 0) * 8);
    }
    const int kw = (nch + 3) / 4;
    for (int w = tid; w < kw; w += NT) fl[w] = flags[w];
    __syncthreads();
    // outliers before each word: lane l takes words WPT l .. WPT l + WPT - 1
    int o = 0;
    {
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) cnt += __builtin_popcount(fl[w]);
        }
        int run = block_excl_scan<NT>(cnt, wtot, o);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) {
                pf[w] = run;
                uint32_t f = fl[w];
                if (blockIdx.x == 0) {
                    int p = run;
                    while (f) {
                        idx[p++] = w * 32 + __builtin_ctz(f);
                        f &= f - 1u;
                    }
                }
                run += __builtin_popcount(fl[w]);
            }
        }
    }
    const int opad = (o + 15) & ~15;
    if (blockIdx.x == 0 && tid == 0) {
        count[0] = o;
        count[1] = opad;
    }
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowCache; ++i) {
        const int c = tid + NT * i;
        if (c < nch) {
            const uint32_t fm = (fl[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = __builtin_fabsf(h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
                mx = ((fm >> e) & 1u) ? mx : __builtin_fmaxf(mx, a);
            }
        }
    }
    mx = wave_max(mx);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = mx;
    __syncthreads();   // red, and the word prefixes pf
    mx = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) mx = __builtin_fmaxf(mx, red[i]);
    const float qk = HT == kHalfF16 ? 1.0f : qfactor(mx);   // fp16 scales are >= 2^-24
    const float r = mx > 0.0f ? 127.0f / (mx * qk) : 0.0f;
    uint16_t* xo_row = xo + t * opad;
#pragma unroll
    for (int i = 0; i < kRowCache; ++i) {
        const int c = tid + NT * i;
        if (c >= nch) continue;
        const uint32_t word = fl[c >> 2];
        const uint32_t fm = (word >> ((c & 3) * 8)) & 0xFFu;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
            const uint32_t q = ((fm >> e) & 1u) ? 0u : (uint32_t)(uint8_t)quant(x * qk, r);
            packed[e >> 2] |= q << ((e & 3) * 8);
        }
        *reinterpret_cast<uint2*>(xq + blk_offset(t, (int64_t)c * 8, T, K)) = make_uint2(packed[0], packed[1]);
        if (fm) {
            const int base_bit = (c & 3) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if ((fm >> e) & 1u) {
                    const int bit = base_bit + e;
                    const int pos = pf[c >> 2] + __builtin_popcount(word & ((1u << bit) - 1u));
                    xo_row[pos] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
    for (int j = o + tid; j < opad; j += NT) xo_row[j] = 0;   // +0 in both types
    if (tid == 0) sx[t] = mx;
}

// Row-wise quantization with each row held in registers, for many rows
// (T > kOwnedMaxT) of up to kRegMaxK values.  A workgroup of kRQWaves waves
// takes kRQWaves / WR rows, WR waves per row, each lane CH 16-byte chunks of
// it (chunk c = 64 (i WR + w) + lane for wave w of the row, so each load
// instruction reads one contiguous kilobyte).  With one wave per row the row
// maximum needs no barrier at all, and a compute unit holds a dozen rows in
// flight.
//   - The detection's partial bitmaps are loaded first (small and cached),
//     then the row, so waiting for the bitmap leaves the row in flight; the
//     workgroup ORs the partials into LDS and scans the words' popcounts for
//     the outliers' positions (workgroup 0 also writes the ascending index
//     list and the count).
//   - Row maximum over the non-outlier columns on the 16-bit patterns of |x|
//     (for non-negative halves the unsigned order is the numeric order) by
//     packed unsigned max, outlier halves masked to zero in the few chunks
//     that hold one; one conversion to float per lane.
//   - q = rint(x * r) as fp32(x * r) (one rounding) + 1.5 * 2^23 (rounds to
//     the nearest integer, ties to even): the low byte of the sum's bit
//     pattern is q as int8.  |x| <= s_x in a non-outlier column keeps
//     |x * r| <= 127 (1 + 2^-23), so q lies in [-127, 127] without a clamp;
//     outlier columns are zeroed afterwards by a byte mask.
constexpr int kDetectGroups = kDetectParts;  // partial bitmaps of the detection
constexpr int64_t kRegMaxK = 49152;          // longest row held in registers

template <int HT, int NW, int WR, int CH>
__global__ __launch_bounds__(NW * kWave) void k_rowquant_regs(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ parts,
    int nparts, int64_t kwp, int32_t* __restrict__ idx, int32_t* __restrict__ count,
    int8_t* __restrict__ xq, float* __restrict__ sx, uint16_t* __restrict__ xo) {
    constexpr int kRQThreads = NW * kWave;
    constexpr int RPW = NW / WR;                        // rows per workgroup
    constexpr int KW = WR * CH * 64 * 8 / 32;          // bitmap words of the longest row
    constexpr int WPT = (KW + kRQThreads - 1) / kRQThreads;
    static_assert(NW % WR == 0, "whole rows per workgroup");
    __shared__ uint32_t fl[KW];
    __shared__ int pf[KW];
    __shared__ int wtot[NW];
    __shared__ float wmx[NW];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WR;
    const int64_t t = (int64_t)blockIdx.x * RPW + wave / WR;
    const bool live = t < T;                            // uniform over the wave
    const int nch = (int)(K / 8);
    const int kw = (int)((K + 31) / 32);

    // partial bitmaps, then the row (rows past T read row 0; nothing uses it)
    uint32_t fr[WPT][kDetectGroups];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int w = tid + kRQThreads * j;
#pragma unroll
        for (int r = 0; r < kDetectGroups; ++r)
            fr[j][r] = (w < kw && r < nparts) ? parts[(int64_t)r * kwp + w] : 0u;
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* row = X + (live ? t : 0) * K;
    uint4 v[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = (i * WR + wr) * kWave + lane;
        v[i] = *reinterpret_cast<const uint4*>(row + (int64_t)(c < nch ? c : 0) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int w = tid + kRQThreads * j;
        uint32_t f = 0;
#pragma unroll
        for (int r = 0; r < kDetectGroups; ++r) f |= fr[j][r];
        if (w < kw) fl[w] = f;
    }
    __syncthreads();   // fl
    // outliers before each word: thread l scans words WPT l .. WPT l + WPT - 1
    int o = 0;
    {
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) cnt += __builtin_popcount(fl[w]);
        }
        int run = block_excl_scan<kRQThreads>(cnt, wtot, o);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) {
                pf[w] = run;
                uint32_t f = fl[w];
                if (blockIdx.x == 0) {
                    int p = run;
                    while (f) {
                        idx[p++] = w * 32 + __builtin_ctz(f);
                        f &= f - 1u;
                    }
                }
                run += __builtin_popcount(fl[w]);
            }
        }
    }
    const int opad = (o + 15) & ~15;
    if (blockIdx.x == 0 && tid == 0) {
        count[0] = o;
        count[1] = opad;
    }
    // row maximum over the non-outlier columns
    uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = (i * WR + wr) * kWave + lane;
        if (c < nch) {
            const uint32_t fm = (fl[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            uint32_t keep[4] = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
            if (fm) {
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    keep[d] = (((fm >> (2 * d)) & 1u) ? 0u : 0x00007FFFu) |
                              (((fm >> (2 * d + 1)) & 1u) ? 0u : 0x7FFF0000u);
            }
            m0 = pk_max_u16(m0, pk_max_u16(w[0] & keep[0], w[1] & keep[1]));
            m1 = pk_max_u16(m1, pk_max_u16(w[2] & keep[2], w[3] & keep[3]));
        }
    }
    const uint32_t m = pk_max_u16(m0, m1);
    const uint32_t mh = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
    float mx = wave_max(h16_to_f32<HT>((uint16_t)mh));
    if constexpr (WR > 1) {
        if (lane == 0) wmx[wave] = mx;
    }
    __syncthreads();   // pf (and, several waves per row, the waves' maxima)
    if constexpr (WR > 1) {
        const int w0 = wave - wr;
        mx = wmx[w0];
#pragma unroll
        for (int q = 1; q < WR; ++q) mx = __builtin_fmaxf(mx, wmx[w0 + q]);
    }
    if (!live) return;
    const float qk = HT == kHalfF16 ? 1.0f : qfactor(mx);   // fp16 scales are >= 2^-24
    const float rr = mx > 0.0f ? 127.0f / (mx * qk) : 0.0f;   // IEEE fp32 divide
    uint16_t* xo_row = xo + t * opad;
    // Xq addresses: with every k-tile 64 wide (K % 64 == 0) chunk i of the
    // lane is q0 + i * qstep in the panel-blocked layout (lane l holds bytes
    // 8 (l % 8) of k-tile 8 (i WR + w) + l / 8), else blk_offset
    const bool whole_tiles = K % kKTile == 0;
    const int64_t p0 = t - t % kPanel;
    const int64_t prow = T - p0 < kPanel ? T - p0 : kPanel;
    const int64_t qstep = 8 * WR * kKTile * prow;
    const int64_t q0 = p0 * K + (t - p0) * kKTile + 8 * (lane & 7) +
                       (int64_t)(8 * wr + (lane >> 3)) * kKTile * prow;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = (i * WR + wr) * kWave + lane;
        if (c >= nch) continue;
        const uint32_t word = fl[c >> 2];
        const uint32_t fm = (word >> ((c & 3) * 8)) & 0xFFu;
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
            const float p = __builtin_fmaf(x * qk, rr, 0.0f);
            f[e] = __builtin_bit_cast(uint32_t, __fadd_rn(p, 12582912.0f));
        }
        uint32_t packed[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t lo = __builtin_amdgcn_perm(f[4 * h + 1], f[4 * h], 0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm(f[4 * h + 3], f[4 * h + 2], 0x0c0c0400u);
            packed[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        if (fm) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t keep = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    keep |= ((fm >> (4 * h + e)) & 1u) ? 0u : (0xFFu << (8 * e));
                packed[h] &= keep;
            }
            const int base_bit = (c & 3) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if ((fm >> e) & 1u) {
                    const int bit = base_bit + e;
                    const int pos = pf[c >> 2] + __builtin_popcount(word & ((1u << bit) - 1u));
                    xo_row[pos] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
        const int64_t qo = whole_tiles ? q0 + i * qstep : blk_offset(t, (int64_t)c * 8, T, K);
        *reinterpret_cast<uint2*>(xq + qo) = make_uint2(packed[0], packed[1]);
    }
    for (int j = o + wr * kWave + lane; j < opad; j += WR * kWave) xo_row[j] = 0;   // +0 in both types
    if (wr == 0 && lane == 0) sx[t] = mx;
}

// Rows of more than 32768 values and at most kStreamMaxT rows go to
// k_rowquant_stream below.  Activation pass (detection + quantization),
// against k_rowquant_regs<16, 8, 12>, one run: K=49152 with T=2048 and 625
// outlier dims (Laplace rows) 123.1 -> 98.0 us, 9 dims 96.2 -> 84.5 us;
// T=1024, K=40016 48.5 -> 41.0 us; T=700 46.2 -> 36.0 us; T=129 15.5 ->
// 14.0 us; T=300, K=36864 19.4 -> 20.3 us; T=4096: 625 dims 264.2 ->
// 235.7 us, 256 dims 253.8 -> 229.7 us but 8 dims 215.2 -> 228.6 us, so
// the larger T keep the two-row kernel.
constexpr int64_t kStreamMaxT = 2048;

// Row quantization for long rows (K > 32768) by persistent workgroups of WR
// waves that hold one row at a time in registers (CH 16-byte chunks per
// lane, chunk c = 64 (i WR + w) + lane for wave w) and take rows
// blockIdx.x, blockIdx.x + G, ... (G = gridDim.x): as soon as a chunk is
// quantized and stored, its registers are loaded with the same chunk of the
// workgroup's next row, so that row's loads fly while the current one is
// quantized and stored.  (k_rowquant_regs, two rows per workgroup and every
// load issued at once, ran its rounds of workgroups as loads, then
// arithmetic, then stores.)  Per row as k_rowquant_regs: row maximum over
// the non-outlier columns on the 16-bit patterns by packed unsigned max,
// quantization by the magic add, outlier halves zeroed by a byte mask and
// gathered into xo.
template <int HT, int WR, int CH>
__global__ __launch_bounds__(WR * kWave, 4) void k_rowquant_stream(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ parts,
    int nparts, int64_t kwp, int32_t* __restrict__ idx, int32_t* __restrict__ count,
    int8_t* __restrict__ xq, float* __restrict__ sx, uint16_t* __restrict__ xo) {
    constexpr int NT = WR * kWave;
    constexpr int KW = WR * CH * 64 * 8 / 32;          // bitmap words of the longest row
    constexpr int WPT = (KW + NT - 1) / NT;
    __shared__ uint32_t fl[KW];
    __shared__ int pf[KW];
    __shared__ int wtot[WR];
    __shared__ float wmx[2][WR];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wr = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nch = (int)(K / 8);
    const int kw = (int)((K + 31) / 32);
    const int64_t G = gridDim.x;
    // row of this workgroup in round j (rows G j .. G j + G - 1): with G a
    // multiple of 16, rows 2k and 2k+1 - the two 64-byte halves of each
    // 128-byte line of Xq - go to workgroups b and b + 8, which the
    // round-robin dispatch puts on the same XCD (one L2)
    const int64_t b = blockIdx.x;
    auto row_of = [&](int64_t j) -> int64_t {
        if (G % 16 == 0) return G * j + 2 * ((b >> 4) * 8 + (b & 7)) + ((b >> 3) & 1);
        return G * j + b;
    };

    // (a row pointer in scalar registers plus a 32-bit byte offset per load)
    auto load_row = [&](uint4 (&v)[CH], int64_t t) {
        const char* row = reinterpret_cast<const char*>(X + t * K);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = (i * WR + wr) * kWave + lane;
            v[i] = *reinterpret_cast<const uint4*>(row + (uint32_t)(c < nch ? c : 0) * 16u);
        }
    };

    // partial bitmaps, then the first row
    uint32_t fr[WPT][kDetectGroups];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int w = tid + NT * j;
#pragma unroll
        for (int r = 0; r < kDetectGroups; ++r)
            fr[j][r] = (w < kw && r < nparts) ? parts[(int64_t)r * kwp + w] : 0u;
    }
    __builtin_amdgcn_sched_barrier(0);
    int64_t t = row_of(0);   // the grid has at most T workgroups, so t < T
    uint4 v[CH];
    load_row(v, t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int w = tid + NT * j;
        uint32_t f = 0;
#pragma unroll
        for (int r = 0; r < kDetectGroups; ++r) f |= fr[j][r];
        if (w < kw) fl[w] = f;
    }
    __syncthreads();   // fl
    int o = 0;
    {
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) cnt += __builtin_popcount(fl[w]);
        }
        int run = block_excl_scan<NT>(cnt, wtot, o);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int w = WPT * tid + i;
            if (w < kw) {
                pf[w] = run;
                uint32_t f = fl[w];
                if (blockIdx.x == 0) {
                    int p = run;
                    while (f) {
                        idx[p++] = w * 32 + __builtin_ctz(f);
                        f &= f - 1u;
                    }
                }
                run += __builtin_popcount(fl[w]);
            }
        }
    }
    const int opad = (o + 15) & ~15;
    if (blockIdx.x == 0 && tid == 0) {
        count[0] = o;
        count[1] = opad;
    }
    __syncthreads();   // pf
    const bool whole_tiles = K % kKTile == 0;

    // one row: maximum, scale, quantize, store (slot: which wmx half); each
    // chunk's registers then take the next row's chunk (tn < 0: none)
    auto process = [&](int64_t tr, int slot, int64_t tn) {
        // the lane index through an empty asm: every per-chunk value is
        // recomputed for each row instead of twelve of each being hoisted
        // out of the row loop into registers
        int lane = threadIdx.x & (kWave - 1);
        asm volatile("" : "+v"(lane));
        const char* nrow = reinterpret_cast<const char*>(X + (tn >= 0 ? tn : 0) * K);
        // the row has arrived (one wait outside the per-chunk branches, so
        // the compiler knows no load into v is pending in the quantize loop
        // but the next row's, and adds no wait before each chunk there)
        __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0), expcnt and lgkmcnt not waited
        uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = (i * WR + wr) * kWave + lane;
            if (c < nch) {
                const uint32_t fm = (fl[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                uint32_t keep[4] = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
                if (fm) {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        keep[d] = (((fm >> (2 * d)) & 1u) ? 0u : 0x00007FFFu) |
                                  (((fm >> (2 * d + 1)) & 1u) ? 0u : 0x7FFF0000u);
                }
                m0 = pk_max_u16(m0, pk_max_u16(w[0] & keep[0], w[1] & keep[1]));
                m1 = pk_max_u16(m1, pk_max_u16(w[2] & keep[2], w[3] & keep[3]));
            }
        }
        const uint32_t m = pk_max_u16(m0, m1);
        const uint32_t mh = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
        float mx = wave_max(h16_to_f32<HT>((uint16_t)mh));
        if (lane == 0) wmx[slot][wr] = mx;
        __syncthreads();   // the waves' maxima of this row (the other slot is the next row's)
        mx = wmx[slot][0];
#pragma unroll
        for (int q = 1; q < WR; ++q) mx = __builtin_fmaxf(mx, wmx[slot][q]);
        const float qk = HT == kHalfF16 ? 1.0f : qfactor(mx);   // fp16 scales are >= 2^-24
        const float rr = mx > 0.0f ? 127.0f / (mx * qk) : 0.0f;   // IEEE fp32 divide
        uint16_t* xo_row = xo + tr * opad;
        const int64_t p0 = tr - tr % kPanel;
        const int64_t prow = T - p0 < kPanel ? T - p0 : kPanel;
        const int64_t qstep = 8 * WR * kKTile * prow;
        const int64_t q0 = p0 * K + (tr - p0) * kKTile + 8 * (lane & 7) +
                           (int64_t)(8 * wr + (lane >> 3)) * kKTile * prow;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = (i * WR + wr) * kWave + lane;
            if (c >= nch) continue;
            const uint32_t word = fl[c >> 2];
            const uint32_t fm = (word >> ((c & 3) * 8)) & 0xFFu;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            uint32_t f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
                const float p = __builtin_fmaf(x * qk, rr, 0.0f);
                f[e] = __builtin_bit_cast(uint32_t, __fadd_rn(p, 12582912.0f));
            }
            uint32_t packed[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t lo = __builtin_amdgcn_perm(f[4 * h + 1], f[4 * h], 0x0c0c0400u);
                const uint32_t hi = __builtin_amdgcn_perm(f[4 * h + 3], f[4 * h + 2], 0x0c0c0400u);
                packed[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
            if (fm) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t keep = 0u;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        keep |= ((fm >> (4 * h + e)) & 1u) ? 0u : (0xFFu << (8 * e));
                    packed[h] &= keep;
                }
                const int base_bit = (c & 3) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((fm >> e) & 1u) {
                        const int bit = base_bit + e;
                        const int pos = pf[c >> 2] + __builtin_popcount(word & ((1u << bit) - 1u));
                        xo_row[pos] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                    }
                }
            }
            const int64_t qo = whole_tiles ? q0 + i * qstep : blk_offset(tr, (int64_t)c * 8, T, K);
            *reinterpret_cast<uint2*>(xq + qo) = make_uint2(packed[0], packed[1]);
            if (tn >= 0) v[i] = *reinterpret_cast<const uint4*>(nrow + (uint32_t)c * 16u);
            // keep each reload after its chunk's use (no second register set)
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int j = o + tid; j < opad; j += NT) xo_row[j] = 0;   // +0 in both types
        if (tid == 0) sx[tr] = mx;
    };

    for (int64_t j = 1;; ++j) {
        const int64_t tn = row_of(j) < T ? row_of(j) : -1;   // uniform
        process(t, (int)(j & 1), tn);
        if (tn < 0) break;
        t = tn;
    }
}

// ---- activation pass for T <= kSmallT rows, two kernels over column
// segments.  A workgroup of 256 lanes owns kSegCols = 2048 columns, a lane 8
// of them in every row, so a column's outlier flag is the OR over the lane's
// own rows and needs no exchange.

constexpr int kSegThreads = kSegCols / 8;
static_assert(kSegThreads == 256 && kSmallT % 16 == 0, "row reductions: 16 rows x 16 lanes x 16 entries");

// Pass 1: the segment's outlier flags (whole bitmap words, written without
// atomics), per row the maximum |x| over its non-outlier columns, and its
// outlier count.  TB: T rounded up to a power of two; rows T .. TB-1 re-read
// row T-1 (a repeated row changes no flag and no maximum), so the loads are
// unconditional and all in flight together.
template <int HT, int TB>
__global__ __launch_bounds__(kSegThreads) void k_seg_scan(const uint16_t* __restrict__ X,
                                                          int64_t T, int64_t K, float tau,
                                                          uint32_t* __restrict__ flags,
                                                          float* __restrict__ segmax,
                                                          int32_t* __restrict__ segcnt) {
    __shared__ __attribute__((aligned(16))) float red[TB][kSegThreads];
    __shared__ int wtot[kSegThreads / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int64_t c0 = (int64_t)blockIdx.x * kSegCols + tid * 8;
    const bool in = c0 < K;
    uint4 v[TB];
    const uint16_t* xc = X + (in ? c0 : 0);
#pragma unroll
    for (int t = 0; t < TB; ++t) v[t] = *reinterpret_cast<const uint4*>(xc + (t < T ? t : T - 1) * K);
    uint32_t fm = 0;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
            fm |= (__builtin_fabsf(x) >= tau ? 1u : 0u) << e;
        }
    }
    // lanes past K (which read column 0) flag nothing
    if (!in) fm = 0;
    uint32_t word = fm << ((lane & 3) * 8);
    word |= __shfl_xor(word, 1);
    word |= __shfl_xor(word, 2);
    if ((lane & 3) == 0 && in) flags[c0 >> 5] = word;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        {
            const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
            float mx = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = __builtin_fabsf(h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16))));
                mx = ((fm >> e) & 1u) ? mx : __builtin_fmaxf(mx, a);
            }
            red[t][tid] = in ? mx : 0.0f;
        }
    }
    int total = 0;
    block_excl_scan(__builtin_popcount(fm), wtot, total);   // (its barrier also covers red)
    // row t = 16 g + tid / 16: each of 16 lanes takes the maximum of 16
    // entries, then 4 exchanges inside the group of 16 lanes (instead of a
    // 6-step wave reduction per row)
#pragma unroll
    for (int g = 0; g < (TB + 15) / 16; ++g) {
        const int t = g * 16 + (tid >> 4), part = tid & 15;
        float mx = 0.0f;
        if (t < T) {
            const float4* q = reinterpret_cast<const float4*>(&red[t][part * 16]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 f = q[i];
                mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(f.x, f.y), __builtin_fmaxf(f.z, f.w)));
            }
        }
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, d));
        if (part == 0 && t < T) segmax[blockIdx.x * kSmallT + t] = mx;
    }
    if (tid == 0) segcnt[blockIdx.x] = total;
}

// Pass 2: row scales s_x = max over the segments' maxima, outlier positions
// = outliers of earlier segments + prefix inside this one; writes idx, the
// quantized rows, the gathered outlier values (and, last segment, their zero
// padding) and, from segment 0, s_x and the count.  Grid: segments x groups
// of kQuantRows rows (rows past T re-read row T-1 and store nothing), so the
// quantization is spread over T / kQuantRows times more workgroups; every
// row group recomputes the segment's prefix from the bitmap.
constexpr int kQuantRows = 2;
template <int HT>
__global__ __launch_bounds__(kSegThreads) void k_seg_quant(
    const uint16_t* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ flags,
    const float* __restrict__ segmax, const int32_t* __restrict__ segcnt, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, int8_t* __restrict__ xq, float* __restrict__ sx,
    uint16_t* __restrict__ xo) {
    constexpr int RB = kQuantRows, PARTS = kSegThreads / RB;
    __shared__ float red[PARTS][RB];
    __shared__ int cnt[2][PARTS];
    __shared__ float sxs[RB], rxs[RB], qks[RB];
    __shared__ int wtot[kSegThreads / kWave];
    const int tid = threadIdx.x;
    const int seg = blockIdx.x, nseg = gridDim.x;
    const int t0 = blockIdx.y * RB;                // this workgroup's rows t0 .. t0+RB-1
    const int64_t c0 = (int64_t)seg * kSegCols + tid * 8;
    const bool in = c0 < K;
    uint4 v[RB];
    const uint16_t* xc = X + (in ? c0 : 0);
#pragma unroll
    for (int r = 0; r < RB; ++r) v[r] = *reinterpret_cast<const uint4*>(xc + (t0 + r < T ? t0 + r : T - 1) * K);
    const uint32_t fm = in ? (flags[c0 >> 5] >> ((c0 >> 3) & 3) * 8) & 0xFFu : 0u;
    // the segments' maxima of the RB rows and the outlier counts: thread
    // (row r = tid % RB, part = tid / RB) takes segments part, part + PARTS, ...
    {
        const int r = tid % RB, part = tid / RB;
        const int t = t0 + r < T ? t0 + r : T - 1;
        float mx = 0.0f;
        int before = 0, all = 0;
        for (int s = part; s < nseg; s += PARTS) {
            mx = __builtin_fmaxf(mx, segmax[s * kSmallT + t]);
            const int c = segcnt[s];
            before += s < seg ? c : 0;
            all += c;
        }
        red[part][r] = mx;
        if (r == 0) {
            cnt[0][part] = before;
            cnt[1][part] = all;
        }
    }
    __syncthreads();
    // row scales: RB groups of 64 lanes reduce the parts (wave-wide maximum)
    {
        const int r = tid / kWave, l = tid & (kWave - 1);
        if (r < RB) {
            float mx = 0.0f;
            for (int p = l; p < PARTS; p += kWave) mx = __builtin_fmaxf(mx, red[p][r]);
            mx = wave_max(mx);
            if (l == 0) {
                const float qk = HT == kHalfF16 ? 1.0f : qfactor(mx);   // fp16: >= 2^-24
                sxs[r] = mx;
                qks[r] = qk;
                rxs[r] = mx > 0.0f ? 127.0f / (mx * qk) : 0.0f;   // IEEE fp32 divide
            }
        }
    }
    // outliers before this segment, and in all: each wave sums the parts
    int before = 0, o = 0;
    {
        const int l = tid & (kWave - 1);
        for (int p = l; p < PARTS; p += kWave) {
            before += cnt[0][p];
            o += cnt[1][p];
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            before += __shfl_xor(before, d);
            o += __shfl_xor(o, d);
        }
    }
    const int opad = (o + 15) & ~15;
    int seg_total = 0;
    const int pos0 = before + block_excl_scan(__builtin_popcount(fm), wtot, seg_total);   // barrier: sxs, rxs ready
    if (seg == 0 && blockIdx.y == 0 && tid == 0) {
        count[0] = o;
        count[1] = opad;
    }
    if (seg == 0 && tid < RB && t0 + tid < T) sx[t0 + tid] = sxs[tid];
    if (seg == nseg - 1)
        for (int e = tid; e < RB * (opad - o); e += kSegThreads) {
            const int r = e / (opad - o), j = o + e % (opad - o);
            if (t0 + r < T) xo[(int64_t)(t0 + r) * opad + j] = 0;   // +0 in both types
        }
    if (!in) return;
    if (fm && blockIdx.y == 0) {
        int pos = pos0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((fm >> e) & 1u) idx[pos++] = (int32_t)(c0 + e);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t t = t0 + r;
        if (t < T) {
            const float rr = rxs[r], qk = qks[r];
            const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = h16_to_f32<HT>((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
                const uint32_t q = ((fm >> e) & 1u) ? 0u : (uint32_t)(uint8_t)quant(x * qk, rr);
                packed[e >> 2] |= q << ((e & 3) * 8);
            }
            *reinterpret_cast<uint2*>(xq + blk_offset(t, c0, T, K)) = make_uint2(packed[0], packed[1]);
            if (fm) {
                int pos = pos0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((fm >> e) & 1u) xo[t * opad + pos++] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

template <int HT, int TB>
void launch_seg(const uint16_t* xb, int64_t T, int64_t K, float tau, const Workspace& ws,
                hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(K, kSegCols));
    hipLaunchKernelGGL((k_seg_scan<HT, TB>), grid, dim3(kSegThreads), 0, stream, xb, T, K, tau,
                       ws.flags, ws.segmax, ws.segcnt);
    const dim3 qgrid(grid.x, (unsigned)ceil_div(T, kQuantRows));
    hipLaunchKernelGGL((k_seg_quant<HT>), qgrid, dim3(kSegThreads), 0, stream, xb, T, K,
                       ws.flags, ws.segmax, ws.segcnt, ws.idx, ws.count, ws.xq, ws.sx, ws.xo);
}

// Shape of the register-resident row quantization for rows of K values:
// waves per workgroup, waves per row and 16-byte chunks per lane.  Many
// waves with few chunks each measured fastest (rows in flight at different
// stages overlap their loads, arithmetic and stores): about 6 chunks per
// lane, 4 to 8 waves per row; at K = 32768 4 waves of 16 chunks; past it 8
// waves of 12 chunks, two rows per workgroup (whole calls, down projection:
// -0.4% against 16 waves of 6, +1% with 4 waves of 24).
// Activation pass alone, against one workgroup of 512 lanes per row:
// T=2048, K=12288 32.5 -> 25.2 us; T=2048, K=49152 110.1 -> 94.0 us;
// T=4096, K=12288 57.3 -> 44.1 us; T=3000, K=24576 86.2 -> 62.5 us.
template <int HT>
void launch_rowquant_regs(const uint16_t* xb, int64_t T, int64_t K, int nparts, int64_t kwp,
                          const Workspace& ws, hipStream_t stream) {
    auto go = [&](auto kern, int nw, int wr) {
        const unsigned grid = (unsigned)ceil_div(T, nw / wr);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(nw * kWave), 0, stream, xb, T, K, ws.flags, nparts,
                           kwp, ws.idx, ws.count, ws.xq, ws.sx, ws.xo);
    };
    if (K <= 4096) go(k_rowquant_regs<HT, 4, 2, 4>, 4, 2);
    else if (K <= 8192) go(k_rowquant_regs<HT, 4, 4, 4>, 4, 4);
    else if (K <= 12288) go(k_rowquant_regs<HT, 4, 4, 6>, 4, 4);
    else if (K <= 16384) go(k_rowquant_regs<HT, 8, 8, 4>, 8, 8);
    else if (K <= 24576) go(k_rowquant_regs<HT, 8, 8, 6>, 8, 8);
    else if (K <= 32768) go(k_rowquant_regs<HT, 4, 4, 16>, 4, 4);
    else if (T <= kStreamMaxT) {
        // persistent, two workgroups of 8 waves per CU
        const int64_t g = std::min<int64_t>(T, 2 * (int64_t)device_cus());
        hipLaunchKernelGGL((k_rowquant_stream<HT, 8, 12>), dim3((unsigned)g), dim3(8 * kWave), 0, stream, xb, T, K,
                           ws.flags, nparts, kwp, ws.idx, ws.count, ws.xq, ws.sx, ws.xo);
    } else {
        go(k_rowquant_regs<HT, 16, 8, 12>, 16, 8);
    }
}

}  // namespace

template <int HT>
static void launch_activation_typed(const uint16_t* xb, int64_t T, int64_t K, float tau,
                             const Workspace& ws, hipStream_t stream, int32_t* zero, int64_t nzero) {
    if (T <= kSmallT) {
        const dim3 grid((unsigned)ceil_div(K, kSegCols));
        if (T <= 1) launch_seg<HT, 1>(xb, T, K, tau, ws, stream);
        else if (T <= 2) launch_seg<HT, 2>(xb, T, K, tau, ws, stream);
        else if (T <= 4) launch_seg<HT, 4>(xb, T, K, tau, ws, stream);
        else if (T <= 8) launch_seg<HT, 8>(xb, T, K, tau, ws, stream);
        else launch_seg<HT, 16>(xb, T, K, tau, ws, stream);
        return;
    }
    const int64_t kw = ceil_div(K, 32);
    if (T <= kOwnedMaxT) {
        // few enough rows for one workgroup per column block: flags stored
        // whole, no clearing kernel
        hipLaunchKernelGGL(k_detect_owned<HT>, dim3((unsigned)ceil_div(K, kOwnedCols)),
                           dim3(kOwnedWaves * kWave), 0, stream, xb, T, K, tau, ws.flags);
    } else if (K <= kRegMaxK) {
        // row groups: partial bitmaps, ORed by the quantize kernel
        const int64_t kwp = bitmap_stride(K);
        const int groups = (int)std::min<int64_t>(kDetectGroups, ceil_div(T, kColRowsPerPass));
        if (K > 16384)
            hipLaunchKernelGGL((k_detect_cols<HT, kColBlockLong>), dim3((unsigned)ceil_div(K, kColBlockLong), (unsigned)groups),
                               dim3(kColWaves * kWave), 0, stream, xb, T, K, tau, ws.flags, kwp, zero, nzero);
        else
            hipLaunchKernelGGL((k_detect_cols<HT, kColBlockShort>), dim3((unsigned)ceil_div(K, kColBlockShort), (unsigned)groups),
                               dim3(kColWaves * kWave), 0, stream, xb, T, K, tau, ws.flags, kwp, zero, nzero);
        launch_rowquant_regs<HT>(xb, T, K, groups, kwp, ws, stream);
        return;
    } else {
        hipLaunchKernelGGL((k_detect_cols<HT, kColBlockLong>), dim3((unsigned)ceil_div(K, kColBlockLong), 1u),
                           dim3(kColWaves * kWave), 0, stream, xb, T, K, tau, ws.flags, (int64_t)0, zero,
                           nzero);
    }
    // rows held in registers: the quantize kernel isolates the outliers too
    if (K <= (int64_t)kRowThreads * 4 * 8) {
        hipLaunchKernelGGL((k_rowquant_cached<HT, 4, kRowThreads>), dim3((unsigned)T), dim3(kRowThreads), 0,
                           stream, xb, T, K, ws.flags, ws.idx, ws.count, ws.xq, ws.sx, ws.xo);
    } else if (K <= (int64_t)kRowThreads * 12 * 8) {
        hipLaunchKernelGGL((k_rowquant_cached<HT, 12, kRowThreads>), dim3((unsigned)T), dim3(kRowThreads), 0,
                           stream, xb, T, K, ws.flags, ws.idx, ws.count, ws.xq, ws.sx, ws.xo);
    } else {
        hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, stream, ws.flags, kw,
                           ws.wprefix, ws.idx, ws.count);
        hipLaunchKernelGGL(k_rowquant<HT>, dim3((unsigned)T), dim3(kQuantThreads), 0, stream, xb,
                           T, K, ws.flags, ws.wprefix, ws.count, ws.xq, ws.sx, ws.xo);
    }
}

hipError_t launch_activation_pass(const uint16_t* X, int ht, int64_t T, int64_t K, float tau,
                                  const Workspace& ws, hipStream_t stream, int32_t* zero,
                                  int64_t nzero) {
    // only the column detection (more than kOwnedMaxT rows) zeroes words
    if (nzero > 0 && (!zero || T <= kOwnedMaxT)) return hipErrorInvalidValue;
    if (ht == kHalfBF16) launch_activation_typed<kHalfBF16>(X, T, K, tau, ws, stream, zero, nzero);
    else launch_activation_typed<kHalfF16>(X, T, K, tau, ws, stream, zero, nzero);
    return hipGetLastError();
}

namespace {
// Debug copy of the quantized activations: the workspace's panel-blocked
// Xq to a row-major [T,K] array, one 16-byte piece per thread.
__global__ void k_unblock(const int8_t* __restrict__ src, int64_t T, int64_t K,
                          int8_t* __restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = K / 16;
    if (i >= T * per) return;
    const int64_t t = i / per, k = (i - t * per) * 16;
    *reinterpret_cast<uint4*>(dst + t * K + k) =
        *reinterpret_cast<const uint4*>(src + blk_offset(t, k, T, K));
}
}  // namespace

hipError_t launch_debug_copies(const Workspace& ws, int64_t T, int64_t K, int32_t* count,
                               int32_t* idx, int8_t* xq, float* sx, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if (count && e == hipSuccess)
        e = hipMemcpyAsync(count, ws.count, sizeof(int32_t), hipMemcpyDeviceToDevice, stream);
    if (idx && e == hipSuccess)
        e = hipMemcpyAsync(idx, ws.idx, sizeof(int32_t) * (size_t)K, hipMemcpyDeviceToDevice,
                           stream);
    if (xq && e == hipSuccess) {
        const int64_t pieces = T * (K / 16);
        hipLaunchKernelGGL(k_unblock, dim3((unsigned)ceil_div(pieces, 256)), dim3(256), 0, stream,
                           ws.xq, T, K, xq);
        e = hipGetLastError();
    }
    if (sx && e == hipSuccess)
        e = hipMemcpyAsync(sx, ws.sx, sizeof(float) * (size_t)T, hipMemcpyDeviceToDevice, stream);
    return e;
}

Workspace carve_workspace(void* base, int64_t T, int64_t K, int64_t N, bool wrec, int ksplit,
                          int dslabs) {
    Workspace w{};
    const int64_t kw = ceil_div(K, 32);
    size_t off = 0;
    char* b = static_cast<char*>(base);
    auto take = [&](size_t n) {
        char* p = b ? b + off : nullptr;
        off += align256(n);
        return p;
    };
    // partial bitmaps only for the detection in row groups
    const bool groups = T > kOwnedMaxT && K <= kRegMaxK;
    w.flags = reinterpret_cast<uint32_t*>(
        take(sizeof(uint32_t) * (size_t)(groups ? kDetectParts * bitmap_stride(K) : kw)));
    w.wprefix = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)kw));
    w.count = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 4));
    const int64_t nseg = ceil_div(K, kSegCols);
    w.segmax = reinterpret_cast<float*>(take(sizeof(float) * (size_t)(nseg * kSmallT)));
    w.segcnt = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)nseg));
    w.idx = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)K));
    w.sx = reinterpret_cast<float*>(take(sizeof(float) * (size_t)T));
    w.xq = reinterpret_cast<int8_t*>(take((size_t)T * (size_t)K));
    // worst case: every dimension an outlier, o = K (K % 16 == 0, so opad <= K)
    w.xo = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * (size_t)T * (size_t)K));
    // optional regions after the fixed ones, so that a smaller workspace is a
    // valid prefix: the recovered outlier rows, then the K split (which
    // needs them)
    if (wrec) {
        w.wrec_rows = K < kRecoverRows ? K : kRecoverRows;
        w.wrec = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * (size_t)w.wrec_rows * (size_t)N));
    }
    if (wrec && ksplit >= 2) {
        // after everything else, so the layout without the split is a prefix;
        // one counter per split tile and the partial sums of each part:
        // large-tile kernel (more than 128 rows) two halves of 256 x 256,
        // streaming kernel S slabs of its tile
        if (T > 128 && !stream_256x128(T, K, N)) {
            const int64_t nsplit = gemm_ksplit_plan(T, K, N).nsplit;
            w.ks_count = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)nsplit));
            w.ks_part = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)nsplit * 2 * 65536));
        } else {
            const StreamSplit sp = stream_split(T, K, N);
            w.ks_count = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)sp.tiles));
            w.ks_part = reinterpret_cast<int32_t*>(take((size_t)sp.tiles * (size_t)sp.s * (size_t)sp.tile_bytes));
        }
    }
    if (dslabs > 0) {
        w.dslabs = dslabs;
        w.dpart = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)dslabs * (size_t)T * (size_t)N));
    }
    w.bytes = off;
    return w;
}

}  // namespace i8mm
