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
//   - one workgroup per compute unit owns bpw whole 16-row blocks of Wq
//     (bpw = ceil(blocks / CUs), so the weight spreads evenly over the chip);
//     the blocks are cut into 16 KB chunks (16 rows x 1024 k) that the eight
//     waves take from an LDS counter as they go, so waves that the SIMD
//     arbitration favours simply take more chunks and all of them finish
//     together; each chunk's int32 partial sums are added into LDS (exact and
//     order independent);
//   - the workgroup recomputes the activation side from X (T*K fp16, cache
//     resident): a thread owns whole 8-column pieces across all T rows, so
//     the outlier flags of its columns need no exchange; row absmax by a
//     transposed butterfly and LDS; ascending outlier indices by a popcount
//     prefix scan; Xq to LDS.  Every wave's first chunk goes out in four
//     parts over that work once X has arrived, and (K = 8192 with more than
//     16 chunks per workgroup) its second chunk before the last barrier;
//   - Wq goes from global memory straight into registers as the A operand of
//     v_mfma_i32_16x16x64_i8 (16 weight rows x 64 k), through a ring of two
//     chunks of 16 loads per wave; the B operand (the T activation rows as
//     columns, zero padded) is read from LDS per k-step;
//   - after the stream the workgroup dequantizes the int32 sums, adds the
//     fp16 outlier product in fp32 (W16 values of the first outliers were
//     fetched during the stream) and rounds Y to fp16 once.
// Limits (host checks them; other shapes use the general kernels):
// T <= 16, K in {4096, 8192}, T*K <= 65536.
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <type_traits>

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
constexpr int kMaxBpw = 12;            // 16-row blocks per workgroup (N <= 49152 in one round)
constexpr int kSmallBpw = 8;           // LDS sized for at most this many in the common case
constexpr int kW16Cache = 16;          // outliers whose W16 values are staged in LDS
constexpr int kChunkKConst = 1024;     // k covered by one weight chunk


struct DecodeArgs {
    const uint16_t* x;      // [T,K] 16-bit (fp16, or bf16 for the bf16 variant)
    const int8_t* wq;       // [N,K]
    const float* sw;        // [N]
    const uint16_t* w16;    // [K,N] 16-bit, or NULL: outlier rows recovered from wq
    uint16_t* y;            // [T,N] 16-bit
    float tau;
    uint32_t tau16;         // bits of the smallest 16-bit value >= tau (+inf if none finite)
    int T, K, N;
    int bpw;                // 16-row blocks per workgroup (1..kMaxBpw)
    int ileave;             // 1: workgroup g owns blocks g, g + groups, ...; 0: bpw consecutive blocks
    int cpb;                // K / 1024 (used when the chunk count is not a template constant)
    // activation side computed beforehand by the activation-pass kernels
    // (precomputed mode only): Xq [T,K], s_x [T], count {o, opad}, idx [o],
    // the outlier columns of X [T,opad] 16-bit
    const int8_t* xq_pre;
    const float* sx_pre;
    const int32_t* count_pre;
    const int32_t* idx_pre;
    const uint16_t* xo_pre;
    // K slabs (precomputed mode): the grid is slabs x groups of bpw blocks,
    // slab s covers k-chunks s*cps .. (at most cps of them, cpb in all); with
    // slabs > 1 each workgroup writes its int32 sums to part [slabs][T][N]
    // and k_decode_finish completes Y
    int slabs;
    int cps;
    int32_t* part;
    // optional debug outputs (NULL to skip); workgroup 0 writes all but acc
    int32_t* dbg_count;
    int32_t* dbg_idx;
    int8_t* dbg_xq;
    float* dbg_sx;
    int32_t* dbg_acc;
};

// Xq rows carry a 16-byte pad: the B-operand read has 16 lanes on 16
// different rows, which then fall on distinct banks.
// XK: bytes of Xq; IDXN: outlier dimensions kept; OXL: outliers whose X
// values are kept; NCF: entries of cfirst; MAXB: 16-row blocks per workgroup.
template <int XK, int IDXN, int OXL, int NCF, int MAXB>
struct SmemT {
    int8_t xq[XK + kMaxT * 16];
    int32_t idx[IDXN];                         // outlier dims, ascending
    float xo[kMaxT * OXL];                     // X values of the first outliers
    int32_t acc[MAXB][kRows][16];              // int32 sums [block][row][t]
    uint32_t w16o[kW16Cache][MAXB * kRows / 2];   // W16[idx_j, n] pairs of the rows
    int8_t wqo[kW16Cache][MAXB * kRows];       // Wq[n, idx_j] (memory-halved variant)
    int32_t cfirst[NCF];                       // first outlier at or past k = 1024 c
    float sw[MAXB * kRows];                    // s_w of the rows
    float wmax[kWaves][kMaxT];
    float sx[kMaxT];
    float rx[kMaxT];                           // 127 / (s_x * qk) (0 when s_x = 0)
    float qk[kMaxT];                           // tiny-scale factor of the row (qfactor)
    int32_t wtot[kWaves * 2];
    int32_t next;                              // next chunk to hand out
};
// activation side computed in the kernel: every outlier dimension in LDS
template <int MAXB>
using Smem = SmemT<kMaxXK, kMaxK, kMaxOutliersLds, kMaxK / kChunkKConst + 1, MAXB>;
// activation side precomputed: twice the Xq room, only the first outliers
constexpr int kMaxXKPre = 131072;              // T*K bytes of Xq kept in LDS
constexpr int kOutliersLdsPre = 64;
constexpr int kMaxCpbPre = kMaxXKPre / kChunkKConst;
template <int MAXB>
using SmemPre = SmemT<kMaxXKPre, kW16Cache, kOutliersLdsPre, kMaxCpbPre + 1, MAXB>;
static_assert(sizeof(SmemPre<kMaxBpw>) <= 160 * 1024, "LDS of one workgroup");

template <int HT>
__device__ inline float chunk_val(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return h16_to_f32<HT>((uint16_t)(w >> ((e & 1) * 16)));
}

constexpr int kLoads = 16;                    // 16-byte loads per lane per chunk (16 KB/wave)
constexpr int kChunkK = kLoads * 64;          // k covered by one chunk
static_assert(kChunkK == kChunkKConst, "chunk size");


// CPB = K / 1024 chunks per 16-row block; a thread owns CPT = K / 4096
// chunks of 8 columns (c = tid + 512 j) in the activation prologue, for all
// T <= TMAX = 64 / CPB rows (so T * CPT <= 16 chunks of X per thread).
// PRE: the activation side was computed by the activation-pass kernels and
// is read from their workspace (CPB = 0: the chunk count is a.cpb); this
// serves T <= 16 for any K that is a multiple of 1024 with T*K <= 128 KB
// (the host sends it T <= 8 only, and longer K in slabs).
// MAXB: the most 16-row blocks a workgroup owns (a.bpw <= MAXB); the LDS
// arrays per row are sized for it (kSmallBpw keeps the common case's
// footprint and code as small as they were).  EARLY (activation side
// computed in the kernel only): the second ring slot's chunk is issued
// before the prologue's last barrier.
template <int CPB, int HT, bool PRE, int MAXB, bool EARLY>
__global__ __launch_bounds__(kThreads) void k_decode(DecodeArgs a) {
    static_assert(PRE == (CPB == 0), "the precomputed mode takes its chunk count at run time");
    static_assert(!(PRE && EARLY), "the early second chunk belongs to the in-kernel prologue");
    // W16 values of the first outliers fetched per thread during the stream
    constexpr int kW16Pairs = MAXB * kRows / 2;
    constexpr int kW16PerThread = kW16Cache * kW16Pairs / kThreads;
    static_assert(kW16Cache * kW16Pairs == kW16PerThread * kThreads, "whole loads per thread");
    constexpr int CPT = PRE ? 1 : CPB / 4;
    constexpr int TMAX = PRE ? 1 : 64 / CPB;
    constexpr int OXL = PRE ? kOutliersLdsPre : kMaxOutliersLds;
    using SM = typename std::conditional<PRE, SmemPre<MAXB>, Smem<MAXB>>::type;
    static_assert(sizeof(SM::acc) % 16 == 0, "cleared in 16-byte pieces");
    __shared__ __attribute__((aligned(16))) SM sm;
    // slab and block group of this workgroup (slab-major grid)
    const int groups = PRE ? (int)gridDim.x / a.slabs : (int)gridDim.x;
    const int slab = PRE ? (int)blockIdx.x / groups : 0;
    const int grp = (int)blockIdx.x - slab * groups;
    // k-chunks of this workgroup's slab (all of K without slabs) and the
    // slab's first k
    const int cpb = PRE ? (a.cpb - slab * a.cps < a.cps ? a.cpb - slab * a.cps : a.cps) : CPB;
    const int kbase = PRE ? slab * a.cps * kChunkK : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (a scalar), so the chunk loop below is uniform control flow
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = a.T, K = a.K, N = a.N;
    const int ldx = cpb * kChunkK + 16;        // LDS row stride of Xq (the slab's k)
    const int nblocks = (N + kRows - 1) / kRows;
    // this workgroup's blocks: slot s holds block b0 + s * bstep (rows past N
    // are read as row N-1 and never stored); chunk id -> slot id / cpb,
    // k-chunk id % cpb.  Consecutive blocks (bstep = 1), or with ileave the
    // blocks grp, grp + groups, ... (see launch_decode)
    const bool ilv = a.ileave != 0;
    const int b0 = ilv ? grp : grp * a.bpw;
    const int bstep = ilv ? groups : 1;
    const int nbw = ilv ? (nblocks - grp + groups - 1) / groups
                        : (a.bpw < nblocks - b0 ? a.bpw : nblocks - b0);
    const int rows = nbw * kRows;
    // weight row of the workgroup's row r (slot r / 16)
    auto nrow = [&](int r) { return (b0 + (r >> 4) * bstep) * kRows + (r & 15); };
    const int total = nbw * cpb;

    // Load i of a chunk: lane l holds weight row nrow(16 (id / cpb) + l % 16)
    // and bytes 1024 (id % cpb) + 64 i + 16 (l / 16) .. +16 of its k range.
    // In the panel-blocked layout (K % 1024 == 0, so every k-tile is 64
    // wide) a block's 16 rows lie in one panel and load i reads one
    // contiguous kilobyte of k-tile 16 (id % cpb) + i; consecutive loads are
    // one block (64 x the panel's rows) apart.  Ids past the end read the
    // first 16 bytes of Wq on every lane instead (never used): loads stay
    // unconditional, so the wait counts stay exact.
    const int kl = (lane >> 4) * 16;
    // loads lo .. hi-1 of chunk id into buf (lo and hi are constants)
    auto issue_part = [&](int id, v4i (&buf)[kLoads], int lo, int hi) {
        const int n = (b0 + (id / cpb) * bstep) * kRows + (lane & 15);
        const int64_t nc = n < N ? n : N - 1;
        const int64_t p0 = nc - nc % kPanel;
        const int64_t prow = N - p0 < kPanel ? N - p0 : kPanel;
        const bool live = id < total;
        const int64_t off = live ? p0 * K + (int64_t)(kbase + (id % cpb) * kChunkK) * prow +
                                       (nc - p0) * kKTile + kl
                                 : 0;
        const int64_t step = live ? kKTile * prow : 0;
        const int8_t* p = a.wq + off;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            if (i >= lo && i < hi) buf[i] = *reinterpret_cast<const v4i*>(p + i * step);
    };
    auto issue = [&](int id, v4i (&buf)[kLoads]) { issue_part(id, buf, 0, kLoads); };

    // s_w of the rows, one float4 per thread (a block's first row and N are
    // multiples of 8, so a group of 4 rows is all in range or read as the last 4)
    float4 sw4;
    {
        const int n = tid * 4 < rows && nrow(tid * 4) < N ? nrow(tid * 4) : N - 4;
        sw4 = *reinterpret_cast<const float4*>(a.sw + n);
    }
    {
        constexpr int kClr = (int)(sizeof(sm.acc) / 16);   // 16-byte pieces
#pragma unroll
        for (int i = 0; i < (kClr + kThreads - 1) / kThreads; ++i) {
            const int q = tid + kThreads * i;
            if (kClr % kThreads == 0 || q < kClr)
                reinterpret_cast<uint4*>(&sm.acc[0][0][0])[q] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if (tid == 0) sm.next = 2 * kWaves;   // chunks 0 .. 15 go out statically

    // wave w starts with chunks w and w + 8; later ones come from the LDS
    // counter, so each wave's ids increase in the order it uses them.
    // X is loaded before any weight: vector-memory counters retire in order,
    // so a wait on X would also wait for weight loads issued before it.  The
    // first chunk then goes out in four parts spread over the activation
    // work: the memory pipe takes a CU's requests only as fast as it returns
    // data, so a wave issuing all of it at once would stall there instead of
    // computing (issuing more of the weight earlier, before X or from the
    // second chunk, measured slower).  Scheduling barriers keep each part
    // where it is.
    constexpr int G1 = kLoads / 4, G2 = kLoads / 2, G3 = 3 * kLoads / 4;
    // two slots: whole calls measured equal or faster than with three (T=4,
    // K=4096, N=14336 19.1 -> 17.5 us; T=8, K=12288, N=36864 94.7 -> 93.0 us)
    v4i ring[2][kLoads];
    int id0 = wave, id1 = wave + kWaves;

    int o = 0, opad = 0;   // outlier count (and, precomputed mode, its padded value)
    if constexpr (!PRE) {
        // X: rows t >= T re-read row T-1: a repeated row changes neither the
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
        // order is the numeric order (fp16 and bf16 alike), so |x| >= tau <=>
        // bits(|x|) >= tau16, with tau16 the bits of the smallest 16-bit value
        // >= tau (+inf when none is finite).
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
        // the flags must be final (so X has arrived) before more weight loads
        // are issued: an empty asm that consumes them and orders memory
    #pragma unroll
        for (int j = 0; j < CPT; ++j) asm volatile("" ::"v"(fm[j]) : "memory");
        if (tid * 4 < rows) *reinterpret_cast<float4*>(&sm.sw[tid * 4]) = sw4;
        issue_part(id0, ring[0], 0, G1);
        __builtin_amdgcn_sched_barrier(0);

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
            rmax[t] = h16_to_f32<HT>((uint16_t)mh);
        }
        // Row maxima over the wave by a transposed butterfly: each exchange at
        // distance d = 32, 16, ... halves the rows a lane carries (it keeps the
        // half picked by its lane bit d and sends the other half); plain
        // exchanges then finish the one row left.  Lane l ends with the maximum
        // of row l / (64 / TMAX): log2(64) + TMAX - 1 exchanges instead of
        // log2(64) per row.
        {
            float v[TMAX];
    #pragma unroll
            for (int t = 0; t < TMAX; ++t) v[t] = rmax[t];
    #pragma unroll
            for (int cnt = TMAX, d = 32; cnt > 1; cnt >>= 1, d >>= 1) {
                const bool up = (lane & d) != 0;
    #pragma unroll
                for (int i = 0; i < cnt / 2; ++i) {
                    const float send = up ? v[i] : v[i + cnt / 2];
                    const float keep = up ? v[i + cnt / 2] : v[i];
                    v[i] = __builtin_fmaxf(keep, __shfl_xor(send, d));
                }
            }
    #pragma unroll
            for (int d = 32 / TMAX; d >= 1; d >>= 1) v[0] = __builtin_fmaxf(v[0], __shfl_xor(v[0], d));
            const int r = lane / (64 / TMAX);
            if (lane % (64 / TMAX) == 0 && r < T) sm.wmax[wave][r] = v[0];
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_part(id0, ring[0], G1, G2);
        __builtin_amdgcn_sched_barrier(0);
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
        __builtin_amdgcn_sched_barrier(0);
        issue_part(id0, ring[0], G2, G3);
        __builtin_amdgcn_sched_barrier(0);
        if (tid < T) {
            float v = sm.wmax[0][tid];
    #pragma unroll
            for (int w = 1; w < kWaves; ++w) v = __builtin_fmaxf(v, sm.wmax[w][tid]);
            const float qk = HT == kHalfF16 ? 1.0f : qfactor(v);   // fp16 scales are >= 2^-24
            sm.sx[tid] = v;
            sm.qk[tid] = qk;
            sm.rx[tid] = v > 0.0f ? 127.0f / (v * qk) : 0.0f;   // IEEE fp32 divide
        }
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
        __syncthreads();   // sx, rx ready
        __builtin_amdgcn_sched_barrier(0);
        issue_part(id0, ring[0], G3, kLoads);
        __builtin_amdgcn_sched_barrier(0);
        // Quantize the owned columns into LDS and gather the outliers.
        // q = rint(x * r) by the 1.5 * 2^23 addition: for |p| < 2^22, p + 1.5*2^23
        // rounds p to the nearest integer (ties to even) and the low byte of the
        // result's bit pattern is that integer as int8.  |x| <= s_x makes
        // |p| <= 127 * (1 + 2^-23), so q is within [-127, 127] without a clamp.
        // The product and the add stay separate roundings: p = fma(x, r, +0) is
        // the fp32 product x * r rounded once (one mixed fp16/fp32 instruction),
        // then the add rounds again.  Bytes are packed with v_perm.
    #pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + kThreads * j;
            // byte mask that zeroes the outlier columns of the piece
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
                const float rr = t < T ? sm.rx[t] : 0.0f;
                const float qk = HT == kHalfF16 ? 1.0f : (t < T ? sm.qk[t] : 1.0f);
                uint32_t f[8];
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __builtin_fmaf(chunk_val<HT>(xr[j][t], e) * qk, rr, 0.0f);
                    f[e] = __builtin_bit_cast(uint32_t, __fadd_rn(p, 12582912.0f));
                }
                uint32_t packed[2];
    #pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t lo = __builtin_amdgcn_perm(f[4 * h + 1], f[4 * h], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm(f[4 * h + 3], f[4 * h + 2], 0x0c0c0400u);
                    packed[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) & keep[h];
                }
                *reinterpret_cast<uint2*>(&sm.xq[t * ldx + c * 8]) = make_uint2(packed[0], packed[1]);
            }
            if (fm[j]) {
                int pos = pc[j];
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((fm[j] >> e) & 1u) {
                        sm.idx[pos] = c * 8 + e;
                        if (blockIdx.x == 0 && a.dbg_idx) a.dbg_idx[pos] = c * 8 + e;
                        if (pos < OXL) {
    #pragma unroll
                            for (int t = 0; t < TMAX; ++t)
                                sm.xo[t * OXL + pos] = chunk_val<HT>(xr[j][t], e);
                        }
                        ++pos;
                    }
                }
            }
        }
        // number of outliers before each 1024-column chunk: the thread owning the
        // first 8-column piece of chunk cc knows it (its prefix count)
    #pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c8 = tid + kThreads * j;
            if ((c8 & (kChunkK / 8 - 1)) == 0) sm.cfirst[c8 / (kChunkK / 8)] = pc[j];
        }
        // EARLY: the second chunk goes out here rather than after the last
        // barrier; the first has landed by now, so the HBM would otherwise
        // idle through the barrier and the W16 fetch (decode workload 45.8 ->
        // 45.3 us per call; when the 16 chunks the waves start with are all
        // of a workgroup's, as at K = 4096, N = 14336, 2.4-3.3% slower).  A
        // run-time choice made the compiler's wait counts at the loop entry
        // cover both orders (up to 10% slower), hence a template parameter.
        if constexpr (EARLY) {
            __builtin_amdgcn_sched_barrier(0);
            issue(id1, ring[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (tid == 0) sm.cfirst[K / kChunkK] = o;
        if (blockIdx.x == 0 && tid == 0 && a.dbg_count) a.dbg_count[0] = o;
        if (blockIdx.x == 0 && a.dbg_sx && tid < T) a.dbg_sx[tid] = sm.sx[tid];
        __syncthreads();   // Xq, idx, xo ready
        if (blockIdx.x == 0 && a.dbg_xq) {
            for (int i = tid; i < T * (K / 8); i += kThreads) {
                const int t = i / (K / 8), c8 = (i % (K / 8)) * 8;
                *reinterpret_cast<uint2*>(a.dbg_xq + (int64_t)t * K + c8) =
                    *reinterpret_cast<const uint2*>(&sm.xq[t * ldx + c8]);
            }
        }
    } else {
        // Activation side from the workspace of the activation-pass kernels:
        // Xq rows into LDS, the row scales, the first outliers' dimensions
        // and X values, and per 1024-column chunk how many of those first
        // outliers precede it.  Xq (L2-resident) goes out first, all of it at
        // once, then the first weight chunk, so that waiting for Xq leaves
        // the weight loads in flight.
        o = a.count_pre[0];
        opad = a.count_pre[1];
        constexpr int XV = kMaxXKPre / 16 / kThreads;   // 16-byte pieces per thread
        const int pr = cpb * (kChunkK / 16);            // pieces per row of the slab
        const int nx = T * pr;
        uint4 xv[XV];
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int i = tid + kThreads * u;
            const int t = i / pr, c = i - t * pr;
            xv[u] = i < nx ? *reinterpret_cast<const uint4*>(a.xq_pre + blk_offset(t, kbase + c * 16, T, K))
                           : make_uint4(0u, 0u, 0u, 0u);
        }
        issue(id0, ring[0]);
        if (tid * 4 < rows) *reinterpret_cast<float4*>(&sm.sw[tid * 4]) = sw4;
        if (tid < T) sm.sx[tid] = a.sx_pre[tid];
        if (tid < kW16Cache) sm.idx[tid] = tid < o ? a.idx_pre[tid] : 0;
        for (int e = tid; e < T * OXL; e += kThreads) {
            const int t = e / OXL, j = e - t * OXL;
            sm.xo[t * OXL + j] = j < o ? h16_to_f32<HT>(a.xo_pre[(int64_t)t * opad + j]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const int i = tid + kThreads * u;
            if (i < nx) {
                const int t = i / pr, c = i - t * pr;
                *reinterpret_cast<uint4*>(&sm.xq[t * ldx + c * 16]) = xv[u];
            }
        }
        __syncthreads();   // the first outliers' dimensions are in LDS
        // cfirst[c] counts only the first kW16Cache outliers, the only ones
        // whose Int8 codes are picked out of the weight stream
        const int lim = o < kW16Cache ? o : kW16Cache;
        for (int c = tid; c <= cpb; c += kThreads) {
            int before = 0;
            for (int j = 0; j < lim; ++j) before += sm.idx[j] < kbase + c * kChunkK ? 1 : 0;
            sm.cfirst[c] = before;
        }
        __syncthreads();   // Xq, idx, xo, cfirst ready
    }
    // W16 values of the first outliers for the workgroup's rows, fetched now
    // (idx is complete only after the barrier above) so that the end of the
    // kernel does not wait on them: value q = tid + 512 h is outlier slot
    // q / kW16Pairs, row pair q % kW16Pairs; slots past o and rows past the
    // workgroup's read the first dword of W16 (never used).
    // Without W16 (memory-halved variant) nothing is fetched: the Int8 codes
    // of the outlier columns are picked out of the weight stream itself.
    uint32_t w16v[kW16PerThread] = {};
    const bool recover = a.w16 == nullptr;
    // with K slabs the outlier terms are added by k_decode_finish
    const bool split = PRE && a.slabs > 1;
    if (!recover && !split) {
#pragma unroll
        for (int h = 0; h < kW16PerThread; ++h) {
            const int q = tid + kThreads * h;
            const int j = q / kW16Pairs;
            const int r = 2 * (q % kW16Pairs);
            const int n = r < rows && nrow(r) < N ? nrow(r) : 0;
            const int64_t off = j < o ? (int64_t)sm.idx[j] * N + n : 0;
            w16v[h] = *reinterpret_cast<const uint32_t*>(a.w16 + off);
        }
    }
    if constexpr (!EARLY) issue(id1, ring[1]);

    // ---- stream the workgroup's chunks.  The loop body is unrolled over the
    // two ring slots (compile-time register indices) and every slot is
    // re-issued on every pass, with one exit test at the end: each path into
    // a slot's use then has the other slot's loads behind it, so the wait
    // before a chunk leaves them in flight.  A slot whose id is past the
    // end skips its MFMAs (a uniform branch with no loads inside).  A chunk's
    // next id is taken from the LDS counter before its MFMAs, used after them.
    const int tcol = lane & 15;                         // B column = activation row t
    const int8_t* xrow = &sm.xq[(tcol < T ? tcol : 0) * ldx + kl];
    // 16x16 accumulator layout: lane holds column lane%16 (t) and, in
    // register v, row 4*(lane/16) + v of the block
    int32_t* accrow = &sm.acc[0][4 * (lane >> 4)][tcol];
    auto consume = [&](int id, v4i (&buf)[kLoads]) -> int {
        if (id >= total) return total;
        int nid = 0;
        if (lane == 0) nid = atomicAdd(&sm.next, 1);
        const int8_t* xk = xrow + (id % cpb) * kChunkK;
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const v4i xb = tcol < T ? *reinterpret_cast<const v4i*>(xk + i * 64) : v4i{0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(buf[i], xb, acc, 0, 0, 0);
        }
        int32_t* d = accrow + (id / cpb) * (kRows * 16);
#pragma unroll
        for (int v = 0; v < 4; ++v) atomicAdd(d + v * 16, acc[v]);
        if (recover && !split) {
            // memory-halved variant: the chunk holds Wq[n, k] for its 16 rows
            // and 1024 columns; copy the codes of the outlier columns in it
            // (the first kW16Cache outliers) to LDS.  Column k sits in load
            // (k / 64) % 16, on lanes 16 ((k / 16) % 4) + row, byte k % 16.
            const int c = id % cpb;
            const int jhi = sm.cfirst[c + 1] < kW16Cache ? sm.cfirst[c + 1] : kW16Cache;
            for (int j = sm.cfirst[c]; j < jhi; ++j) {
                const int k = sm.idx[j] - kbase - c * kChunkK;
                const int ii = k >> 6;
                v4i v = buf[0];
#pragma unroll
                for (int m = 1; m < kLoads; ++m) v = ii == m ? buf[m] : v;
                const int b = k & 15;
                const int dw = (b >> 2) == 0 ? v[0] : (b >> 2) == 1 ? v[1] : (b >> 2) == 2 ? v[2] : v[3];
                if ((lane >> 4) == ((k >> 4) & 3))
                    sm.wqo[j][(id / cpb) * kRows + (lane & 15)] = (int8_t)(dw >> (8 * (b & 3)));
            }
        }
        return __builtin_amdgcn_readfirstlane(nid);
    };
    // ids increase in the order the slots are used (0, 1, 0, ...), so once
    // slot 0's next id is past the end every pending one is
    if (id0 < total) {
        do {
            id0 = consume(id0, ring[0]);
            issue(id0, ring[0]);
            id1 = consume(id1, ring[1]);
            issue(id1, ring[1]);
        } while (id0 < total);
    }
    if (!recover && !split) {
#pragma unroll
        for (int h = 0; h < kW16PerThread; ++h) {
            const int q = tid + kThreads * h;
            sm.w16o[q / kW16Pairs][q % kW16Pairs] = w16v[h];
        }
    }
    __syncthreads();   // sums and W16 values (or codes) complete
    if constexpr (PRE) {
        if (split) {
            // this slab's int32 sums of the workgroup's rows
            for (int e = tid; e < rows * T; e += kThreads) {
                const int r = e % rows, t = e / rows;
                const int n = nrow(r);
                if (n < N) a.part[((int64_t)slab * T + t) * N + n] = sm.acc[r >> 4][r & 15][t];
            }
            return;
        }
    }

    // ---- epilogue: y = acc * s_x * s_w / 127^2 + sum_j X[t, idx_j] W16[idx_j, n],
    // one fp16 rounding; consecutive threads take consecutive rows n.
    const int oc = o < kW16Cache ? o : kW16Cache;
    for (int e = tid; e < rows * T; e += kThreads) {
        const int r = e % rows, t = e / rows;
        const int n = nrow(r);
        if (n >= N) continue;
        const int32_t acc = sm.acc[r >> 4][r & 15][t];
        if (a.dbg_acc) a.dbg_acc[(int64_t)t * N + n] = acc;
        float y = (float)acc * sm.sx[t] * (sm.sw[r] * (1.0f / 16129.0f));
        if (!recover) {
            for (int j = 0; j < oc; ++j) {
                const uint32_t pr = sm.w16o[j][r >> 1];
                y += sm.xo[t * OXL + j] *
                     h16_to_f32<HT>((uint16_t)((r & 1) ? pr >> 16 : pr & 0xFFFFu));
            }
        } else {
            const float dr = sm.sw[r] / 127.0f;
            for (int j = 0; j < oc; ++j)
                y += sm.xo[t * OXL + j] *
                     h16_to_f32<HT>(recover_weight<HT>(sm.wqo[j][r], dr));
        }
        for (int j = oc; j < o; ++j) {
            const int k = PRE ? a.idx_pre[j] : sm.idx[j];
            const float xv = j < OXL ? sm.xo[t * OXL + j]
                             : PRE ? h16_to_f32<HT>(a.xo_pre[(int64_t)t * opad + j])
                                   : h16_to_f32<HT>(a.x[(int64_t)t * K + k]);
            const uint16_t w = recover ? recover_weight<HT>(a.wq[blk_offset(n, k, N, K)], sm.sw[r] / 127.0f)
                                       : a.w16[(int64_t)k * N + n];
            y += xv * h16_to_f32<HT>(w);
        }
        a.y[(int64_t)t * N + n] = f32_to_h16<HT>(y);
    }
}

// Completes a call whose K was cut into slabs: acc = the sum of the slabs'
// int32 partial sums (exact, in any order), then the decode kernel's
// epilogue, y = acc * s_x * s_w / 127^2 + sum_j X[t, idx_j] W16[idx_j, n]
// rounded once.  One thread per output (t, n): grid (N / 256, T), so the
// partial sums are read coalesced along n and enough workgroups are in
// flight to hide their latency; the W16 rows (or, memory-halved variant,
// the Int8 codes the weight is recovered from) are read once per t, from
// L2 after the first.
template <int HT>
__global__ __launch_bounds__(256) void k_decode_finish(DecodeArgs a) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int t = blockIdx.y;
    const int T = a.T, K = a.K, N = a.N;
    if (n >= N) return;
    const int o = a.count_pre[0], opad = a.count_pre[1];
    const float swn = a.sw[n];
    const bool recover = a.w16 == nullptr;
    const float dr = swn / 127.0f;
    const int32_t* p = a.part + (int64_t)t * N + n;
    const int64_t sstride = (int64_t)T * N;
    int32_t acc = 0;
#pragma unroll 4
    for (int sl = 0; sl < a.slabs; ++sl) acc += p[sl * sstride];
    if (a.dbg_acc) a.dbg_acc[(int64_t)t * N + n] = acc;
    float y = (float)acc * a.sx_pre[t] * (swn * (1.0f / 16129.0f));
    const uint16_t* xo = a.xo_pre + (int64_t)t * opad;
    for (int j = 0; j < o; ++j) {
        const int k = a.idx_pre[j];
        const uint16_t w = recover ? recover_weight<HT>(a.wq[blk_offset(n, k, N, K)], dr)
                                   : a.w16[(int64_t)k * N + n];
        y += h16_to_f32<HT>(xo[j]) * h16_to_f32<HT>(w);
    }
    a.y[(int64_t)t * N + n] = f32_to_h16<HT>(y);
}

}  // namespace

// Bits of the smallest 16-bit value (binary16, or bfloat16 for ht = bf16)
// >= tau (tau >= 0 and not NaN), or the +inf pattern when no finite value
// reaches tau.  Found by a binary search over the non-negative bit patterns,
// whose unsigned order is the numeric order; both widenings to fp32 are
// exact.
uint32_t tau_to_h16_ceil(float tau, int ht) {
    const uint32_t inf = ht == kHalfBF16 ? 0x7F80u : 0x7C00u;
    uint32_t lo = 0, hi = inf;   // answer in [lo, hi]
    while (lo < hi) {
        const uint32_t mid = (lo + hi) / 2;
        const float v = ht == kHalfBF16 ? __builtin_bit_cast(float, mid << 16)
                                        : (float)__builtin_bit_cast(_Float16, (uint16_t)mid);
        if (v >= tau) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

hipError_t launch_finish_partials(int ht, int64_t T, int64_t K, int64_t N, int slabs,
                                  const int32_t* part, const int8_t* Wq, const float* sw,
                                  const uint16_t* W16, const float* sx, const int32_t* count,
                                  const int32_t* idx, const uint16_t* xo, uint16_t* Y,
                                  int32_t* dbg_acc, hipStream_t stream) {
    DecodeArgs a{};
    a.wq = Wq;
    a.sw = sw;
    a.w16 = W16;
    a.y = Y;
    a.T = (int)T;
    a.K = (int)K;
    a.N = (int)N;
    a.sx_pre = sx;
    a.count_pre = count;
    a.idx_pre = idx;
    a.xo_pre = xo;
    a.slabs = slabs;
    a.part = const_cast<int32_t*>(part);
    a.dbg_acc = dbg_acc;
    const dim3 fgrid((unsigned)ceil_div(N, 256), (unsigned)T);
    if (ht == kHalfBF16)
        hipLaunchKernelGGL(k_decode_finish<kHalfBF16>, fgrid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_decode_finish<kHalfF16>, fgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

bool decode_path_supported(int64_t T, int64_t K, int64_t N) {
    (void)N;
    return T >= 1 && T <= kMaxT && (K == 4096 || K == 8192) && T * K <= kMaxXK;
}

// Compute units of the current device, cached per device (an immutable
// property; concurrent first calls store the same value).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// One instantiation per 16-bit type and LDS size (the smaller one whenever
// the workgroup owns at most kSmallBpw blocks).
template <int CPB, bool PRE, bool EARLY>
static void launch_k2(int ht, const DecodeArgs& a, unsigned grid, hipStream_t stream) {
    const bool small = a.bpw <= kSmallBpw;
    if (ht == kHalfBF16) {
        if (small)
            hipLaunchKernelGGL((k_decode<CPB, kHalfBF16, PRE, kSmallBpw, EARLY>), dim3(grid), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((k_decode<CPB, kHalfBF16, PRE, kMaxBpw, EARLY>), dim3(grid), dim3(kThreads), 0, stream, a);
    } else {
        if (small)
            hipLaunchKernelGGL((k_decode<CPB, kHalfF16, PRE, kSmallBpw, EARLY>), dim3(grid), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((k_decode<CPB, kHalfF16, PRE, kMaxBpw, EARLY>), dim3(grid), dim3(kThreads), 0, stream, a);
    }
}
// The early second chunk for K = 8192 when a workgroup has more chunks than
// the 16 its waves start with (in-kernel prologue only).  Measured per call
// against the late issue: K = 8192, N = 28672 with T = 8 and 1 and N = 36864
// with T = 8 -0.8 to -1.2%; at K = 4096 T = 2, N = 36864 -1.4% but T = 4,
// N = 49152 +2.7%, so K = 4096 keeps the late issue.
template <int CPB, bool PRE>
static void launch_k(int ht, const DecodeArgs& a, unsigned grid, hipStream_t stream) {
    if constexpr (!PRE && CPB == 8) {
        if ((int64_t)a.bpw * CPB > 2 * kWaves) {
            launch_k2<CPB, PRE, true>(ht, a, grid, stream);
            return;
        }
    }
    launch_k2<CPB, PRE, false>(ht, a, grid, stream);
}

// Which blocks a workgroup owns.  Measured per call (alternated, one box,
// Y bit-identical): with 12 blocks per workgroup (N = 49152, and the K-slab
// plans that give 12 per group), owning blocks g, g + groups, ... instead of
// 12 consecutive ones was faster on 12 of 13 shapes (K = 4096 T = 1..16
// -15 to -16.5%, K = 5120 -8.5%, K = 12288 -11 to -12%, K = 16384 -5.7%,
// T = 8 and 16 with K = 49152, N = 12288 in slabs -11% and -5%; T = 12,
// K = 32768, N = 12288 in slabs +2.9%); with 7, 9 or 11 blocks it was
// slower on the decode workload (+10.6%) and mixed elsewhere (-9% to +8%),
// so only the 12-block split interleaves.
static int interleave_blocks(int bpw) { return bpw == kMaxBpw ? 1 : 0; }

hipError_t launch_decode(const uint16_t* X, int ht, int64_t T, int64_t K, const int8_t* Wq,
                         const float* sw, const uint16_t* W16, int64_t N, float tau,
                         uint16_t* Y, int32_t* dbg_count, int32_t* dbg_idx, int8_t* dbg_xq,
                         float* dbg_sx, int32_t* dbg_acc, hipStream_t stream) {
    // One workgroup per compute unit (the LDS footprint allows no more), each
    // owning bpw whole 16-row blocks: bpw = ceil(blocks / CUs) spreads the
    // weight evenly (N = 28672: 1792 blocks = 256 CUs x 7; N = 49152: x 12);
    // past kMaxBpw blocks per CU the grid grows instead.
    const int64_t nblocks = ceil_div(N, kRows);
    const int bpw = (int)std::min<int64_t>(kMaxBpw, std::max<int64_t>(1, ceil_div(nblocks, device_cus())));
    DecodeArgs a{X, Wq, sw, W16, Y, tau, tau_to_h16_ceil(tau, ht), (int)T, (int)K, (int)N, bpw,
                 interleave_blocks(bpw), (int)(K / kChunkK), nullptr, nullptr, nullptr, nullptr, nullptr,
                 1, (int)(K / kChunkK), nullptr,
                 dbg_count, dbg_idx, dbg_xq, dbg_sx, dbg_acc};
    const unsigned grid = (unsigned)ceil_div(nblocks, bpw);
    if (K != 4096 && K != 8192) return hipErrorInvalidValue;
    if (K == 4096) launch_k<4, false>(ht, a, grid, stream);
    else launch_k<8, false>(ht, a, grid, stream);
    return hipGetLastError();
}

// Which few-row shapes the decode kernel's precomputed mode takes.  Past 8
// rows the streaming matmul kernel is faster unless K is long (measured,
// whole calls: T=9..16 with K=8192, N=28672 2.5-4 us faster on the matmul;
// T=12 and 16 with K=12288 and 16384 2-15 us faster; T=8..16 with K=49152,
// N=12288 the K slabs 8-17 us faster; T=1..8 with K=12288 the precomputed
// mode 1-5 us faster).
constexpr int kMaxTPre = 8;                 // rows of the precomputed mode without slabs
constexpr int64_t kSlabLongK = 32768;       // K from which 9..16 rows take the slabs

bool decode_pre_supported(int64_t T, int64_t K, int64_t N) {
    (void)N;
    return T >= 1 && T <= kMaxTPre && K % kChunkK == 0 && T * K <= kMaxXKPre;
}

hipError_t launch_decode_pre(int ht, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                             const uint16_t* W16, int64_t N, uint16_t* Y, const Workspace& ws,
                             int32_t* dbg_acc, hipStream_t stream) {
    if (!decode_pre_supported(T, K, N)) return hipErrorInvalidValue;
    const int64_t nblocks = ceil_div(N, kRows);
    const int bpw = (int)std::min<int64_t>(kMaxBpw, std::max<int64_t>(1, ceil_div(nblocks, device_cus())));
    DecodeArgs a{nullptr, Wq, sw, W16, Y, 0.0f, 0u, (int)T, (int)K, (int)N, bpw,
                 interleave_blocks(bpw), (int)(K / kChunkK), ws.xq, ws.sx, ws.count, ws.idx, ws.xo,
                 1, (int)(K / kChunkK), nullptr,
                 nullptr, nullptr, nullptr, nullptr, dbg_acc};
    const unsigned grid = (unsigned)ceil_div(nblocks, bpw);
    launch_k<0, true>(ht, a, grid, stream);
    return hipGetLastError();
}

// K slabs for T <= 16 rows whose Xq exceeds the LDS room: at least
// smin = ceil(chunks / most chunks per slab) slabs; up to three more are
// tried, each with bpw = the blocks per workgroup that fill the chip once,
// and the one with the least weight per compute unit (rounds of the grid x
// the rows and k of one workgroup) wins.  The workspace holds smin + 3.
namespace {
struct SlabPlan {
    int slabs, cps, bpw;
};
int split_smin(int64_t T, int64_t K) {
    const int64_t chunks = K / kChunkK;
    const int64_t per = kMaxXKPre / (T * kChunkK);   // >= 8 for T <= 16
    return (int)ceil_div(chunks, per);
}
SlabPlan plan_slabs(int64_t T, int64_t K, int64_t N, int reserve) {
    const int64_t chunks = K / kChunkK;
    const int64_t nblocks = ceil_div(N, kRows);
    const int64_t cus = device_cus();
    SlabPlan best{0, 0, 0};
    int64_t best_cost = 0;
    for (int s = split_smin(T, K); s <= reserve; ++s) {
        const int64_t cps = ceil_div(chunks, s);
        const int64_t se = ceil_div(chunks, cps);   // slabs actually used
        const int64_t bpw = std::min<int64_t>(kMaxBpw, std::max<int64_t>(1, ceil_div(nblocks * se, cus)));
        const int64_t grid = ceil_div(nblocks, bpw) * se;
        const int64_t cost = ceil_div(grid, cus) * bpw * cps;
        if (best.slabs == 0 || cost < best_cost) {
            best = SlabPlan{(int)se, (int)cps, (int)bpw};
            best_cost = cost;
        }
    }
    return best;
}
}  // namespace

int decode_split_reserve(int64_t T, int64_t K, int64_t N) {
    (void)N;
    if (!(T >= 1 && T <= kMaxT && K % kChunkK == 0 && T * K > kMaxXKPre)) return 0;
    if (T > kMaxTPre && K < kSlabLongK) return 0;
    return (int)std::min<int64_t>(split_smin(T, K) + 3, K / kChunkK);
}

hipError_t launch_decode_split(int ht, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                               const uint16_t* W16, int64_t N, uint16_t* Y, const Workspace& ws,
                               int32_t* dbg_acc, hipStream_t stream) {
    const int reserve = decode_split_reserve(T, K, N);
    if (reserve == 0 || !ws.dpart || ws.dslabs < reserve) return hipErrorInvalidValue;
    const SlabPlan p = plan_slabs(T, K, N, reserve);
    const int64_t nblocks = ceil_div(N, kRows);
    DecodeArgs a{nullptr, Wq, sw, W16, Y, 0.0f, 0u, (int)T, (int)K, (int)N, p.bpw,
                 interleave_blocks(p.bpw), (int)(K / kChunkK), ws.xq, ws.sx, ws.count, ws.idx, ws.xo,
                 p.slabs, p.cps, ws.dpart,
                 nullptr, nullptr, nullptr, nullptr, dbg_acc};
    const unsigned grid = (unsigned)(ceil_div(nblocks, p.bpw) * p.slabs);
    launch_k<0, true>(ht, a, grid, stream);
    const dim3 fgrid((unsigned)ceil_div(N, 256), (unsigned)T);
    if (ht == kHalfBF16)
        hipLaunchKernelGGL(k_decode_finish<kHalfBF16>, fgrid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(k_decode_finish<kHalfF16>, fgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace i8mm
