// C ABI of libint8mm (declared in include/int8mm.h): host-side argument
// validation, workspace layout and the launch sequence of each entry point.
// No entry point allocates, frees or synchronizes.
#include <math.h>

#include "../../include/int8mm.h"
#include "common.hpp"

using namespace i8mm;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int64_t T, int64_t K, int64_t N) {
    if (T < 1 || K < 1 || N < 1) return INT8MM_E_SHAPE;
    if (K % 16 != 0 || N % 8 != 0 || K > INT8MM_MAX_K) return INT8MM_E_SHAPE;
    // launch limits: one workgroup of 256 lanes per row in the quantize pass
    // and per 128x128 output tile in the matmul keep every grid below 2^32
    // work-items
    if (T > INT8MM_MAX_T || (double)T * (double)N > INT8MM_MAX_TN) return INT8MM_E_SHAPE;
    return INT8MM_OK;
}

int check_tau(float tau) {
    if (isnan(tau) || tau < 0.0f) return INT8MM_E_TAU;
    return INT8MM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? INT8MM_OK : INT8MM_E_HIP; }

// Optional workspace regions in use: for few rows with a long K (decode
// shapes whose Xq exceeds the decode kernel's LDS) the K-slab partial sums;
// otherwise the recovered outlier rows of the memory-halved variant, then
// the matmul's K split (gemm_ksplit); each only when the workspace is large
// enough for it.  The size query reserves what applies, and every entry
// point decides the same way from the same (T, K, N, workspace_bytes), so
// calls on one workspace always agree on its layout.
Workspace layout_for(void* base, int64_t T, int64_t K, int64_t N, size_t workspace_bytes) {
    const int ds = decode_split_reserve(T, K, N);
    if (ds > 0 && workspace_bytes >= carve_workspace(nullptr, T, K, N, false, 1, ds).bytes)
        return carve_workspace(base, T, K, N, false, 1, ds);
    const bool wrec = workspace_bytes >= carve_workspace(nullptr, T, K, N, true, 1).bytes;
    const int want = gemm_ksplit(T, K, N);
    const int ks = wrec && want >= 2 &&
                           workspace_bytes >= carve_workspace(nullptr, T, K, N, true, want).bytes
                       ? want
                       : 1;
    return carve_workspace(base, T, K, N, wrec, ks);
}

// Steps 3-4 on a prepared workspace.  Few rows (T <= 8, or T <= 16 with a
// long K) stream the weight
// through the decode kernel's precomputed mode (with K slabs when Xq is long
// and the workspace has their region); otherwise the GEMM runs, and without
// W16 (memory-halved variant) the outlier rows are first recovered into the
// workspace when it has room.  ks_zeroed: the K-split tile counters were set
// to zero by this call's activation pass.
int run_prepared(const Workspace& ws, int ht, int64_t T, int64_t K, const int8_t* Wq,
                 const float* sw, const uint16_t* w16, int64_t N, uint16_t* y16, int32_t* acc,
                 hipStream_t stream, bool ks_zeroed = false) {
    if (decode_pre_supported(T, K, N))
        return hip_status(launch_decode_pre(ht, T, K, Wq, sw, w16, N, y16, ws, acc, stream));
    if (ws.dpart)
        return hip_status(launch_decode_split(ht, T, K, Wq, sw, w16, N, y16, ws, acc, stream));
    const uint16_t* rows = w16;
    int64_t nrows = 0;
    if (!w16 && ws.wrec) {
        hipError_t e = launch_recover_rows(Wq, sw, ws.idx, ws.count, K, N, ht, ws.wrec,
                                           ws.wrec_rows, stream);
        if (e != hipSuccess) return INT8MM_E_HIP;
        rows = ws.wrec;
        nrows = ws.wrec_rows;
    }
    GemmArgs g{ws.xq, ws.sx, Wq, sw, ws.xo, ws.idx, ws.count, rows, nrows, y16, acc, T, K, N,
               ws.ks_count ? gemm_ksplit(T, K, N) : 1, ws.ks_count, ws.ks_part, 0, ks_zeroed ? 1 : 0};
    return hip_status(launch_gemm(g, ht, stream));
}

// Validation shared by int8_mixed_matmul and its debug variant.
int check_matmul(const void* X, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                 const void* W16, int64_t N, float tau, void* Y, void* workspace,
                 size_t workspace_bytes) {
    if (!X || !Wq || !sw || !Y || !workspace) return INT8MM_E_NULL;
    int st = check_shape(T, K, N);
    if (st) return st;
    st = check_tau(tau);
    if (st) return st;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(sw) || !aligned16(Y) ||
        !aligned16(workspace) || (W16 && !aligned16(W16)))
        return INT8MM_E_ALIGN;
    if (workspace_bytes < carve_workspace(nullptr, T, K, N, false, 1).bytes)
        return INT8MM_E_WORKSPACE;
    return INT8MM_OK;
}

// ht: 16-bit type of X, W16 and Y (kHalfF16, or kHalfBF16 for the bf16 variant)
int run_matmul(const void* X, int ht, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
               const void* W16, int64_t N, float tau, void* Y, void* workspace,
               size_t workspace_bytes, hipStream_t stream, int32_t* count, int32_t* idx,
               int8_t* xq, float* sx, int32_t* acc) {
    const uint16_t* x16 = static_cast<const uint16_t*>(X);
    const uint16_t* w16 = static_cast<const uint16_t*>(W16);
    uint16_t* y16 = static_cast<uint16_t*>(Y);
    if (decode_path_supported(T, K, N))
        return hip_status(launch_decode(x16, ht, T, K, Wq, sw, w16, N, tau, y16, count, idx, xq,
                                        sx, acc, stream));
    Workspace ws = layout_for(workspace, T, K, N, workspace_bytes);
    // with the K split (more than 128 rows) the activation pass zeroes the
    // matmul's tile counters, one launch fewer
    const int64_t ntiles = ws.ks_count ? gemm_ksplit_plan(T, K, N).nsplit : 0;
    hipError_t e = launch_activation_pass(x16, ht, T, K, tau, ws, stream, ws.ks_count, ntiles);
    if (e != hipSuccess) return INT8MM_E_HIP;
    const int st = run_prepared(ws, ht, T, K, Wq, sw, w16, N, y16, acc, stream, ntiles > 0);
    if (st) return st;
    return hip_status(launch_debug_copies(ws, T, K, count, idx, xq, sx, stream));
}

}  // namespace

extern "C" {

const char* int8mm_status_string(int status) {
    switch (status) {
        case INT8MM_OK: return "ok";
        case INT8MM_E_NULL: return "a required pointer is NULL";
        case INT8MM_E_SHAPE: return "shape outside the supported limits";
        case INT8MM_E_TAU: return "tau is NaN or negative";
        case INT8MM_E_ALIGN: return "a pointer is not 16-byte aligned";
        case INT8MM_E_WORKSPACE: return "workspace too small";
        case INT8MM_E_UNSUPPORTED: return "unsupported request";
        case INT8MM_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int int8_mixed_matmul_workspace_size(int64_t T, int64_t K, int64_t N, size_t* bytes) {
    if (!bytes) return INT8MM_E_NULL;
    int st = check_shape(T, K, N);
    if (st) return st;
    // the single-kernel decode path uses no workspace regions beyond the
    // fixed ones (which int8mm_quantize_activations still needs); decode
    // shapes with a long K take the K-slab partial sums instead of the
    // matmul's regions
    const int ds = decode_split_reserve(T, K, N);
    const bool gemm = !decode_path_supported(T, K, N) && ds == 0;
    *bytes = carve_workspace(nullptr, T, K, N, gemm, gemm ? gemm_ksplit(T, K, N) : 1, ds).bytes;
    return INT8MM_OK;
}

int int8_quantize_weight_size(int64_t K, int64_t N, size_t* bytes) {
    if (!bytes) return INT8MM_E_NULL;
    int st = check_shape(1, K, N);
    if (st) return st;
    *bytes = (size_t)wq_bytes(K, N);
    return INT8MM_OK;
}

int int8_quantize_weight_typed(const void* W, int wtype, int64_t K, int64_t N, int8_t* Wq,
                               float* sw, void* W16_out, void* stream) {
    static_assert(INT8MM_WEIGHT_F16 == kWeightF16 && INT8MM_WEIGHT_BF16 == kWeightBF16 &&
                      INT8MM_WEIGHT_F32 == kWeightF32,
                  "weight type codes");
    if (!W || !Wq || !sw) return INT8MM_E_NULL;
    int st = check_shape(1, K, N);
    if (st) return st;
    if (wtype != INT8MM_WEIGHT_F16 && wtype != INT8MM_WEIGHT_BF16 && wtype != INT8MM_WEIGHT_F32)
        return INT8MM_E_UNSUPPORTED;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(sw) || (W16_out && !aligned16(W16_out)))
        return INT8MM_E_ALIGN;
    return hip_status(launch_quantize_weight(W, wtype, K, N, Wq, sw,
                                             static_cast<_Float16*>(W16_out),
                                             static_cast<hipStream_t>(stream)));
}

int int8_quantize_weight(const void* W16, int64_t K, int64_t N, int8_t* Wq, float* sw,
                         void* stream) {
    return int8_quantize_weight_typed(W16, INT8MM_WEIGHT_F16, K, N, Wq, sw, nullptr, stream);
}

int int8_mixed_matmul(const void* X, int64_t T, int64_t K, const int8_t* Wq, const float* sw,
                      const void* W16, int64_t N, float tau, void* Y, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int st = check_matmul(X, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes);
    if (st) return st;
    return run_matmul(X, kHalfF16, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, nullptr,
                      nullptr);
}

int int8_mixed_matmul_bf16(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                           const float* sw, const void* W16, int64_t N, float tau, void* Y,
                           void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_matmul(X, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes);
    if (st) return st;
    return run_matmul(X, kHalfBF16, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, nullptr,
                      nullptr);
}

static int matmul_debug(int ht, const void* X, int64_t T, int64_t K, const int8_t* Wq,
                        const float* sw, const void* W16, int64_t N, float tau, void* Y,
                        void* workspace, size_t workspace_bytes, void* stream, int32_t* count,
                        int32_t* idx, int8_t* xq, float* sx, int32_t* acc) {
    int st = check_matmul(X, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes);
    if (st) return st;
    if ((count && !aligned16(count)) || (idx && !aligned16(idx)) || (xq && !aligned16(xq)) ||
        (sx && !aligned16(sx)) || (acc && !aligned16(acc)))
        return INT8MM_E_ALIGN;
    return run_matmul(X, ht, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream), count, idx, xq, sx, acc);
}

int int8_mixed_matmul_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                            const float* sw, const void* W16, int64_t N, float tau, void* Y,
                            void* workspace, size_t workspace_bytes, void* stream,
                            int32_t* count, int32_t* idx, int8_t* xq, float* sx, int32_t* acc) {
    return matmul_debug(kHalfF16, X, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes,
                        stream, count, idx, xq, sx, acc);
}

int int8_mixed_matmul_bf16_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                 const float* sw, const void* W16, int64_t N, float tau, void* Y,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t* count, int32_t* idx, int8_t* xq, float* sx,
                                 int32_t* acc) {
    return matmul_debug(kHalfBF16, X, T, K, Wq, sw, W16, N, tau, Y, workspace, workspace_bytes,
                        stream, count, idx, xq, sx, acc);
}

int int8mm_quantize_activations(const void* X, int64_t T, int64_t K, int64_t N, float tau,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!X || !workspace) return INT8MM_E_NULL;
    int st = check_shape(T, K, N);
    if (st) return st;
    st = check_tau(tau);
    if (st) return st;
    if (!aligned16(X) || !aligned16(workspace)) return INT8MM_E_ALIGN;
    if (workspace_bytes < carve_workspace(nullptr, T, K, N, false, 1).bytes)
        return INT8MM_E_WORKSPACE;
    Workspace ws = layout_for(workspace, T, K, N, workspace_bytes);
    return hip_status(launch_activation_pass(static_cast<const uint16_t*>(X), kHalfF16, T, K, tau, ws,
                                             static_cast<hipStream_t>(stream)));
}

int int8mm_matmul_prepared(void* workspace, size_t workspace_bytes, int64_t T, int64_t K,
                           const int8_t* Wq, const float* sw, const void* W16, int64_t N,
                           void* Y, void* stream) {
    if (!workspace || !Wq || !sw || !Y) return INT8MM_E_NULL;
    int st = check_shape(T, K, N);
    if (st) return st;
    if (!aligned16(workspace) || !aligned16(Wq) || !aligned16(sw) || !aligned16(Y) ||
        (W16 && !aligned16(W16)))
        return INT8MM_E_ALIGN;
    if (workspace_bytes < carve_workspace(nullptr, T, K, N, false, 1).bytes)
        return INT8MM_E_WORKSPACE;
    Workspace ws = layout_for(workspace, T, K, N, workspace_bytes);
    return run_prepared(ws, kHalfF16, T, K, Wq, sw, static_cast<const uint16_t*>(W16), N,
                    static_cast<uint16_t*>(Y), nullptr, static_cast<hipStream_t>(stream));
}

}  // extern "C"
