// Allocation-free entry point: int8_mixed_matmul with the library's own
// scratch buffer as its workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Declared in include/int8mm.h.
//
// The scratch is a file-scope device array of kScratchBytes; every GPU the
// library runs this entry point on holds its own copy until the process
// ends.  Its device address is looked up once per device (the first call on
// that device, with the device current) and kept; in host code the array's
// name is only a host-side stand-in, never passed to a kernel.  Calls on
// one GPU share the array, so calls that overlap on one GPU race.  Every
// kernel writes what it reads of the workspace before reading it (bitmap
// words, counters and partial sums are cleared or stored whole inside each
// call), so the previous call's contents do not matter.
#include <math.h>

#include <mutex>

#include "../../include/int8mm.h"
#include "common.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // 128 MiB per device
constexpr int kMaxDevices = 256;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int scratch_pointer(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return INT8MM_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return INT8MM_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return INT8MM_E_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return INT8MM_OK;
}

}  // namespace

extern "C" int int8_mixed_matmul_noalloc(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                         const float* sw, const void* W16, int64_t N, float tau,
                                         void* Y, void* stream) {
    // the checks that need no device come first, in the order of the
    // regular entry point, then the scratch size
    if (!X || !Wq || !sw || !Y) return INT8MM_E_NULL;
    size_t need = 0;
    int st = int8_mixed_matmul_workspace_size(T, K, N, &need);   // shape limits
    if (st) return st;
    if (isnan(tau) || tau < 0.0f) return INT8MM_E_TAU;
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!a16(X) || !a16(Wq) || !a16(sw) || !a16(Y) || (W16 && !a16(W16))) return INT8MM_E_ALIGN;
    if (i8mm::carve_workspace(nullptr, T, K, N, false, 1).bytes > kScratchBytes)
        return INT8MM_E_WORKSPACE;
    void* ws = nullptr;
    st = scratch_pointer(&ws);
    if (st) return st;
    // the regular entry point on the scratch: it takes the optional
    // workspace regions that fit, and allocates nothing
    return int8_mixed_matmul(X, T, K, Wq, sw, W16, N, tau, Y, ws, kScratchBytes, stream);
}
