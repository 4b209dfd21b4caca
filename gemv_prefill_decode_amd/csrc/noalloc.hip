// qmm_gemm_noalloc: qmm_gemm_ws whose workspace is the library's own device
// array instead of caller memory, for callers that cannot allocate (code
// under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below lives in this code object's device memory: each
// GPU the library runs on holds its own copy, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address, so it is never passed to a kernel or a runtime call: the
// first call on each device looks up that device's address once with
// hipGetSymbolAddress (with the device current) and every later call passes
// that pointer as the workspace.  Nothing here allocates.
#include "qmm.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr int64_t SCRATCH_BYTES = (int64_t)64 << 20;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[MAX_DEVICES];

// This device's address of `scratch`, or null if the runtime cannot give it.
void* scratch_ptr(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();  // leave no sticky error for the next call
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

int64_t qmm_gemm_noalloc_max_bytes(void) { return SCRATCH_BYTES; }

int qmm_gemm_noalloc(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qtype,
                     int path, hipStream_t stream) {
    if (!dst || !w || !x) return QMM_ERR_NULL;
    // the plan's workspace size (also validates qtype, sizes and path)
    const int64_t need = qmm_gemm_workspace_bytes(m, k, n, qtype, path);
    if (need < 0) return (int)-need;
    if (need > SCRATCH_BYTES) return QMM_ERR_SCRATCH;
    if (need == 0) return qmm_gemm_ws(dst, w, x, m, k, n, qtype, path, nullptr, 0, stream);  // GEMV
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        return QMM_ERR_LAUNCH;
    }
    void* ws = scratch_ptr(dev);
    if (!ws) return QMM_ERR_LAUNCH;
    return qmm_gemm_ws(dst, w, x, m, k, n, qtype, path, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"
