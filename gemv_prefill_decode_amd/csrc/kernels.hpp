// Host-side launchers implemented by the kernel translation units.  Each one
// assumes its arguments were validated by qmm_api.cpp and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// Launch-shape choices for the streaming (GEMV / MoE / load-only) kernels.
struct GemvTuning {
    int num_cu;     // compute units of the device
    int wg_per_cu;  // work groups per CU the grid is sized for
    int rows;       // rows per lane group (1 or 2)
    int depth;      // items of weight loads kept in flight per wave (2, 4 or 8)
    int lds_per_wg; // bytes of LDS one work group may allocate
    int lds_per_cu; // bytes of LDS per CU (limits resident work groups)
};

void launch_gemv(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                 int qt, int64_t rb, const GemvTuning& tune, hipStream_t st);

// Launch plan of the MFMA kernel: k split into n_split ranges of sps steps
// (64 k each; sps even), and the workspace bytes that needs (0 if n_split = 1).
struct MfmaPlan {
    int n_split;
    int sps;
    int64_t ws_bytes;
};

// Floats between consecutive k splits' partial results in the workspace:
// n*m rounded up to a multiple of 64 (256 bytes).
__host__ __device__ constexpr int64_t splitk_stride(int64_t n, int64_t m) { return (n * m + 63) / 64 * 64; }

// The plan for an m x k x n product on a device with num_cu compute units.
MfmaPlan plan_gemm_mfma(int64_t m, int64_t k, int64_t n, int num_cu);

// Launch with plan pl; ws (256-byte aligned, pl.ws_bytes) holds the k
// splits' partial results when pl.n_split > 1 (then two kernels are launched).
void launch_gemm_mfma(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int qt, int64_t rb, const MfmaPlan& pl, void* ws, hipStream_t st);

void launch_moe(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                const int* ids, const float* scale, const float* x, int64_t t, int64_t n_used,
                int64_t n_expert, int64_t in_f, int64_t n_ff, int qt, int64_t rb,
                const GemvTuning& tune, hipStream_t st);

void launch_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k, int qt, int64_t rb,
                     const GemvTuning& tune, hipStream_t st);

// Largest byte window (relative to a 16-byte-aligned base) one GEMV work
// group addresses, for the host's 32-bit offset check.
int64_t gemv_max_window_bytes(int qt, int64_t k, int64_t rb);
int gemv_unit_elems(int qt);

// Tile sizes of the MFMA kernel (rows of W, tokens) for the host's checks.
constexpr int MFMA_BM = 128;
constexpr int MFMA_BN = 128;

}  // namespace qmm
