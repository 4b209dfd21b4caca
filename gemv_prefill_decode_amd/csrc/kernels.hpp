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
};

void launch_gemv(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                 int qt, int64_t rb, const GemvTuning& tune, hipStream_t st);

void launch_gemm_mfma(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int qt, int64_t rb, hipStream_t st);

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
