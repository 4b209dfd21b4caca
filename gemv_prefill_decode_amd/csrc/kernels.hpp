// Host-side launchers implemented by the kernel translation units.  Each one
// assumes its arguments were validated by qmm_api.cpp and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// Launch-shape choices for the streaming (GEMV / MoE / load-only) kernels.
// log2 of the largest lane group per weight row in the streams that apply
// each weight to several activation rows (the GEMV at n > 2 and the MoE), and
// the smallest value the MoE tuning may set (the row windows' range checks
// assume it)
constexpr int LPR_CAP_MULTI = 4, LPR_CAP_MIN = 3;

struct GemvTuning {
    int num_cu;     // compute units of the device
    int wg_per_cu;  // work groups per CU the grid is sized for
    int moe_wg_per_cu;  // the same for the MoE kernels
    int rows;       // rows per lane group (1 or 2)
    int depth;      // items of weight loads kept in flight per wave (2, 4 or 8)
    int moe_lpr_cap;  // log2 of the largest lane group per row in the MoE streams
    int moe_mfma_min; // MoE chunks of at least this many pairs use the matrix-core stream (0: never)
    int gemv_mfma_min; // GEMV calls with at least this many activation rows use it (0: never)
    int gemv_mfma_tt;  // its token groups: 4 * gemv_mfma_tt rows at most (1 or 2)
    int lds_per_wg; // bytes of LDS one work group may allocate
    int lds_per_cu; // bytes of LDS per CU (limits resident work groups)
};

// x rows are ldx floats apart (ldx >= k, a multiple of 4), dst rows ldd
// floats apart (ldd >= m); ldx = k and ldd = m for contiguous tensors.
// The GEMV's two streams: f32 products on FMAs, or on the matrix cores
// (v_mfma_f32_4x4x1f32); GEMV_AUTO takes the matrix cores for n >=
// tune.gemv_mfma_min.  Both stage the activations in LDS where they fit; the
// matrix-core stream needs 4 rows of them in one work group's LDS and falls
// back to the FMA stream otherwise.
enum : int { GEMV_AUTO = 0, GEMV_FMA = 1, GEMV_MATRIX = 2 };
void launch_gemv(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                 int qt, int64_t rb, int64_t ldx, int64_t ldd, int kind, const GemvTuning& tune, hipStream_t st);
// Activation rows per token group of the matrix-core stream for this call
// (4 or 8), or 0 if the FMA stream runs it.
int gemv_matrix_tokens(int64_t m, int64_t k, int64_t n, int qt, int kind, const GemvTuning& tune);

// Launch plan of the prefill (MFMA) kernels.  x16 = 0: gemm_mfma.hip's
// kernel (128 x 128 tiles, f32 activations converted in the k loop).
// x16 = 2: gemm_lds.hip's kernel ((64*wm) x 128 tiles; f16 activations from
// its own pre-pass, weight bytes and activations streamed through an LDS
// ring; k % 64 == 0 only); x16 = 3: the same kernel with 128 x 256 tiles
// (wm = 2); x16 = 5: with 64 x 64 tiles (wm = 1: twice the work groups of
// 64 x 128 tiles for products of few tiles); x16 = 6: 64 x 64 tiles on the
// f32 activations (as x16 = 4).  x16 = 4: the same kernel with 128 x 128 tiles reading the f32
// activations into its ring and rounding them as it reads (no pre-pass, no
// f16 workspace).  kg = 2: two groups of 4 waves take alternate k steps of
// each tile.  Any of them may split k into n_split ranges of sps steps (64 k
// each; sps even) whose partial results go to the workspace (after the f16
// activations), summed by a second kernel.  (x16 = 1 is not used.)
struct MfmaPlan {
    int x16;
    int wm;
    int kg;  // k groups per work group (1 or 2)
    int n_split;
    int sps;
    int64_t ws_bytes;
};

// Floats between consecutive k splits' partial results in the workspace:
// n*m rounded up to a multiple of 64 (256 bytes).
__host__ __device__ constexpr int64_t splitk_stride(int64_t n, int64_t m) { return (n * m + 63) / 64 * 64; }

// Halves per row of the f16 activations: k rounded up to whole 64-k steps.
__host__ __device__ constexpr int64_t x16_row_halves(int64_t k) { return (k + 63) / 64 * 64; }

// Workspace bytes of the f16 activations (n rows), rounded up to 256.
__host__ __device__ constexpr int64_t x16_bytes(int64_t n, int64_t k) {
    return (n * x16_row_halves(k) * 2 + 255) / 256 * 256;
}

// A plan forced by the caller (kernel family and k split), for tuning.
struct MfmaForce {
    int x16;
    int wm;
    int n_split;
    int kg;
};

// The plan for an m x k x n product on a device with num_cu compute units,
// with (have_ws) or without a workspace; force (or null) restricts the
// choice.  Without a workspace: gemm_mfma.hip's kernel, unsplit.
MfmaPlan plan_gemm_mfma(int64_t m, int64_t k, int64_t n, int qt, int num_cu, bool have_ws,
                        const MfmaForce* force);

// Launch with plan pl; ws (256-byte aligned, pl.ws_bytes) when pl.x16.
void launch_gemm_mfma(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int qt, int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd,
                      hipStream_t st);
void launch_gemm_lds(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qt,
                     int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd, hipStream_t st);
// Whether the LDS ring of gemm_lds.hip holds tiles of tile_rows x
// tile_tokens for format qt with kg k groups (its stages, or the k-group
// reduction, must fit the 160 KB of LDS).
bool lds_ring_fits(int qt, int tile_rows, int tile_tokens, int kg, bool xf);
// Work groups of that kernel the CU's LDS holds at once (1 or 2), 0 if none fits.
int lds_ring_per_cu(int qt, int tile_rows, int tile_tokens, int kg, bool xf);

// dst[(i / m)*ldd + i % m] = sum over z < n_split of part[z*zstride + i], in
// order of z, i < count.
void launch_splitk_sum(float* dst, const float* part, int64_t count, int64_t zstride, int n_split,
                       int64_t m, int64_t ldd, hipStream_t st);

void launch_moe(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                const int* ids, const float* scale, const float* x, int64_t t, int64_t n_used,
                int64_t n_expert, int64_t in_f, int64_t n_ff, int qt, int64_t rb,
                const GemvTuning& tune, hipStream_t st);

// MoE down projection: per-pair scaled rows into pair_out [n_pairs][d_model]
// (the gate/up kernel with one plane and each pair's own activation row),
// then y[tau] = the token's n_used pair rows summed in slot order.
void launch_moe_down(float* y, float* pair_out, const void* w_down, const int* ids,
                     const float* scale, const float* act, int64_t t, int64_t n_used,
                     int64_t n_expert, int64_t n_ff, int64_t d_model, int qt, int64_t rb,
                     const GemvTuning& tune, hipStream_t st);

// The gate and up projections fused with the SwiGLU/clamp activation:
// act[p][r] = silu(min(g, limit)) * clamp(u, -limit, limit) with g, u the
// scaled projections of launch_moe (f32 activations, or Q8_1 activations
// for NVFP4 / NVFP4 V2 weights).
void launch_moe_act(float* act, const void* wg, const void* wu, const int* ids, const float* sc, const float* x,
                    int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qt, int64_t rb,
                    float limit, const GemvTuning& tune, hipStream_t st);
void launch_moe_act_q8(float* act, const void* wg, const void* wu, const int* ids, const float* sc,
                       const int8_t* xq, const float* xd, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                       int64_t n_ff, int qt, int64_t rb, float limit, const GemvTuning& tune, hipStream_t st);

// The down projection on Q8_1 pair activations (aq [n_pairs][n_ff] codes, ad
// their block scales; NVFP4 or NVFP4 V2 weights), then the slot sum.
void launch_moe_down_q8(float* y, float* pair_out, const void* wd, const int* ids, const float* sc,
                        const int8_t* aq, const float* ad, int64_t t, int64_t n_used, int64_t n_expert, int64_t n_ff,
                        int64_t d_model, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st);

// The measurement twins of launch_moe (arm 1: load-only, 2: math-only) on
// NVFP4 / NVFP4 V2 weights: the same grid, de-duplication and addresses.
void launch_moe_probe(int arm, float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                      const float* x, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff,
                      int qt, int64_t rb, const GemvTuning& tune, hipStream_t st);

// NVFP4 rows (rows x k/64 groups of 36 bytes) -> the NVFP4 V2 layout.
void launch_nvfp4_repack_v2(void* dst, const void* src, int64_t rows, int64_t k, hipStream_t st);

// MoE gate/up with Q8_1 activations (codes xq [t][in_f], block scales xd
// [t][in_f/32]); NVFP4 or NVFP4 V2 weights.  LDS bytes it stages per work group:
void launch_moe_q8(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                   const int* ids, const float* scale, const int8_t* xq, const float* xd, int64_t t,
                   int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qt, int64_t rb,
                   const GemvTuning& tune, hipStream_t st);
int64_t moe_q8_lds_bytes(int64_t in_f);

// Q8_1 quantization of nblk blocks of 32 activations.
void launch_quantize_q8_1(int8_t* q, float* d, const float* x, int64_t nblk, hipStream_t st);

void launch_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k, int qt, int64_t rb,
                     const GemvTuning& tune, hipStream_t st);

// Largest byte window (relative to a 16-byte-aligned base) one GEMV work
// group addresses, for the host's 32-bit offset check.
int64_t gemv_max_window_bytes(int qt, int64_t k, int64_t rb);
int gemv_unit_elems(int qt);

// Largest tile sizes of the MFMA kernels (rows of W, tokens), for the host's
// 32-bit offset checks.
constexpr int MFMA_BM = 128;
constexpr int MFMA_BN = 128;
constexpr int MFMA_BM_MAX = 256;

}  // namespace qmm
