/*
 * qmm.h - dequant-fused projection matmul on block-quantized weights (gfx950).
 *
 * The operation (cera 0.4.0 examples/wgpu_gemm_bench.rs, the Shape doc
 * comment and the SHADER diff comment):
 *
 *     dst[j*m + i] = sum_{c<k} deq(W)[i][c] * x[j*k + c]     0<=i<m, 0<=j<n
 *
 * i.e. dst[n, m] = src0[m, k] * src1[n, k] with dst column-major, stride m.
 * W is m rows of row_bytes(qtype, k) bytes, blocks along k, rows contiguous,
 * no padding (the packed sizes of the VARIANTS table on the same page;
 * NVFP4 from memra-engine moe_rows_ceiling_bench.rs, synth_rows).
 *
 * Conventions for every entry point below:
 *  - Pointers marked DEVICE are device (HBM) pointers owned by the caller;
 *    the library never frees or retains them.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).  No
 *    call allocates device memory, synchronizes, or keeps state beyond lazily
 *    cached device properties (compute units, LDS sizes) and the parsed
 *    tuning variables (QMM_GEMV_MAX_N below; QMM_GEMV_WG_PER_CU and
 *    QMM_MOE_WG_PER_CU 1..64, QMM_GEMV_ROWS 1..2, QMM_GEMV_DEPTH 2/4/8,
 *    QMM_MOE_LPR_LOG2 3..6 (log2 of the MoE streams' largest lane group per
 *    row; rows of few units take smaller groups, down to 8 lanes) for the
 *    streaming kernels' launch shape; QMM_GEMV_MFMA_MIN 0..64 (default 3:
 *    the smallest n that QMM_PATH_GEMV runs on its matrix-core stream, 0 =
 *    never), QMM_GEMV_MFMA_TT 1..2 (that stream's activation rows per pass
 *    over the weights: at most 4 or 8), QMM_MOE_MFMA_MIN 0..4 (default 2:
 *    with more than one token, the MoE kernels run the experts' chunks of at
 *    least that many pairs on the matrix-core stream, 0 = never);
 *    a malformed value makes the calls that use it return
 *    QMM_ERR_RANGE; QMM_MFMA_PLAN is read again at every call that plans a
 *    prefill), so the calls can be recorded into a hipGraph.
 *  - Arguments are validated on the host before anything is launched; a
 *    rejected call returns a non-zero qmm_status and launches nothing.  A
 *    launch failure reported by the runtime returns QMM_ERR_LAUNCH.
 *  - Outputs are a pure function of the inputs: kernels read only the bytes
 *    the shapes define (loads past the end are bounds-checked by the buffer
 *    descriptors and return zero) and use no float atomics, so two identical
 *    calls produce bit-identical results.
 *  - Outputs must not overlap inputs (or each other): every entry point
 *    checks the byte ranges its sizes define and returns QMM_ERR_ALIAS,
 *    after all other checks and before any launch.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  Block sizes (elements / bytes): F32 1/4, Q4_0 32/18,
 * Q8_0 32/34, Q4_K 256/144, Q6_K 256/210, NVFP4 64/36 (the packed-size
 * formulas of cera wgpu_gemm_bench.rs VARIANTS and memra synth_rows).
 * NVFP4_V2 holds the values of NVFP4 rows in two streams per row (memra
 * moe_rows_ceiling_bench.rs, the V2 rows: 18 bytes per 32 weights, 16 of
 * quants and 2 of scales, the scales contiguous): the k/2 quant bytes (byte
 * 16g+j: weight 32g+j in its low nibble, 32g+16+j in its high nibble), then
 * the k/16 E4M3 scale bytes (byte 2g+i scales weights 32g+16i .. +15); k is
 * a multiple of 64 and a row is k/64*36 bytes, as for NVFP4.  qmm_nvfp4_repack_v2
 * converts.  NVFP4_V2 is accepted by the streaming paths (GEMV, MoE, load-only
 * twin); the matrix-core path returns QMM_ERR_QTYPE for it. */
typedef enum {
    QMM_F32 = 0,
    QMM_Q4_0 = 1,
    QMM_Q8_0 = 2,
    QMM_Q4_K = 3,
    QMM_Q6_K = 4,
    QMM_NVFP4 = 5,
    QMM_NVFP4_V2 = 6
} qmm_qtype;

typedef enum {
    QMM_OK = 0,
    QMM_ERR_NULL = 1,      /* a required pointer is null                      */
    QMM_ERR_SHAPE = 2,     /* a size is < 1, or a product overflows int64      */
    QMM_ERR_K_ALIGN = 3,   /* k is not a multiple of the block size (and of 4) */
    QMM_ERR_QTYPE = 4,     /* unknown qtype, or not valid for this entry point */
    QMM_ERR_ALIGN = 5,     /* w not 16-byte aligned, or x/dst not 16-byte aligned */
    QMM_ERR_LAUNCH = 6,    /* the runtime reported a launch error              */
    QMM_ERR_PATH = 7,      /* unknown path selector                            */
    QMM_ERR_RANGE = 8,     /* a size exceeds what the kernels index (see below) */
    QMM_ERR_WORKSPACE = 9, /* workspace smaller than qmm_gemm_workspace_bytes()  */
    QMM_ERR_ALIAS = 10,    /* an output overlaps an input that must stay intact  */
    QMM_ERR_SCRATCH = 11   /* qmm_gemm_noalloc: the plan needs more than the
                              library's static scratch holds                    */
} qmm_status;

/* Kernel path selector for qmm_gemm_path. */
typedef enum {
    QMM_PATH_AUTO = 0,     /* n <= qmm_gemv_max_n() -> GEMV, else MFMA       */
    QMM_PATH_GEMV = 1,     /* the f32 decode path, any n: GEMV_FMA for n below
                              QMM_GEMV_MFMA_MIN (3), GEMV_MATRIX from n = 8,
                              between them GEMV_MATRIX where the weights have
                              at least 4 row groups of 8 rows per CU or rows
                              of at least 64 blocks' units (k >= 2048 at 32
                              weights per unit), else GEMV_FMA               */
    QMM_PATH_MFMA = 2,     /* f16 MFMA tiles, f32 accumulation, any n (prefill) */
    QMM_PATH_GEMV_FMA = 3, /* the f32 decode path on f32 FMAs                  */
    QMM_PATH_GEMV_MATRIX = 4 /* the f32 decode path with its products on
                              v_mfma_f32_4x4x1f32 (f32 inputs, f32 sums), 4 or
                              8 activation rows per pass over the weights; where
                              4 rows do not fit one work group's LDS (k above
                              about 9000) it runs as GEMV_FMA                   */
} qmm_path;

/*
 * qmm_gemm: the projection above.
 *   dst   DEVICE float[n*m], written (every element), column-major stride m.
 *   w     DEVICE packed weights, m*row_bytes(qtype,k) bytes, 16-byte aligned.
 *         For QMM_F32, float[m*k].
 *   x     DEVICE float[n*k] activations, row-major, 16-byte aligned.
 *   m,k,n >= 1; k % block_elems(qtype) == 0 and k % 4 == 0.
 *   qtype one of QMM_F32..QMM_NVFP4_V2 (NVFP4_V2 on the GEMV path only).
 * Dispatch (the decode-GEMV / prefill-GEMM split of aprender-serve
 * cublas_prefill, its cublas_gemm_threshold): the f32 GEMV for n <= 32
 * (results within 1e-5 * sum|w*x| of the exact value; its products on f32
 * FMAs for n < 3 and on v_mfma_f32_4x4x1f32 above, f32 inputs and sums
 * either way: QMM_PATH_GEMV below), the MFMA kernel for
 * n > 32, which rounds W and x to f16 (RNE) and accumulates in f32 (within
 * 2e-3 * sum|w*x|).  With QMM_GEMV_MAX_N set: the GEMV for n <= that value,
 * else MFMA (the measured MI355X speed crossover is n = 8..16 on large
 * weight matrices; moving the threshold trades the tight tolerance for it).
 * Limits: the bytes of one 256-row weight tile (or one GEMV row group) and
 * of 128 (GEMV: 8) token rows of x each below 2^31; m, n, k below 2^31.
 * Larger values return QMM_ERR_RANGE.
 * qmm_gemm never splits k on the MFMA path (it has no workspace); products
 * with few output tiles run faster through qmm_gemm_ws.
 */
int qmm_gemm(float* dst, const void* w, const float* x,
             int64_t m, int64_t k, int64_t n, int qtype, hipStream_t stream);

/* qmm_gemm with an explicit kernel path (QMM_PATH_*).  Same arguments and
 * errors as qmm_gemm; QMM_ERR_PATH for an unknown path. */
int qmm_gemm_path(float* dst, const void* w, const float* x,
                  int64_t m, int64_t k, int64_t n, int qtype, int path,
                  hipStream_t stream);

/*
 * qmm_gemm_ws: qmm_gemm_path with a caller-owned workspace for the MFMA
 * path, where it lets the library
 *  - round the activations to f16 once per call (a pre-pass writing them
 *    into the workspace in the weight tiles' k order) for the kernels that
 *    read f16 activations; and
 *  - split k when the product has too few output tiles to fill the device:
 *    separate work groups write partial results to the workspace and a
 *    second kernel on the same stream adds them in a fixed order, so two
 *    identical calls still give bit-identical results.
 * A cost model fitted to MI355X measurements picks the kernel family, tile
 * shape, k groups and k split.  The families (the "x16" code of
 * qmm_gemm_plan and QMM_MFMA_PLAN):
 *   0  f32 activations rounded in the k loop, 128 x 128 tiles (1 or 2 k
 *      groups); the only family of calls without a workspace;
 *   2  the LDS ring (weight bytes and f16 activations streamed into a ring
 *      of LDS stages by buffer-to-LDS loads; weights decoded straight into
 *      the matrix-core operands), 64, 128 or 256 weight rows x 128 tokens,
 *      1 or 2 k groups; k a multiple of 64;
 *   3  the LDS ring with 128 x 256 tiles (half the decode work per
 *      matrix-core op; for products of many tiles);
 *   4  the LDS ring on the f32 activations themselves (no pre-pass and no
 *      f16 workspace), 64 or 128 weight rows x 128 tokens;
 *   5  the LDS ring with 64 x 64 tiles (four times the work groups of
 *      128 x 128 tiles, for products with fewer 64 x 128 tiles than CUs);
 *   6  the same 64 x 64 tiles on the f32 activations (as code 4);
 *   7  the LDS ring with 256 x 256 tiles, eight waves in two token groups
 *      sharing each stage (half the activation traffic per weight row).
 * (Code 1 is not used.)
 * Every family rounds each decoded weight and each activation to f16 once
 * (RNE) and accumulates in f32, so the tolerance is the one of qmm_gemm.
 * The plan is a pure function of (m, k, n, qtype) and the device's
 * compute-unit count; the environment variable
 * QMM_MFMA_PLAN="x16,wm,n_split[,kg]" forces it (tuning and tests only:
 * x16 0 with wm 2; 2 with wm 1, 2 or 4; 3 with wm 2; 4 with wm 1 or 2;
 * 5 or 6 with wm 1; 7 with wm 4 and kg 1; kg 1 or 2;
 * malformed -> QMM_ERR_RANGE; a family the format or k cannot run falls back
 * to family 0 unsplit).
 *   workspace        DEVICE memory, 256-byte aligned, of at least
 *                    qmm_gemm_workspace_bytes(m, k, n, qtype, path) bytes, or
 *                    NULL (then the f32-activation kernel without a k split).
 *                    No initial contents are needed.  Calls that share a
 *                    workspace must not overlap (order them on one stream).
 *                    The bytes the plan uses must not overlap dst, x or w
 *                    (QMM_ERR_ALIAS).
 *   workspace_bytes  its size; smaller than needed -> QMM_ERR_WORKSPACE.
 * The GEMV path ignores the workspace.  Other arguments and errors as
 * qmm_gemm_path.
 */
int qmm_gemm_ws(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                int qtype, int path, void* workspace, int64_t workspace_bytes,
                hipStream_t stream);

/*
 * qmm_gemm_ex: qmm_gemm_ws on row-strided activations and output (the F9
 * stride fields of cera wgpu_gemm_bench.rs's MulMatParams, where the rows of
 * src1 and dst need not be packed):
 *     dst[j*ldd + i] = sum_c deq(W)[i][c] * x[j*ldx + c]
 *   ldx   floats between consecutive rows of x: >= k (QMM_ERR_SHAPE) and a
 *         multiple of 4 (QMM_ERR_ALIGN), so every row is 16-byte aligned.
 *   ldd   floats between consecutive rows of dst: >= m (QMM_ERR_SHAPE).
 *         Elements of dst between m and ldd are not written.
 * qmm_gemm_ws(...) is qmm_gemm_ex with ldx = k and ldd = m.  Limits as
 * qmm_gemm with k replaced by ldx in the activation windows (8 rows for the
 * GEMV, 128 for the matrix-core tiles, below 2^31 bytes).
 */
int qmm_gemm_ex(float* dst, int64_t ldd, const void* w, const float* x, int64_t ldx, int64_t m, int64_t k,
                int64_t n, int qtype, int path, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * qmm_gemm_noalloc: qmm_gemm_ws without caller memory, for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is the library's own
 * static device array of qmm_gemm_noalloc_max_bytes() bytes (64 MiB), one
 * per GPU, held until the process ends; nothing is allocated by the call.
 *   Arguments and errors as qmm_gemm_path, plus QMM_ERR_SCRATCH when
 *   qmm_gemm_workspace_bytes(m, k, n, qtype, path) exceeds the array (no
 *   launch; such products can still run through qmm_gemm, unsplit, or
 *   qmm_gemm_ws with caller memory).  The plan, kernels and results are
 *   those of qmm_gemm_ws with a workspace of that size, bit for bit.
 *   The first call on a device looks up that device's address of the array
 *   (hipGetSymbolAddress, not a stream operation); QMM_ERR_LAUNCH if the
 *   runtime cannot give it.
 *   Every call on one GPU shares that GPU's array: calls that may overlap
 *   in time on one GPU (different streams without ordering, several host
 *   threads) race and must not be issued; calls ordered on one stream are
 *   safe.  The array needs no initial contents; it keeps whatever the last
 *   call left.
 */
int qmm_gemm_noalloc(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                     int qtype, int path, hipStream_t stream);

/* Bytes of qmm_gemm_noalloc's static scratch array (per GPU). */
int64_t qmm_gemm_noalloc_max_bytes(void);

/* Workspace bytes qmm_gemm_ws uses for this product on the current device:
 * 0 on the GEMV path, at least 256 on the MFMA path; < 0 is -qmm_status. */
int64_t qmm_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int qtype, int path);

/*
 * qmm_gemm_plan: the kernels a call with these sizes runs on the current
 * device, with (with_workspace != 0: qmm_gemm_ws) or without a workspace.
 *   out  HOST int32[6], written: path (QMM_PATH_GEMV for the three GEMV
 *        paths, or QMM_PATH_MFMA); then for the GEMV: 1 if it runs on the
 *        matrix-core stream (else 0), its activation rows per pass (4 or 8;
 *        0 on the FMA stream), zeros; for the MFMA path: the kernel family
 *        (0, 2, 3 or 4, as listed at qmm_gemm_ws; families 2 and 3 round the
 *        activations to f16 in a pre-pass), weight rows per tile, k groups
 *        per work group, k splits, and 64-k steps per split.
 * Errors as qmm_gemm_workspace_bytes; QMM_ERR_NULL for a null out.
 */
int qmm_gemm_plan(int64_t m, int64_t k, int64_t n, int qtype, int path, int with_workspace,
                  int32_t* out);

/*
 * qmm_moe_gateup: the MoE gate and up projections over the routed experts
 * (memra-engine moe_rows_ceiling_bench.rs: gate/up planes, in_f -> n_ff,
 * n_used experts per token, per-pair f32 scales indexed plane*n_pairs+pair as
 * the pointer table is).  With n_pairs = t*n_used, pair p = tau*n_used + s and
 * expert e = expert_ids[p]:
 *     gate_out[p*n_ff + r] = pair_scale[p]           * sum_c Wg[e][r][c] * x[tau*in_f + c]
 *     up_out  [p*n_ff + r] = pair_scale[n_pairs + p] * sum_c Wu[e][r][c] * x[tau*in_f + c]
 *   gate_out, up_out  DEVICE float[n_pairs*n_ff], written.
 *   w_gate, w_up      DEVICE, each n_expert*n_ff rows of row_bytes(qtype,in_f)
 *                     bytes (expert-major), 16-byte aligned.
 *   expert_ids        DEVICE int32[n_pairs]; an id outside [0, n_expert) makes
 *                     that pair's outputs NaN (no out-of-range read).
 *   pair_scale        DEVICE float[2*n_pairs] (gate plane, then up plane).
 *   x                 DEVICE float[t*in_f], 16-byte aligned.
 *   qtype             QMM_NVFP4 (the other formats are accepted too).
 * Each selected expert's rows are read once per call and applied to every
 * token that chose it.  f32 arithmetic; results within 1e-5*|scale|*sum|w*x|.
 */
int qmm_moe_gateup(float* gate_out, float* up_out,
                   const void* w_gate, const void* w_up,
                   const int32_t* expert_ids, const float* pair_scale,
                   const float* x, int64_t t, int64_t n_used, int64_t n_expert,
                   int64_t in_f, int64_t n_ff, int qtype, hipStream_t stream);

/*
 * qmm_moe_gateup_act: qmm_moe_gateup fused with the activation between the
 * gate/up and down projections (memra-engine moe_rows_ceiling_bench.rs: the
 * served gate/up is the "preclamp" kernel with argument 7.0, and its down
 * arm takes a SwiGLU output as input).  The page does not spell out the
 * clamp; the reading implemented: with g = gate_out[p*n_ff + r] and
 * u = up_out[p*n_ff + r] of qmm_moe_gateup,
 *     act[p*n_ff + r] = silu(min(g, limit)) * clamp(u, -limit, limit),
 *     silu(z) = z / (1 + exp(-z)),
 * so the gate is clamped above and the up projection on both sides before
 * SwiGLU.  limit = +inf is plain SwiGLU.
 *   act         DEVICE float[n_pairs*n_ff], written: the down projection's
 *               input (qmm_moe_down's act).
 *   limit       > 0 (7.0 on the page), or +inf; <= 0 or NaN -> QMM_ERR_RANGE.
 * Each selected expert's gate and up rows are read once per call, by work
 * groups that stream a row group's gate rows and then its up rows and
 * apply the activation in f32 (no gate/up output in memory).  Results
 * within tau*S_act of the exact value, where S_act carries the projections'
 * 1e-5 bound through the epilogue (clamps 1-Lipschitz, silu 1.1-Lipschitz)
 * plus 8 f32 ulps of |act|.  An invalid expert id gives NaN rows.  Other
 * arguments and errors as qmm_moe_gateup.
 */
int qmm_moe_gateup_act(float* act, const void* w_gate, const void* w_up, const int32_t* expert_ids,
                       const float* pair_scale, const float* x, int64_t t, int64_t n_used, int64_t n_expert,
                       int64_t in_f, int64_t n_ff, int qtype, float limit, hipStream_t stream);

/* qmm_moe_gateup_act on Q8_1 activations (xq, xd from qmm_quantize_q8_1,
 * the served arithmetic of the same page): the projections of
 * qmm_moe_gateup_q8, then the activation.  qtype QMM_NVFP4 or QMM_NVFP4_V2;
 * in_f at most 8320.  Other arguments and errors as qmm_moe_gateup_act. */
int qmm_moe_gateup_act_q8(float* act, const void* w_gate, const void* w_up, const int32_t* expert_ids,
                          const float* pair_scale, const int8_t* xq, const float* xd, int64_t t, int64_t n_used,
                          int64_t n_expert, int64_t in_f, int64_t n_ff, int qtype, float limit, hipStream_t stream);

/*
 * qmm_moe_gateup_probe: the measurement twins of qmm_moe_gateup (memra
 * moe_rows_ceiling_bench.rs, its ceiling-probe arms): the same grid, expert
 * de-duplication, descriptors and addresses as the served kernel, with
 *   arm 1  (load-only) the arithmetic deleted: each row's raw words folded
 *          by XOR into its output slot (a checksum, not a projection);
 *   arm 2  (math-only) every item loading the first unit of its row group
 *          (so every load hits the cache) and the full arithmetic run on it.
 * The outputs are not projections; they only keep the work live.  qtype
 * QMM_NVFP4 or QMM_NVFP4_V2; arm other than 1 or 2 -> QMM_ERR_PATH.  Other
 * arguments and errors as qmm_moe_gateup.  For measurement only.
 */
int qmm_moe_gateup_probe(int arm, float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                         const int32_t* expert_ids, const float* pair_scale, const float* x, int64_t t,
                         int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qtype,
                         hipStream_t stream);

/*
 * qmm_moe_down: the MoE down projection (memra-engine moe_rows_ceiling_bench.rs,
 * the down arm: one plane of d_model rows over n_ff inputs per expert, each
 * pair's own activation row (the SwiGLU output of its gate/up pair), the down
 * plane's per-pair scale, and the token's pairs accumulated into a zeroed y).
 * With n_pairs = t*n_used, pair p = tau*n_used + s and e = expert_ids[p]:
 *     pair_out[p*d_model + r] = pair_scale[p] * sum_c Wd[e][r][c] * act[p*n_ff + c]
 *     y[tau*d_model + r]      = sum over s = 0 .. n_used-1, in that order, of
 *                               pair_out[(tau*n_used + s)*d_model + r]
 *   y           DEVICE float[t*d_model], written (not accumulated into).
 *   pair_out    DEVICE float[n_pairs*d_model], written: the per-pair terms.
 *               Must not overlap y.
 *   w_down      DEVICE, n_expert*d_model rows of row_bytes(qtype, n_ff) bytes
 *               (expert-major), 16-byte aligned.
 *   expert_ids  DEVICE int32[n_pairs]; an id outside [0, n_expert) makes that
 *               pair's pair_out row, and so its token's y row, NaN (no
 *               out-of-range read).
 *   pair_scale  DEVICE float[n_pairs]: the down plane's scales (the third
 *               n_pairs block of the page's 3*n_pairs scale array).
 *   act         DEVICE float[n_pairs*n_ff], 16-byte aligned.
 *   qtype       QMM_NVFP4 (the other formats are accepted too).
 * Two launches on stream: the gate/up kernel with one plane and per-pair
 * activation rows (each selected expert's rows read once per call), then a
 * slot sum in fixed order, so identical calls give bit-identical results.
 * f32 arithmetic; y within 1e-5*sum_s |pair_scale|*sum_c |w*act|.
 * Errors as qmm_moe_gateup.
 */
int qmm_moe_down(float* y, float* pair_out, const void* w_down, const int32_t* expert_ids,
                 const float* pair_scale, const float* act, int64_t t, int64_t n_used,
                 int64_t n_expert, int64_t n_ff, int64_t d_model, int qtype, hipStream_t stream);

/*
 * qmm_moe_down_q8: qmm_moe_down on Q8_1 pair activations (memra
 * moe_rows_ceiling_bench.rs, the down arm: each pair's activation row is
 * quantized with quantize_q8_1 before moe_down8_fma_q8_rows).  With
 * act_hat[p*n_ff + c] = ad[p*n_ff/32 + c/32] * aq[p*n_ff + c], the outputs
 * are those of qmm_moe_down on act_hat; each 16-weight group's dot product
 * (E2M1 weights times int8 codes) is exact, its E4M3 scale, the block scale
 * and the sum over groups are applied in f32: within 1e-5 * sum_s
 * |pair_scale| * sum_c |w * act_hat|.
 *   aq, ad      DEVICE, as written by qmm_quantize_q8_1 for n_pairs rows of
 *               n_ff; aq 16-byte aligned.
 *   qtype       QMM_NVFP4 or QMM_NVFP4_V2 (else QMM_ERR_QTYPE).
 *   n_ff        a multiple of 64, at most 8320 (LDS: QMM_ERR_RANGE above).
 * Other arguments and errors as qmm_moe_down.
 */
int qmm_moe_down_q8(float* y, float* pair_out, const void* w_down, const int32_t* expert_ids,
                    const float* pair_scale, const int8_t* aq, const float* ad, int64_t t, int64_t n_used,
                    int64_t n_expert, int64_t n_ff, int64_t d_model, int qtype, hipStream_t stream);

/*
 * qmm_quantize_q8_1: Q8_1 activations (memra-engine moe_rows_ceiling_bench.rs
 * quantizes the activations with quantize_q8_1 before its served gate/up
 * kernel; the format is ggml's, not printed on the pages).  Per block of 32
 * consecutive activations of a row, in f32: d = max|x| / 127, then
 * q = round-half-away-from-zero(x * (1/d)), or q = 0 when d = 0.
 *   q     DEVICE int8[rows*k], written, 16-byte aligned.
 *   d     DEVICE float[rows*k/32], written (one scale per block).
 *   x     DEVICE float[rows*k], 16-byte aligned.
 *   k     a multiple of 32 (QMM_ERR_K_ALIGN).
 */
int qmm_quantize_q8_1(int8_t* q, float* d, const float* x, int64_t rows, int64_t k, hipStream_t stream);

/*
 * qmm_moe_gateup_q8: qmm_moe_gateup on Q8_1 activations (the served
 * arithmetic of memra-engine moe_rows_ceiling_bench.rs: quantized activations
 * and integer dot products).  With x_hat[tau*in_f + c] = xd[tau*in_f/32 + c/32]
 * * xq[tau*in_f + c], the outputs are those of qmm_moe_gateup on x_hat.  Each
 * 16-weight group's dot product (E2M1 weights times int8 codes) is exact;
 * its E4M3 scale, the block scale and the sum over groups are applied in f32,
 * so results are within 1e-5*|scale|*sum|w*x_hat|.
 *   xq, xd      DEVICE, as written by qmm_quantize_q8_1 for t rows of in_f;
 *               xq 16-byte aligned.
 *   qtype       QMM_NVFP4 or QMM_NVFP4_V2 (else QMM_ERR_QTYPE).
 *   in_f        a multiple of 64, at most 8320 (LDS: QMM_ERR_RANGE above).
 * Other arguments and errors as qmm_moe_gateup.
 */
int qmm_moe_gateup_q8(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                      const int32_t* expert_ids, const float* pair_scale, const int8_t* xq,
                      const float* xd, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                      int64_t n_ff, int qtype, hipStream_t stream);

/*
 * qmm_nvfp4_repack_v2: NVFP4 rows -> the same values as NVFP4_V2 rows (memra
 * moe_rows_ceiling_bench.rs repacks the expert rows once before its V2 arms).
 * Per row and 36-byte group G: the 32 quant bytes (group bytes 4..35) go to
 * row bytes 32G..32G+31, the scale word (group bytes 0..3) to row bytes
 * k/2 + 4G .. +3.  A pure byte permutation: decoding gives identical values.
 *   dst, src  DEVICE, rows * (k/64*36) bytes each, 4-byte aligned, not
 *             overlapping (QMM_ERR_ALIAS).
 *   rows      rows of k weights (for expert tensors: n_expert * rows per expert).
 *   k         a multiple of 64 (QMM_ERR_K_ALIGN).
 */
int qmm_nvfp4_repack_v2(void* dst, const void* src, int64_t rows, int64_t k, hipStream_t stream);

/*
 * qmm_stream_loadonly: the load-only twin of the GEMV (memra-engine
 * moe_rows_ceiling_bench.rs, the "loadonly" ceiling-probe arm: the same
 * addresses with the arithmetic deleted).  Reads every byte of the m packed
 * rows with the GEMV's access pattern and writes one checksum word per row to
 * sink (DEVICE uint32[m]) so the loads stay live.  Used only to measure the
 * access-pattern ceiling.
 */
int qmm_stream_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k,
                        int qtype, hipStream_t stream);

/* Packed bytes of one row of k weights; < 0 is -qmm_status on error.
 * (Sizes per the VARIANTS table of cera wgpu_gemm_bench.rs and memra
 * synth_rows.) */
int64_t qmm_row_bytes(int qtype, int64_t k);

/* Elements per block of qtype, or -QMM_ERR_QTYPE. */
int qmm_block_elems(int qtype);

/* The largest n that QMM_PATH_AUTO sends to the GEMV (32 by default); the
 * environment variable QMM_GEMV_MAX_N replaces it by the threshold it gives;
 * a set but unparseable or non-positive value makes this return
 * -QMM_ERR_RANGE and every AUTO call fail with QMM_ERR_RANGE, never a silent
 * default. */
int qmm_gemv_max_n(void);

/* Static string for a status code. */
const char* qmm_status_str(int status);

/* Library ABI version (incremented on incompatible changes). */
int qmm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
