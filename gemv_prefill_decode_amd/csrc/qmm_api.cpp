// C-ABI entry points of libqmm: argument validation, path dispatch, launch
// error reporting.  Declarations and the contract are in include/qmm.h.
#include "qmm.h"

#include <hip/hip_runtime.h>

#include <cerrno>
#include <climits>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "kernels.hpp"

namespace {

struct Fmt {
    int qk;  // elements per block
    int bb;  // bytes per block
};

// Packed sizes: cera wgpu_gemm_bench.rs VARIANTS (f32 e*4, q4_0 e/32*18,
// q8_0 e/32*34, q4_k e/256*144, q6_k e/256*210); memra synth_rows (NVFP4 36
// bytes per 64 weights) and its V2 rows (18 bytes per 32 weights, whole
// 64-weight groups per row).
constexpr Fmt kFmt[] = {{1, 4}, {32, 18}, {32, 34}, {256, 144}, {256, 210}, {64, 36}, {64, 36}};
constexpr int kNumQt = 7;

bool valid_qt(int qt) { return qt >= 0 && qt < kNumQt; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a + an) and [b, b + bn) share a byte (sizes in bytes, >= 0).
bool overlap(const void* a, int64_t an, const void* b, int64_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an > 0 && bn > 0 && x < y + (uintptr_t)bn && y < x + (uintptr_t)an;
}

// a*b without int64 overflow (both >= 0)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// QMM_PATH_AUTO: the GEMV (f32 arithmetic, the tight tolerance) for every
// n <= 32, the matrix-core path above: the decode/prefill split the pages
// draw between a batched GEMV and the GEMM (aprender-serve cublas_prefill,
// the cublas_gemm_threshold crossover), placed where the f32 path's
// precision is kept for all decode batch sizes.  QMM_GEMV_MAX_N moves the
// threshold (the measured MI355X speed crossover lies at n = 8..16 for
// large weight matrices).
constexpr int AUTO_GEMV_N = 32;

int g_gemv_max_n = AUTO_GEMV_N;
std::once_flag g_env_once;

void parse_env() {
    const char* v = std::getenv("QMM_GEMV_MAX_N");
    if (!v) return;
    char* end = nullptr;
    errno = 0;
    const long val = std::strtol(v, &end, 10);
    while (end && *end == ' ') ++end;
    if (errno != 0 || end == v || (end && *end != '\0') || val < 1 || val > INT_MAX)
        g_gemv_max_n = -QMM_ERR_RANGE;  // set but unusable: AUTO calls fail loudly
    else
        g_gemv_max_n = (int)val;
}

// Strict integer from the environment: absent -> dflt; set but not an
// integer in [lo, hi] -> -1 (the caller reports QMM_ERR_RANGE).
int env_int(const char* name, int dflt, int lo, int hi) {
    const char* v = std::getenv(name);
    if (!v) return dflt;
    char* end = nullptr;
    errno = 0;
    const long val = std::strtol(v, &end, 10);
    while (end && *end == ' ') ++end;
    if (errno != 0 || end == v || (end && *end != '\0') || val < lo || val > hi) return -1;
    return (int)val;
}

// Defaults measured on MI355X (graph-replayed, weights rotated through HBM):
// two rows per lane group and two items in flight per wave give the GEMV the
// occupancy to hide its loads.  The MoE grid aims at 8 work groups per CU
// over all the (expert, plane) sets: with one token the single-pair kernel
// holds four waves per SIMD, and the gate/up at t = 1 went from 20.9 to
// 19.7 us against 2 per CU; with many tokens each set keeps its floor of
// MOE_MIN_WG work groups either way.
struct TuneState {
    int wg_per_cu = 4;
    int moe_wg_per_cu = 8;
    int rows = 2;
    int depth = 2;
    int moe_lpr_cap = qmm::LPR_CAP_MULTI;
    int moe_mfma_min = 2;
    int gemv_mfma_min = 3;
    int gemv_mfma_tt = 2;
    bool bad = false;
};
TuneState g_tune;
std::once_flag g_tune_once;
std::mutex g_cu_mu;
struct DevProps {
    int cu = 0;
    int lds_wg = 0;
    int lds_cu = 0;
};
DevProps g_dev[64];

void parse_tune() {
    const int w = env_int("QMM_GEMV_WG_PER_CU", g_tune.wg_per_cu, 1, 64);
    const int mw = env_int("QMM_MOE_WG_PER_CU", g_tune.moe_wg_per_cu, 1, 64);
    const int r = env_int("QMM_GEMV_ROWS", g_tune.rows, 1, 2);
    const int d = env_int("QMM_GEMV_DEPTH", g_tune.depth, 2, 8);
    const int ml = env_int("QMM_MOE_LPR_LOG2", g_tune.moe_lpr_cap, qmm::LPR_CAP_MIN, 6);
    const int mm = env_int("QMM_MOE_MFMA_MIN", g_tune.moe_mfma_min, 0, 4);
    const int gm = env_int("QMM_GEMV_MFMA_MIN", g_tune.gemv_mfma_min, 0, 64);
    const int gt = env_int("QMM_GEMV_MFMA_TT", g_tune.gemv_mfma_tt, 1, 2);
    if (w < 0 || mw < 0 || r < 0 || d < 0 || ml < 0 || mm < 0 || gm < 0 || gt < 0 || (d & (d - 1)) != 0) {
        g_tune.bad = true;
        return;
    }
    g_tune.wg_per_cu = w;
    g_tune.moe_wg_per_cu = mw;
    g_tune.rows = r;
    g_tune.depth = d;
    g_tune.moe_lpr_cap = ml;
    g_tune.moe_mfma_min = mm;
    g_tune.gemv_mfma_min = gm;
    g_tune.gemv_mfma_tt = gt;
}

// QMM_MFMA_PLAN="x16,wm,n_split[,kg]" forces the prefill plan of calls with
// a workspace (tuning and tests): x16 0 (f32-activation kernel, 128-row
// tiles, kg k groups), 2 (the LDS ring, (64*wm)-row tiles), 3 (the LDS ring,
// 128 x 256 tiles), 4 (the LDS ring on f32 activations, (64*wm)-row tiles)
// 5 (the LDS ring, 64 x 64 tiles), 6 (the same on f32 activations) or 7
// (the LDS ring, 256 x 256 tiles in two token groups of 4 waves);
// where the LDS ring cannot run, the unsplit default; unset: the cost model
// chooses.  Malformed -> bad.
struct MfmaForceState {
    bool set = false;
    bool bad = false;
    qmm::MfmaForce f{0, 2, 1, 1};
};
// Parsed on every call (tests and sweeps change it within one process).
MfmaForceState parse_force() {
    MfmaForceState g_force;
    const char* v = std::getenv("QMM_MFMA_PLAN");
    if (!v) return g_force;
    int a = -1, b = -1, c = -1, d = 1;
    char tail = 0;
    const int got = std::sscanf(v, "%d,%d,%d,%d%c", &a, &b, &c, &d, &tail);
    if ((got != 3 && got != 4) || a < 0 || a > 7 || a == 1 || (b != 1 && b != 2 && b != 4) ||
        (b == 4 && a != 2 && a != 7) || (b == 1 && a != 2 && a != 4 && a != 5 && a != 6) ||
        ((a == 5 || a == 6) && b != 1) || (a == 7 && (b != 4 || d != 1)) ||
        c < 1 || c > 16 || (d != 1 && d != 2)) {
        g_force.bad = true;
        return g_force;
    }
    g_force.set = true;
    g_force.f = qmm::MfmaForce{a, b, c, d};
    return g_force;
}

// Tuning for the current device; false if a tuning variable is malformed.
bool gemv_tuning(qmm::GemvTuning* t) {
    std::call_once(g_tune_once, parse_tune);
    if (g_tune.bad) return false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    DevProps p;
    {
        std::lock_guard<std::mutex> lk(g_cu_mu);
        if (dev >= 0 && dev < 64) p = g_dev[dev];
    }
    if (p.cu <= 0) {
        // a failed query leaves the conservative value (64 KB of LDS, 256 CUs)
        auto attr = [dev](hipDeviceAttribute_t a, int dflt) {
            int v = 0;
            return hipDeviceGetAttribute(&v, a, dev) == hipSuccess && v > 0 ? v : dflt;
        };
        p.cu = attr(hipDeviceAttributeMultiprocessorCount, 256);
        p.lds_wg = attr(hipDeviceAttributeMaxSharedMemoryPerBlock, 64 * 1024);
        p.lds_cu = attr(hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, p.lds_wg);
        std::lock_guard<std::mutex> lk(g_cu_mu);
        if (dev >= 0 && dev < 64) g_dev[dev] = p;
    }
    t->num_cu = p.cu;
    t->lds_per_wg = p.lds_wg;
    t->lds_per_cu = p.lds_cu;
    t->wg_per_cu = g_tune.wg_per_cu;
    t->moe_wg_per_cu = g_tune.moe_wg_per_cu;
    t->rows = g_tune.rows;
    t->depth = g_tune.depth;
    t->moe_lpr_cap = g_tune.moe_lpr_cap;
    t->moe_mfma_min = g_tune.moe_mfma_min;
    t->gemv_mfma_min = g_tune.gemv_mfma_min;
    t->gemv_mfma_tt = g_tune.gemv_mfma_tt;
    return true;
}

// A byte range of an input, for the overlap checks.
struct Span {
    const void* p;
    int64_t n;
};
bool overlaps_any(const void* o, int64_t ob, std::initializer_list<Span> ins) {
    for (const Span& s : ins)
        if (overlap(o, ob, s.p, s.n)) return true;
    return false;
}

int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
}

// Common checks for a weight matrix of m rows x k.  On success *rb is the row
// stride in bytes.
int check_weights(const void* w, int64_t m, int64_t k, int qt, int64_t* rb) {
    if (!w) return QMM_ERR_NULL;
    if (!valid_qt(qt)) return QMM_ERR_QTYPE;
    if (m < 1 || k < 1) return QMM_ERR_SHAPE;
    if (k % kFmt[qt].qk != 0 || k % 4 != 0) return QMM_ERR_K_ALIGN;
    if (!aligned(w, 16)) return QMM_ERR_ALIGN;
    if (m > INT_MAX || k > INT_MAX) return QMM_ERR_RANGE;
    *rb = k / kFmt[qt].qk * kFmt[qt].bb;
    int64_t total;
    if (!mul_ok(m, *rb, &total)) return QMM_ERR_SHAPE;
    return QMM_OK;
}

int auto_path(int64_t n) {
    const int lim = qmm_gemv_max_n();
    if (lim < 0) return -1;
    return n <= lim ? QMM_PATH_GEMV : QMM_PATH_MFMA;
}

// Shared validation of the gemm entry points; resolves AUTO.  On success
// *rb is the row stride and *path the concrete path.
int check_gemm(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qtype,
               int64_t ldx, int64_t ldd, int* path, int64_t* rb) {
    if (!dst || !x) return QMM_ERR_NULL;
    int st = check_weights(w, m, k, qtype, rb);
    if (st) return st;
    if (n < 1 || ldx < k || ldd < m) return QMM_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(dst, 16) || ldx % 4 != 0) return QMM_ERR_ALIGN;
    if (n > INT_MAX || ldx > INT_MAX || ldd > INT_MAX) return QMM_ERR_RANGE;
    int64_t t1, t2;
    if (!mul_ok(n, ldx, &t1) || !mul_ok(n, ldd, &t2)) return QMM_ERR_SHAPE;
    const int64_t dst_b = ((n - 1) * ldd + m) * 4, x_b = ((n - 1) * ldx + k) * 4;
    // last of the checks: an output overlapping an input
    auto alias = [&]() {
        return overlap(dst, dst_b, x, x_b) || overlap(dst, dst_b, w, m * *rb) ? QMM_ERR_ALIAS : QMM_OK;
    };
    if (*path == QMM_PATH_AUTO) {
        *path = auto_path(n);
        if (*path < 0) return QMM_ERR_RANGE;
    }
    if (*path == QMM_PATH_GEMV || *path == QMM_PATH_GEMV_FMA || *path == QMM_PATH_GEMV_MATRIX) {
        // one work group addresses at most this window of w, and 8 token rows of x
        if (qmm::gemv_max_window_bytes(qtype, k, *rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
        if ((7 * ldx + k) * 4 >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
        return alias();
    }
    if (*path == QMM_PATH_MFMA) {
        if (qtype == QMM_NVFP4_V2) return QMM_ERR_QTYPE;  // streaming paths only
        if ((int64_t)qmm::MFMA_BM_MAX * *rb + 16 >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
        if (((int64_t)(qmm::MFMA_BN - 1) * ldx + k) * 4 >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
        const int64_t tiles = ((m + qmm::MFMA_BM - 1) / qmm::MFMA_BM) * ((n + qmm::MFMA_BN - 1) / qmm::MFMA_BN);
        // work items (tiles x k splits, at most 16) are counted in int
        if (tiles > INT_MAX / 16) return QMM_ERR_RANGE;
        return alias();
    }
    return QMM_ERR_PATH;
}

int gemm_impl(float* dst, int64_t ldd, const void* w, const float* x, int64_t ldx, int64_t m, int64_t k,
              int64_t n, int qtype, int path, void* ws, int64_t ws_bytes, hipStream_t stream) {
    int64_t rb;
    int st = check_gemm(dst, w, x, m, k, n, qtype, ldx, ldd, &path, &rb);
    if (st) return st;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    if (path == QMM_PATH_GEMV || path == QMM_PATH_GEMV_FMA || path == QMM_PATH_GEMV_MATRIX) {
        const int kind = path == QMM_PATH_GEMV_FMA ? qmm::GEMV_FMA : (path == QMM_PATH_GEMV_MATRIX ? qmm::GEMV_MATRIX : qmm::GEMV_AUTO);
        qmm::launch_gemv(dst, w, x, m, k, n, qtype, rb, ldx, ldd, kind, tune, stream);
        return launch_status();
    }
    const MfmaForceState g_force = parse_force();
    if (g_force.bad) return QMM_ERR_RANGE;
    const qmm::MfmaPlan pl =
        qmm::plan_gemm_mfma(m, k, n, qtype, tune.num_cu, ws != nullptr, g_force.set ? &g_force.f : nullptr);
    if (ws) {
        if (!aligned(ws, 256)) return QMM_ERR_ALIGN;
        if (ws_bytes < pl.ws_bytes) return QMM_ERR_WORKSPACE;
        // the kernels write the workspace while reading x and w and writing
        // dst: the bytes they use must not overlap any of them
        const int64_t dst_b = ((n - 1) * ldd + m) * 4, x_b = ((n - 1) * ldx + k) * 4;
        if (overlap(ws, pl.ws_bytes, dst, dst_b) || overlap(ws, pl.ws_bytes, x, x_b) ||
            overlap(ws, pl.ws_bytes, w, m * rb))
            return QMM_ERR_ALIAS;
    }
    qmm::launch_gemm_mfma(dst, w, x, m, k, n, qtype, rb, pl, ws, ldx, ldd, stream);
    return launch_status();
}

}  // namespace

extern "C" {

int qmm_abi_version(void) { return 1; }

int64_t qmm_row_bytes(int qtype, int64_t k) {
    if (!valid_qt(qtype)) return -QMM_ERR_QTYPE;
    if (k < 1) return -QMM_ERR_SHAPE;
    if (k % kFmt[qtype].qk != 0) return -QMM_ERR_K_ALIGN;
    int64_t r;
    if (!mul_ok(k / kFmt[qtype].qk, kFmt[qtype].bb, &r)) return -QMM_ERR_SHAPE;
    return r;
}

int qmm_block_elems(int qtype) { return valid_qt(qtype) ? kFmt[qtype].qk : -QMM_ERR_QTYPE; }

int qmm_gemv_max_n(void) {
    std::call_once(g_env_once, parse_env);
    return g_gemv_max_n;
}

const char* qmm_status_str(int s) {
    switch (s) {
        case QMM_OK: return "ok";
        case QMM_ERR_NULL: return "null pointer argument";
        case QMM_ERR_SHAPE: return "invalid shape (a size < 1 or an int64 overflow)";
        case QMM_ERR_K_ALIGN: return "k is not a multiple of the block size (and of 4)";
        case QMM_ERR_QTYPE: return "unknown or unsupported qtype";
        case QMM_ERR_ALIGN: return "misaligned pointer (w, x and outputs must be 16-byte aligned)";
        case QMM_ERR_LAUNCH: return "kernel launch failed";
        case QMM_ERR_PATH: return "unknown kernel path";
        case QMM_ERR_RANGE: return "size outside the kernels' index range (or bad QMM_GEMV_MAX_N)";
        case QMM_ERR_WORKSPACE: return "workspace smaller than qmm_gemm_workspace_bytes()";
        case QMM_ERR_ALIAS: return "an output overlaps an input";
        case QMM_ERR_SCRATCH: return "product needs more workspace than the library's static scratch holds";
    }
    return "unknown status";
}

int64_t qmm_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int qtype, int path) {
    if (!valid_qt(qtype)) return -QMM_ERR_QTYPE;
    if (m < 1 || k < 1 || n < 1) return -QMM_ERR_SHAPE;
    if (m > INT_MAX || k > INT_MAX || n > INT_MAX) return -QMM_ERR_RANGE;
    if (path == QMM_PATH_AUTO) {
        path = auto_path(n);
        if (path < 0) return -QMM_ERR_RANGE;
    }
    if (path == QMM_PATH_GEMV || path == QMM_PATH_GEMV_FMA || path == QMM_PATH_GEMV_MATRIX) return 0;
    if (path != QMM_PATH_MFMA) return -QMM_ERR_PATH;
    if (qtype == QMM_NVFP4_V2) return -QMM_ERR_QTYPE;  // streaming paths only
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return -QMM_ERR_RANGE;
    const MfmaForceState g_force = parse_force();
    if (g_force.bad) return -QMM_ERR_RANGE;
    return qmm::plan_gemm_mfma(m, k, n, qtype, tune.num_cu, true, g_force.set ? &g_force.f : nullptr).ws_bytes;
}

int qmm_gemm_plan(int64_t m, int64_t k, int64_t n, int qtype, int path, int with_workspace, int32_t* out) {
    if (!out) return QMM_ERR_NULL;
    if (!valid_qt(qtype)) return QMM_ERR_QTYPE;
    if (m < 1 || k < 1 || n < 1) return QMM_ERR_SHAPE;
    if (m > INT_MAX || k > INT_MAX || n > INT_MAX) return QMM_ERR_RANGE;
    if (path == QMM_PATH_AUTO) {
        path = auto_path(n);
        if (path < 0) return QMM_ERR_RANGE;
    }
    if (path == QMM_PATH_GEMV || path == QMM_PATH_GEMV_FMA || path == QMM_PATH_GEMV_MATRIX) {
        qmm::GemvTuning tune;
        if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
        const int kind = path == QMM_PATH_GEMV_FMA ? qmm::GEMV_FMA : (path == QMM_PATH_GEMV_MATRIX ? qmm::GEMV_MATRIX : qmm::GEMV_AUTO);
        const int tok = qmm::gemv_matrix_tokens(m, k, n, qtype, kind, tune);
        out[0] = QMM_PATH_GEMV;
        out[1] = tok > 0 ? 1 : 0;
        out[2] = tok;
        out[3] = out[4] = out[5] = 0;
        return QMM_OK;
    }
    if (path != QMM_PATH_MFMA) return QMM_ERR_PATH;
    if (qtype == QMM_NVFP4_V2) return QMM_ERR_QTYPE;  // streaming paths only
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    const MfmaForceState g_force = parse_force();
    if (g_force.bad) return QMM_ERR_RANGE;
    const qmm::MfmaPlan pl = qmm::plan_gemm_mfma(m, k, n, qtype, tune.num_cu, with_workspace != 0,
                                                g_force.set ? &g_force.f : nullptr);
    out[0] = QMM_PATH_MFMA;
    out[1] = pl.x16;
    out[2] = 64 * pl.wm;
    out[3] = pl.kg;
    out[4] = pl.n_split;
    out[5] = pl.sps;
    return QMM_OK;
}

int qmm_gemm_ws(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qtype,
                int path, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gemm_impl(dst, m, w, x, k, m, k, n, qtype, path, workspace, workspace_bytes, stream);
}

int qmm_gemm_ex(float* dst, int64_t ldd, const void* w, const float* x, int64_t ldx, int64_t m, int64_t k,
                int64_t n, int qtype, int path, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gemm_impl(dst, ldd, w, x, ldx, m, k, n, qtype, path, workspace, workspace_bytes, stream);
}

int qmm_gemm_path(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                  int qtype, int path, hipStream_t stream) {
    return gemm_impl(dst, m, w, x, k, m, k, n, qtype, path, nullptr, 0, stream);
}

int qmm_gemm(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qtype,
             hipStream_t stream) {
    return qmm_gemm_path(dst, w, x, m, k, n, qtype, QMM_PATH_AUTO, stream);
}

int qmm_moe_gateup(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                   const int32_t* expert_ids, const float* pair_scale, const float* x, int64_t t,
                   int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qtype,
                   hipStream_t stream) {
    if (!gate_out || !up_out || !w_gate || !w_up || !expert_ids || !pair_scale || !x)
        return QMM_ERR_NULL;
    if (t < 1 || n_used < 1 || n_expert < 1 || n_used > n_expert) return QMM_ERR_SHAPE;
    int64_t rb;
    int64_t rows;
    if (!mul_ok(n_expert, n_ff, &rows)) return QMM_ERR_SHAPE;
    int st = check_weights(w_gate, rows, in_f, qtype, &rb);
    if (st) return st;
    st = check_weights(w_up, rows, in_f, qtype, &rb);
    if (st) return st;
    if (!aligned(x, 16) || !aligned(gate_out, 4) || !aligned(up_out, 4) || !aligned(pair_scale, 4) ||
        !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    int64_t n_pairs;
    if (!mul_ok(t, n_used, &n_pairs)) return QMM_ERR_SHAPE;
    if (n_pairs > 65535 || n_ff > INT_MAX || t * in_f * 4 >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::gemv_max_window_bytes(qtype, in_f, rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    {
        const int64_t ob = n_pairs * n_ff * 4, wb = rows * rb;
        if (overlap(gate_out, ob, up_out, ob) || overlap(gate_out, ob, x, t * in_f * 4) ||
            overlap(up_out, ob, x, t * in_f * 4) || overlap(gate_out, ob, w_gate, wb) ||
            overlap(gate_out, ob, w_up, wb) || overlap(up_out, ob, w_gate, wb) ||
            overlap(up_out, ob, w_up, wb) || overlap(gate_out, ob, expert_ids, n_pairs * 4) ||
            overlap(up_out, ob, expert_ids, n_pairs * 4) || overlap(gate_out, ob, pair_scale, n_pairs * 8) ||
            overlap(up_out, ob, pair_scale, n_pairs * 8))
            return QMM_ERR_ALIAS;
    }
    qmm::launch_moe(gate_out, up_out, w_gate, w_up, expert_ids, pair_scale, x, t, n_used, n_expert,
                    in_f, n_ff, qtype, rb, tune, stream);
    return launch_status();
}

// Shared checks of the gate/up family: pairs, both planes' weights, the
// activation window (x_bytes per token row) and the streaming windows.  On
// success *rb, *rows (n_expert * n_ff) and *n_pairs are set.
static int check_moe_gateup(const void* w_gate, const void* w_up, int64_t t, int64_t n_used, int64_t n_expert,
                            int64_t in_f, int64_t n_ff, int qtype, int64_t x_row_bytes, int64_t* rb, int64_t* rows,
                            int64_t* n_pairs) {
    if (t < 1 || n_used < 1 || n_expert < 1 || n_used > n_expert) return QMM_ERR_SHAPE;
    if (!mul_ok(n_expert, n_ff, rows)) return QMM_ERR_SHAPE;
    int st = check_weights(w_gate, *rows, in_f, qtype, rb);
    if (st) return st;
    st = check_weights(w_up, *rows, in_f, qtype, rb);
    if (st) return st;
    if (!mul_ok(t, n_used, n_pairs)) return QMM_ERR_SHAPE;
    if (*n_pairs > 65535 || n_ff > INT_MAX || t * x_row_bytes >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::gemv_max_window_bytes(qtype, in_f, *rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    return QMM_OK;
}

int qmm_moe_gateup_act(float* act, const void* w_gate, const void* w_up, const int32_t* expert_ids,
                       const float* pair_scale, const float* x, int64_t t, int64_t n_used, int64_t n_expert,
                       int64_t in_f, int64_t n_ff, int qtype, float limit, hipStream_t stream) {
    if (!act || !w_gate || !w_up || !expert_ids || !pair_scale || !x) return QMM_ERR_NULL;
    int64_t rb, rows, n_pairs;
    int st = check_moe_gateup(w_gate, w_up, t, n_used, n_expert, in_f, n_ff, qtype, in_f * 4, &rb, &rows, &n_pairs);
    if (st) return st;
    if (!aligned(x, 16) || !aligned(act, 4) || !aligned(pair_scale, 4) || !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    if (!(limit > 0.0f)) return QMM_ERR_RANGE;  // also NaN
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    const int64_t wb = rows * rb;
    if (overlaps_any(act, n_pairs * n_ff * 4, {{x, t * in_f * 4}, {w_gate, wb}, {w_up, wb},
                                                 {expert_ids, n_pairs * 4}, {pair_scale, n_pairs * 8}}))
        return QMM_ERR_ALIAS;
    qmm::launch_moe_act(act, w_gate, w_up, expert_ids, pair_scale, x, t, n_used, n_expert, in_f, n_ff, qtype, rb,
                        limit, tune, stream);
    return launch_status();
}

int qmm_moe_gateup_act_q8(float* act, const void* w_gate, const void* w_up, const int32_t* expert_ids,
                          const float* pair_scale, const int8_t* xq, const float* xd, int64_t t, int64_t n_used,
                          int64_t n_expert, int64_t in_f, int64_t n_ff, int qtype, float limit, hipStream_t stream) {
    if (!act || !w_gate || !w_up || !expert_ids || !pair_scale || !xq || !xd) return QMM_ERR_NULL;
    if (qtype != QMM_NVFP4 && qtype != QMM_NVFP4_V2) return QMM_ERR_QTYPE;
    int64_t rb, rows, n_pairs;
    int st = check_moe_gateup(w_gate, w_up, t, n_used, n_expert, in_f, n_ff, qtype, in_f, &rb, &rows, &n_pairs);
    if (st) return st;
    if (!aligned(xq, 16) || !aligned(xd, 4) || !aligned(act, 4) || !aligned(pair_scale, 4) ||
        !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    if (qmm::moe_q8_lds_bytes(in_f) > 64 * 1024) return QMM_ERR_RANGE;
    if (!(limit > 0.0f)) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    const int64_t wb = rows * rb;
    if (overlaps_any(act, n_pairs * n_ff * 4, {{xq, t * in_f}, {xd, t * in_f / 8}, {w_gate, wb}, {w_up, wb},
                                                 {expert_ids, n_pairs * 4}, {pair_scale, n_pairs * 8}}))
        return QMM_ERR_ALIAS;
    qmm::launch_moe_act_q8(act, w_gate, w_up, expert_ids, pair_scale, xq, xd, t, n_used, n_expert, in_f, n_ff, qtype,
                           rb, limit, tune, stream);
    return launch_status();
}

int qmm_moe_gateup_probe(int arm, float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                         const int32_t* expert_ids, const float* pair_scale, const float* x, int64_t t,
                         int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qtype, hipStream_t stream) {
    if (arm != 1 && arm != 2) return QMM_ERR_PATH;
    if (!gate_out || !up_out || !w_gate || !w_up || !expert_ids || !pair_scale || !x) return QMM_ERR_NULL;
    if (qtype != QMM_NVFP4 && qtype != QMM_NVFP4_V2) return QMM_ERR_QTYPE;
    int64_t rb, rows, n_pairs;
    int st = check_moe_gateup(w_gate, w_up, t, n_used, n_expert, in_f, n_ff, qtype, in_f * 4, &rb, &rows, &n_pairs);
    if (st) return st;
    if (!aligned(x, 16) || !aligned(gate_out, 4) || !aligned(up_out, 4) || !aligned(pair_scale, 4) ||
        !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    const int64_t ob = n_pairs * n_ff * 4, wb = rows * rb;
    for (float* o : {gate_out, up_out})
        if (overlaps_any(o, ob, {{x, t * in_f * 4}, {w_gate, wb}, {w_up, wb}, {expert_ids, n_pairs * 4},
                                 {pair_scale, n_pairs * 8}}))
            return QMM_ERR_ALIAS;
    if (overlap(gate_out, ob, up_out, ob)) return QMM_ERR_ALIAS;
    qmm::launch_moe_probe(arm, gate_out, up_out, w_gate, w_up, expert_ids, pair_scale, x, t, n_used, n_expert, in_f,
                          n_ff, qtype, rb, tune, stream);
    return launch_status();
}

int qmm_moe_down_q8(float* y, float* pair_out, const void* w_down, const int32_t* expert_ids,
                    const float* pair_scale, const int8_t* aq, const float* ad, int64_t t, int64_t n_used,
                    int64_t n_expert, int64_t n_ff, int64_t d_model, int qtype, hipStream_t stream) {
    if (!y || !pair_out || !w_down || !expert_ids || !pair_scale || !aq || !ad) return QMM_ERR_NULL;
    if (qtype != QMM_NVFP4 && qtype != QMM_NVFP4_V2) return QMM_ERR_QTYPE;
    if (t < 1 || n_used < 1 || n_expert < 1 || n_used > n_expert) return QMM_ERR_SHAPE;
    int64_t rb, rows;
    if (!mul_ok(n_expert, d_model, &rows)) return QMM_ERR_SHAPE;
    int st = check_weights(w_down, rows, n_ff, qtype, &rb);
    if (st) return st;
    if (!aligned(aq, 16) || !aligned(ad, 4) || !aligned(y, 4) || !aligned(pair_out, 4) || !aligned(pair_scale, 4) ||
        !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    int64_t n_pairs, outs;
    if (!mul_ok(t, n_used, &n_pairs) || !mul_ok(n_pairs, d_model, &outs)) return QMM_ERR_SHAPE;
    if (n_pairs > 65535 || d_model > INT_MAX || n_pairs * n_ff >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::gemv_max_window_bytes(qtype, n_ff, rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::moe_q8_lds_bytes(n_ff) > 64 * 1024) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    const int64_t yb = t * d_model * 4, pb = outs * 4, wb = rows * rb;
    for (const Span& o : {Span{y, yb}, Span{pair_out, pb}})
        if (overlaps_any(o.p, o.n, {{aq, n_pairs * n_ff}, {ad, n_pairs * n_ff / 8}, {w_down, wb},
                                    {expert_ids, n_pairs * 4}, {pair_scale, n_pairs * 4}}))
            return QMM_ERR_ALIAS;
    if (overlap(y, yb, pair_out, pb)) return QMM_ERR_ALIAS;
    qmm::launch_moe_down_q8(y, pair_out, w_down, expert_ids, pair_scale, aq, ad, t, n_used, n_expert, n_ff, d_model,
                            qtype, rb, tune, stream);
    return launch_status();
}

int qmm_moe_down(float* y, float* pair_out, const void* w_down, const int32_t* expert_ids,
                 const float* pair_scale, const float* act, int64_t t, int64_t n_used,
                 int64_t n_expert, int64_t n_ff, int64_t d_model, int qtype, hipStream_t stream) {
    if (!y || !pair_out || !w_down || !expert_ids || !pair_scale || !act) return QMM_ERR_NULL;
    if (t < 1 || n_used < 1 || n_expert < 1 || n_used > n_expert) return QMM_ERR_SHAPE;
    int64_t rb;
    int64_t rows;
    if (!mul_ok(n_expert, d_model, &rows)) return QMM_ERR_SHAPE;
    int st = check_weights(w_down, rows, n_ff, qtype, &rb);
    if (st) return st;
    if (!aligned(act, 16) || !aligned(y, 4) || !aligned(pair_out, 4) || !aligned(pair_scale, 4) ||
        !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    int64_t n_pairs, outs;
    if (!mul_ok(t, n_used, &n_pairs) || !mul_ok(n_pairs, d_model, &outs)) return QMM_ERR_SHAPE;
    if (n_pairs > 65535 || d_model > INT_MAX || n_pairs * n_ff * 4 >= ((int64_t)1 << 31))
        return QMM_ERR_RANGE;
    if (qmm::gemv_max_window_bytes(qtype, n_ff, rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    {
        const int64_t yb = t * d_model * 4, pb = outs * 4, wb = rows * rb, ab = n_pairs * n_ff * 4;
        if (overlap(y, yb, pair_out, pb) || overlap(y, yb, act, ab) || overlap(pair_out, pb, act, ab) ||
            overlap(y, yb, w_down, wb) || overlap(pair_out, pb, w_down, wb) ||
            overlap(y, yb, expert_ids, n_pairs * 4) || overlap(pair_out, pb, expert_ids, n_pairs * 4) ||
            overlap(y, yb, pair_scale, n_pairs * 4) || overlap(pair_out, pb, pair_scale, n_pairs * 4))
            return QMM_ERR_ALIAS;
    }
    qmm::launch_moe_down(y, pair_out, w_down, expert_ids, pair_scale, act, t, n_used, n_expert, n_ff,
                         d_model, qtype, rb, tune, stream);
    return launch_status();
}

int qmm_quantize_q8_1(int8_t* q, float* d, const float* x, int64_t rows, int64_t k, hipStream_t stream) {
    if (!q || !d || !x) return QMM_ERR_NULL;
    if (rows < 1 || k < 1) return QMM_ERR_SHAPE;
    if (k % 32 != 0) return QMM_ERR_K_ALIGN;
    if (!aligned(q, 16) || !aligned(x, 16) || !aligned(d, 4)) return QMM_ERR_ALIGN;
    int64_t elems;
    if (!mul_ok(rows, k, &elems)) return QMM_ERR_SHAPE;
    if (overlap(q, elems, d, elems / 8) || overlap(q, elems, x, elems * 4) || overlap(d, elems / 8, x, elems * 4))
        return QMM_ERR_ALIAS;
    qmm::launch_quantize_q8_1(q, d, x, elems / 32, stream);
    return launch_status();
}

int qmm_moe_gateup_q8(float* gate_out, float* up_out, const void* w_gate, const void* w_up,
                      const int32_t* expert_ids, const float* pair_scale, const int8_t* xq,
                      const float* xd, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                      int64_t n_ff, int qtype, hipStream_t stream) {
    if (!gate_out || !up_out || !w_gate || !w_up || !expert_ids || !pair_scale || !xq || !xd)
        return QMM_ERR_NULL;
    if (t < 1 || n_used < 1 || n_expert < 1 || n_used > n_expert) return QMM_ERR_SHAPE;
    if (qtype != QMM_NVFP4 && qtype != QMM_NVFP4_V2) return QMM_ERR_QTYPE;
    int64_t rb;
    int64_t rows;
    if (!mul_ok(n_expert, n_ff, &rows)) return QMM_ERR_SHAPE;
    int st = check_weights(w_gate, rows, in_f, qtype, &rb);
    if (st) return st;
    st = check_weights(w_up, rows, in_f, qtype, &rb);
    if (st) return st;
    if (!aligned(xq, 16) || !aligned(xd, 4) || !aligned(gate_out, 4) || !aligned(up_out, 4) ||
        !aligned(pair_scale, 4) || !aligned(expert_ids, 4))
        return QMM_ERR_ALIGN;
    int64_t n_pairs;
    if (!mul_ok(t, n_used, &n_pairs)) return QMM_ERR_SHAPE;
    if (n_pairs > 65535 || n_ff > INT_MAX || t * in_f >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::gemv_max_window_bytes(qtype, in_f, rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    if (qmm::moe_q8_lds_bytes(in_f) > 64 * 1024) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    {
        const int64_t ob = n_pairs * n_ff * 4, wb = rows * rb;
        if (overlap(gate_out, ob, up_out, ob) || overlap(gate_out, ob, xq, t * in_f) ||
            overlap(up_out, ob, xq, t * in_f) || overlap(gate_out, ob, xd, t * in_f / 8) ||
            overlap(up_out, ob, xd, t * in_f / 8) || overlap(gate_out, ob, w_gate, wb) ||
            overlap(gate_out, ob, w_up, wb) || overlap(up_out, ob, w_gate, wb) ||
            overlap(up_out, ob, w_up, wb) || overlap(gate_out, ob, expert_ids, n_pairs * 4) ||
            overlap(up_out, ob, expert_ids, n_pairs * 4) || overlap(gate_out, ob, pair_scale, n_pairs * 8) ||
            overlap(up_out, ob, pair_scale, n_pairs * 8))
            return QMM_ERR_ALIAS;
    }
    qmm::launch_moe_q8(gate_out, up_out, w_gate, w_up, expert_ids, pair_scale, xq, xd, t, n_used,
                       n_expert, in_f, n_ff, qtype, rb, tune, stream);
    return launch_status();
}

int qmm_nvfp4_repack_v2(void* dst, const void* src, int64_t rows, int64_t k, hipStream_t stream) {
    if (!dst || !src) return QMM_ERR_NULL;
    if (rows < 1 || k < 1) return QMM_ERR_SHAPE;
    if (k % 64 != 0) return QMM_ERR_K_ALIGN;
    if (!aligned(dst, 4) || !aligned(src, 4)) return QMM_ERR_ALIGN;
    int64_t bytes;
    if (!mul_ok(rows, k / 64 * 36, &bytes)) return QMM_ERR_SHAPE;
    const uintptr_t a = (uintptr_t)dst, b = (uintptr_t)src;
    if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes) return QMM_ERR_ALIAS;
    qmm::launch_nvfp4_repack_v2(dst, src, rows, k, stream);
    return launch_status();
}

int qmm_stream_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k, int qtype,
                        hipStream_t stream) {
    if (!sink) return QMM_ERR_NULL;
    int64_t rb;
    int st = check_weights(w, m, k, qtype, &rb);
    if (st) return st;
    if (!aligned(sink, 4)) return QMM_ERR_ALIGN;
    if (qmm::gemv_max_window_bytes(qtype, k, rb) >= ((int64_t)1 << 31)) return QMM_ERR_RANGE;
    qmm::GemvTuning tune;
    if (!gemv_tuning(&tune)) return QMM_ERR_RANGE;
    qmm::launch_loadonly(sink, w, m, k, qtype, rb, tune, stream);
    return launch_status();
}

}  // extern "C"
