// MoE projections on the streaming core (stream.hpp): the gate/up rows with
// per-expert de-duplication, on f32 or Q8_1 activations; the down
// projection and its slot sum; the Q8_1 quantization; the NVFP4 V2 repack.
#include "mstream.hpp"

namespace qmm {

// ------------------------------------------------------------------ MoE gate/up
// grid: x = work groups per (pair, plane) (their waves stride over the row
// groups of one expert's n_ff rows), y = pair p, z = plane (2: gate and up;
// 1: the down projection's single plane, or the fused SwiGLU mode, whose
// work groups stream the gate rows and then the up rows of the same row
// groups).
// The work groups of the FIRST pair routed to expert e gather every pair
// routed to e and apply e's rows to all their activation rows, so each
// selected expert's rows are read once per call when it has at most MOE_NT
// pairs (in chunks of MOE_NT otherwise), with the chunk's activations staged
// in LDS; the work groups of later pairs of the same expert exit after the
// check.  The decision depends on expert_ids only.  The activation row of
// pair q is its token's row q / n_used (gate/up) or its own row q
// (act_pair: the down projection, whose input is the pair's SwiGLU output).
constexpr int MOE_CHUNK = 256;  // pairs examined (and gathered) per pass
constexpr int MOE_NT = 3;       // token rows staged in LDS at a time (FMA stream)
constexpr int MOE_MT = 4;       // token rows of a matrix-core chunk
constexpr unsigned MOE_MIN_WG = 32;  // work groups per (pair, plane) at least

// Kernel modes: the projections per plane; the gate and up projections of
// each row fused with the SwiGLU/clamp activation; the two measurement
// twins of the per-plane mode (load-only and math-only arms).
enum : int { MOE_PLANES = 0, MOE_ACT = 1, MOE_LOADONLY = 2, MOE_MATHONLY = 3 };

struct MoeArgs {
    float* out0;            // gate_out (or the single plane's output, or act)
    float* out1;            // up_out
    const uint8_t* w0;      // gate (or the single) plane's rows
    const uint8_t* w1;      // up plane's rows
    const int* ids;
    const float* pscale;    // plane P's scales at P * n_pairs
    const float* x;         // f32 activation rows
    const int8_t* xq;       // Q8_1 codes and block scales (Q8 kernels)
    const float* xd;
    int t, n_used, n_expert, in_f, n_ff, rb, lpr_log2, n_rg;
    int xl;                 // f32 activations staged in LDS
    int act_pair;           // activation row of pair q is row q (else q / n_used)
    float limit;            // the SwiGLU clamp (MOE_ACT)
    int gbuf_off;           // floats of dynamic LDS before the gate buffer (MOE_ACT)
    int mt_min;             // chunks of at least mt_min pairs run on the matrix-core stream (0: none)
    int mld;                // row stride of the matrix-core chunk's staged activations
    int n_rg_m;             // row groups of the matrix-core stream
};

// The activation between gate/up and down: the gate clamped above at L, the
// up projection clamped to [-L, L], then silu(g) * u with silu(z) = z / (1 +
// exp(-z)) (a reading of the memra page's "preclamp" gate/up with argument
// 7.0, whose down arm consumes a SwiGLU output).  The comparisons keep a NaN
// projection NaN.
__device__ __forceinline__ float swiglu_clamp(float g, float u, float L) {
    const float gc = g > L ? L : g;
    const float uc = u > L ? L : (u < -L ? -L : u);
    return gc / (1.0f + expf(-gc)) * uc;
}

// The chunk [c0, c0 + NT) of the gathered pairs (absent slots repeat a real
// token): per-slot activation rows, pair numbers (-1: absent) and scales of
// plane `plane` (and, with both, of the up plane: MOE_ACT).
template <int NT>
struct Chunk {
    uint32_t row[NT];  // activation row of the slot
    int pj[NT];
    float f0[NT], f1[NT];
    __device__ __forceinline__ Chunk(const MoeArgs& a, const int* plist, const int* tlist, int c0, int cnt,
                                     int plane, bool both) {
        const int n_pairs = a.t * a.n_used;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int c = (c0 + j < cnt) ? c0 + j : c0;
            row[j] = (uint32_t)tlist[c];
            pj[j] = (c0 + j < cnt) ? plist[c] : -1;
            f0[j] = a.pscale[plane * n_pairs + plist[c]];
            f1[j] = both ? a.pscale[n_pairs + plist[c]] : 0.0f;
        }
    }
};

// Slot of (row, token j) in the work group's gate buffer (MOE_ACT): the
// same lane stores a row's gate value and reads it back in the up pass, so
// the index only has to be unique within the work group: row group rg is
// the q-th of wave `wave` (rg = blockIdx.x * 4 + wave + q * 4 * gridDim.x).
__device__ __forceinline__ int gate_slot(int64_t row, int j, int RG, int nt) {
    const int rg = (int)(row / RG);
    const int q = (rg - (int)blockIdx.x * 4 - wave_id()) / (4 * (int)gridDim.x);
    return ((q * 4 + wave_id()) * RG + (int)(row - (int64_t)rg * RG)) * nt + j;
}

// One chunk of pairs on f32 activations (XL: staged in LDS) or Q8_1
// activations (staged in LDS).  MOE_PLANES and the twins: the rows of plane
// blockIdx.z; MOE_ACT: the gate rows, then the up rows, then the activation.
template <int QT, int NT, int R, int D, bool XL, bool Q8, int MODE>
__device__ __forceinline__ void moe_chunk(const MoeArgs& a, int e, const int* plist, const int* tlist, int c0,
                                          int cnt) {
    const int wave = wave_id();
    const int plane = MODE == MOE_ACT ? 0 : (int)blockIdx.z;
    const Chunk<NT> ck(a, plist, tlist, c0, cnt, plane, MODE == MOE_ACT);
    const int64_t n_ff = a.n_ff;
    const int RG = (64 >> a.lpr_log2) * R;
    const StreamGeom g0{(plane == 0 ? a.w0 : a.w1) + (int64_t)e * n_ff * a.rb, n_ff, a.rb, a.in_f, a.lpr_log2};
    float* out = plane == 0 ? a.out0 : a.out1;
    constexpr int ARM = MODE == MOE_LOADONLY ? STREAM_LOADONLY : (MODE == MOE_MATHONLY ? STREAM_MATHONLY : STREAM_SERVED);
    auto store = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0) out[(int64_t)ck.pj[j] * n_ff + row] = ck.f0[j] * v;
    };
    float* gbuf = qmm_dyn_lds + a.gbuf_off;
    auto store_gate = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0) gbuf[gate_slot(row, j, RG, NT)] = ck.f0[j] * v;
    };
    auto store_act = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0)
            a.out0[(int64_t)ck.pj[j] * n_ff + row] =
                swiglu_clamp(gbuf[gate_slot(row, j, RG, NT)], ck.f1[j] * v, a.limit);
    };
    auto run = [&](const auto& xs, auto pre) {
        if constexpr (MODE == MOE_ACT) {
            const StreamGeom g1{a.w1 + (int64_t)e * n_ff * a.rb, n_ff, a.rb, a.in_f, a.lpr_log2};
            gemv_stream<QT, NT, R, D>(g0, blockIdx.x * 4 + wave, gridDim.x * 4, a.n_rg, xs, store_gate, pre);
            gemv_stream<QT, NT, R, D>(g1, blockIdx.x * 4 + wave, gridDim.x * 4, a.n_rg, xs, store_act);
        } else {
            gemv_stream<QT, NT, R, D, std::decay_t<decltype(xs)>, decltype(store), decltype(pre), ARM>(
                g0, blockIdx.x * 4 + wave, gridDim.x * 4, a.n_rg, xs, store, pre);
        }
    };
    const int n_rows = a.act_pair ? a.t * a.n_used : a.t;  // activation rows
    if constexpr (Q8) {
        const rsrc_t qr = make_rsrc(a.xq, (uint32_t)n_rows * (uint32_t)a.in_f);
        const rsrc_t dr = make_rsrc(a.xd, (uint32_t)n_rows * (uint32_t)(a.in_f / 32) * 4u);
        uint32_t qoff[NT], doff[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            qoff[j] = ck.row[j] * (uint32_t)a.in_f;
            doff[j] = ck.row[j] * (uint32_t)(a.in_f / 32) * 4u;
        }
        __syncthreads();  // the previous chunk's waves are done with the staged rows
        _Float16* sx = (_Float16*)qmm_dyn_lds;
        const XLdsQ8<NT> xs{sx, q8pad_len(a.in_f), (const float*)(sx + NT * q8pad_len(a.in_f)), a.in_f / 32};
        Q8Stage<NT> st{sx, qr, dr, {}, {}, a.in_f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            st.qoff[j] = qoff[j];
            st.doff[j] = doff[j];
        }
        run(xs, st);
    } else {
        const rsrc_t xr = make_rsrc(a.x, (uint32_t)n_rows * (uint32_t)a.in_f * 4u);
        uint32_t xoff[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) xoff[j] = ck.row[j] * (uint32_t)a.in_f * 4u;
        if constexpr (XL) {
            __syncthreads();  // the previous chunk's waves are done with the staged x
            constexpr bool SM = GUnit<QT>::RUNS > 0;
            const XLds<NT, SM> xs{qmm_dyn_lds, xpad_len(a.in_f), qmm_dyn_lds + NT * xpad_len(a.in_f), a.in_f >> 4};
            run(xs, make_xstage<NT, SM>(qmm_dyn_lds, xr, xoff, a.in_f));
        } else {
            XGlobal<NT> xs;
            xs.xr = xr;
#pragma unroll
            for (int j = 0; j < NT; ++j) xs.xoff[j] = xoff[j];
            run(xs, NoPre{});
        }
    }
}

// A chunk of up to MOE_MT pairs on the matrix-core stream (f32 activations
// staged in LDS in the quad layout); modes as moe_chunk.
template <int QT, int R, int D, int MODE>
__device__ __forceinline__ void moe_mchunk(const MoeArgs& a, int e, const int* plist, const int* tlist, int c0,
                                           int cnt) {
    constexpr int NT = MOE_MT;
    const int wave = wave_id();
    const int plane = MODE == MOE_ACT ? 0 : (int)blockIdx.z;
    const Chunk<NT> ck(a, plist, tlist, c0, cnt, plane, MODE == MOE_ACT);
    const int64_t n_ff = a.n_ff;
    const int RG = 4 * R;
    const StreamGeom g0{(plane == 0 ? a.w0 : a.w1) + (int64_t)e * n_ff * a.rb, n_ff, a.rb, a.in_f, 4};
    float* out = plane == 0 ? a.out0 : a.out1;
    constexpr int ARM = MODE == MOE_LOADONLY ? STREAM_LOADONLY : (MODE == MOE_MATHONLY ? STREAM_MATHONLY : STREAM_SERVED);
    auto store = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0) out[(int64_t)ck.pj[j] * n_ff + row] = ck.f0[j] * v;
    };
    float* gbuf = qmm_dyn_lds + a.gbuf_off;
    auto store_gate = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0) gbuf[gate_slot(row, j, RG, NT)] = ck.f0[j] * v;
    };
    auto store_act = [&](int64_t row, int j, float v) {
        if (row < n_ff && ck.pj[j] >= 0)
            a.out0[(int64_t)ck.pj[j] * n_ff + row] =
                swiglu_clamp(gbuf[gate_slot(row, j, RG, NT)], ck.f1[j] * v, a.limit);
    };
    const int n_rows = a.act_pair ? a.t * a.n_used : a.t;  // activation rows
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)n_rows * (uint32_t)a.in_f * 4u);
    uint32_t xoff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xoff[j] = ck.row[j] * (uint32_t)a.in_f * 4u;
    __syncthreads();  // the previous chunk's waves are done with the staged rows
    float* sx = qmm_dyn_lds;
    const int nreal = cnt - c0 < NT ? cnt - c0 : NT;
    const XQuad<1> xq = make_xquad<1>(sx, a.mld, a.in_f, nreal);
    const auto st = make_qstage<NT, MTraits<QT>::RUN>(sx, xr, xoff, a.in_f, a.mld, nreal);
    const int first = blockIdx.x * 4 + wave, stride = gridDim.x * 4;
    const int n_iter = first < a.n_rg_m ? (a.n_rg_m - first + stride - 1) / stride : 0;
    if constexpr (MODE == MOE_ACT) {
        const StreamGeom g1{a.w1 + (int64_t)e * n_ff * a.rb, n_ff, a.rb, a.in_f, 4};
        mfma_stream<QT, 1, R, D, 1>(g0, first, stride, a.n_rg_m, n_iter, 0, nullptr, xq, store_gate, st);
        mfma_stream<QT, 1, R, D, 1>(g1, first, stride, a.n_rg_m, n_iter, 0, nullptr, xq, store_act);
    } else {
        mfma_stream<QT, 1, R, D, 1, decltype(store), std::decay_t<decltype(st)>, ARM>(
            g0, first, stride, a.n_rg_m, n_iter, 0, nullptr, xq, store, st);
    }
}

// Chunk paths compiled into a kernel (its registers are those of its
// heaviest path, so fewer paths fit more waves per SIMD):
// MOE_K_SINGLE: every chunk is one pair on the FMA stream (the launch for one
//   token, whose pairs go to distinct experts);
// MOE_K_LEAN: chunks of two or more pairs on the matrix-core stream, single
//   pairs on the FMA stream (QMM_MOE_MFMA_MIN 1 or 2);
// MOE_K_FULL: chunks of 1..3 pairs on the FMA stream, or on Q8_1 codes, and
//   the matrix-core chunks from a.mt_min pairs up when it is set.
enum : int { MOE_K_SINGLE = 0, MOE_K_LEAN = 1, MOE_K_FULL = 2 };

template <int QT, int R, int D, bool Q8, int MODE, int KIND>
__global__ __launch_bounds__(256) void moe_kernel(MoeArgs a) {
    constexpr bool SINGLE = KIND == MOE_K_SINGLE;
    __shared__ int plist[MOE_CHUNK];
    __shared__ int tlist[MOE_CHUNK];
    __shared__ int wcnt[4];
    __shared__ int s_seen;
    const int n_pairs = a.t * a.n_used;
    const int p = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int e = uniform_i32(a.ids[p]);

    // Is p the first pair routed to e?
    if (tid == 0) s_seen = 0;
    __syncthreads();
    for (int q0 = 0; q0 < p; q0 += MOE_CHUNK) {
        const int q = q0 + tid;
        if (q < p && a.ids[q] == e) s_seen = 1;
    }
    __syncthreads();
    if (s_seen) return;

    const int RG = (64 >> a.lpr_log2) * R;
    if (e < 0 || e >= a.n_expert) {  // invalid id: poison every pair that carries it
        float* out = MODE == MOE_ACT || blockIdx.z == 0 ? a.out0 : a.out1;
        for (int q = p; q < n_pairs; ++q) {
            if (a.ids[q] != e) continue;
            for (int rg = blockIdx.x; rg < a.n_rg; rg += gridDim.x)
                for (int r = tid; r < RG; r += 256) {
                    const int64_t row = (int64_t)rg * RG + r;
                    if (row < a.n_ff) out[(int64_t)q * a.n_ff + row] = __builtin_nanf("");
                }
        }
        return;
    }

    for (int q0 = p; q0 < n_pairs; q0 += MOE_CHUNK) {
        // gather the pairs of this chunk routed to e, in pair order
        const int q = q0 + tid;
        const bool hit = q < n_pairs && a.ids[q] == e;
        const uint64_t bal = __ballot(hit);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        __syncthreads();
        if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int off = 0;
        for (int wv = 0; wv < wave; ++wv) off += wcnt[wv];
        if (hit) {
            plist[off + before] = q;
            tlist[off + before] = a.act_pair ? q : q / a.n_used;  // activation row
        }
        const int cnt = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        __syncthreads();
        if constexpr (SINGLE) {
            for (int c0 = 0; c0 < cnt; ++c0) {
                if (Q8 || a.xl) moe_chunk<QT, 1, R, D, true, Q8, MODE>(a, e, plist, tlist, c0, cnt);
                else if constexpr (!Q8) moe_chunk<QT, 1, R, 2, false, Q8, MODE>(a, e, plist, tlist, c0, cnt);
            }
            continue;
        }
        if constexpr (KIND == MOE_K_LEAN && !Q8) {
            for (int c0 = 0; c0 < cnt;) {
                if (cnt - c0 >= a.mt_min) {
                    moe_mchunk<QT, R, D, MODE>(a, e, plist, tlist, c0, cnt);
                    c0 += MOE_MT;
                } else {
                    if (a.xl) moe_chunk<QT, 1, R, D, true, Q8, MODE>(a, e, plist, tlist, c0, cnt);
                    else moe_chunk<QT, 1, R, 2, false, Q8, MODE>(a, e, plist, tlist, c0, cnt);
                    ++c0;
                }
            }
            continue;
        }
        for (int c0 = 0; c0 < cnt;) {
            const int left = cnt - c0;
            if constexpr (!Q8) {
                if (a.mt_min > 0 && left >= a.mt_min) {
                    moe_mchunk<QT, R, D, MODE>(a, e, plist, tlist, c0, cnt);
                    c0 += MOE_MT;
                    continue;
                }
            }
            if (Q8 || a.xl) {
                if (left == 1)
                    moe_chunk<QT, 1, R, D, true, Q8, MODE>(a, e, plist, tlist, c0, cnt);
                else if (left == 2)
                    moe_chunk<QT, 2, R, D, true, Q8, MODE>(a, e, plist, tlist, c0, cnt);
                else
                    moe_chunk<QT, 3, R, D, true, Q8, MODE>(a, e, plist, tlist, c0, cnt);
            } else if constexpr (!Q8) {  // Q8_1 activations are always staged
                moe_chunk<QT, MOE_NT, R, 2, false, Q8, MODE>(a, e, plist, tlist, c0, cnt);
            }
            c0 += MOE_NT;
        }
    }
}

// ------------------------------------------------------------------ launchers

// Largest dynamic LDS one MoE work group takes: the staged activations (at
// most XLDS_MAX_BYTES) plus, in MOE_ACT, the gate buffer.
constexpr int64_t MOE_LDS_MAX = 96 * 1024;
// Largest staged activations of a matrix-core chunk (four rows of up to
// about 4.4K activations: two work groups per CU).
constexpr int64_t MOE_MT_LDS_MAX = 76 * 1024;

// The MoE kernels run two rows per lane group and two items in flight per
// wave (the streaming defaults measured best on MI355X); QMM_GEMV_ROWS and
// QMM_GEMV_DEPTH tune the GEMV only.
template <int QT, bool Q8, int MODE>
static void launch_moe_mode(MoeArgs a, int planes, const GemvTuning& tune, hipStream_t st) {
    {
        constexpr int R = 2, D = 2;
        // lane groups small enough that each lane takes at least 8 units of
        // its row between two lane-group reductions (not below 8 lanes): the
        // down projection's 64-unit rows (n_ff = 2048 NVFP4) in 8-lane
        // groups, t = 16: 99.5 -> 97.8 us (V2 rows 87.0 -> 85.6), t = 1 equal;
        // the gate/up's 128-unit rows keep 16 lanes (8 lanes: 19.8 against
        // 19.5 us at t = 1)
        int l = lpr_for(QT, a.in_f, tune.moe_lpr_cap);
        const int64_t units = (a.in_f + unit_elems_of(QT) - 1) / unit_elems_of(QT);
        while (l > LPR_CAP_MIN && (1 << l) > min_lpr(QT) && (units >> l) < 8) --l;
        const int64_t n_pairs = (int64_t)a.t * a.n_used;
        const int64_t RG = rg_rows(l, R);
        const int64_t n_rg = (a.n_ff + RG - 1) / RG;
        // at most one set of work groups per distinct expert and plane is
        // active; with many pairs the sets are not all distinct, so each set
        // gets at least MOE_MIN_WG work groups
        const int64_t active = planes * (n_pairs < a.n_expert ? n_pairs : a.n_expert);
        GemvTuning mt = tune;
        mt.wg_per_cu = tune.moe_wg_per_cu;
        unsigned gx = stream_grid(n_rg, active, mt);
        const unsigned need = (unsigned)((n_rg + 3) / 4);
        if (gx < MOE_MIN_WG) gx = need < MOE_MIN_WG ? need : MOE_MIN_WG;
        // one token: single-pair chunks (the SINGLE kernel), one staged row
        const int ntc = a.t == 1 ? 1 : MOE_NT;
        int64_t xbytes = Q8 ? (int64_t)q8lds_bytes(ntc, a.in_f)
                            : (int64_t)xlds_floats(ntc, a.in_f, GUnit<QT>::RUNS > 0) * 4;
        a.xl = Q8 || xbytes <= XLDS_MAX_BYTES;
        if (!a.xl) xbytes = 0;
        // chunks of several pairs on the matrix-core stream: with more than
        // one activation row (one token's pairs go to distinct experts), f32
        // activations, and MOE_MT staged rows within the LDS limit
        const int lm = mtraits_lm(QT);
        const int64_t mbytes = (int64_t)qlds_floats(MOE_MT, a.in_f, lm, MTraits<QT>::RUN) * 4;
        const int64_t RGM = 4 * R;
        const int64_t n_rg_m = (a.n_ff + RGM - 1) / RGM;
        a.mt_min = !Q8 && a.t > 1 && mbytes <= MOE_MT_LDS_MAX ? tune.moe_mfma_min : 0;
        a.mld = qld(a.in_f, lm);
        a.n_rg_m = (int)n_rg_m;
        if (a.mt_min > 0 && mbytes > xbytes) xbytes = mbytes;
        int64_t lds = xbytes;
        a.gbuf_off = 0;
        if constexpr (MODE == MOE_ACT) {
            // the gate buffer after the staged activations: a value per row
            // group the work group streams, per row and token slot; more work
            // groups (fewer row groups each) until it fits
            a.gbuf_off = (int)((xbytes + 15) / 16 * 4);
            auto gbytes = [&](unsigned w) {
                const int64_t fma = (n_rg + 4 * (int64_t)w - 1) / (4 * (int64_t)w) * 4 * RG * ntc * 4;
                const int64_t mat = a.mt_min > 0 ? (n_rg_m + 4 * (int64_t)w - 1) / (4 * (int64_t)w) * 4 * RGM * MOE_MT * 4 : 0;
                return fma > mat ? fma : mat;
            };
            while (gx < need && 4 * (int64_t)a.gbuf_off + gbytes(gx) > MOE_LDS_MAX) gx = gx * 2 < need ? gx * 2 : need;
            lds = 4 * (int64_t)a.gbuf_off + gbytes(gx);
        }
        a.lpr_log2 = l;
        a.n_rg = (int)n_rg;
        const dim3 grid(gx, (unsigned)n_pairs, (unsigned)(MODE == MOE_ACT ? 1 : planes));
        if (a.t == 1) moe_kernel<QT, R, D, Q8, MODE, MOE_K_SINGLE><<<grid, 256, (size_t)lds, st>>>(a);
        else if (!Q8 && (a.mt_min == 1 || a.mt_min == 2))
            moe_kernel<QT, R, D, Q8, MODE, MOE_K_LEAN><<<grid, 256, (size_t)lds, st>>>(a);
        else moe_kernel<QT, R, D, Q8, MODE, MOE_K_FULL><<<grid, 256, (size_t)lds, st>>>(a);
    }
}

static MoeArgs moe_args(float* o0, float* o1, const void* w0, const void* w1, const int* ids, const float* sc,
                        const float* x, const int8_t* xq, const float* xd, int64_t t, int64_t n_used,
                        int64_t n_expert, int64_t in_f, int64_t n_ff, int64_t rb, int act_pair, float limit) {
    MoeArgs a{};
    a.out0 = o0;
    a.out1 = o1;
    a.w0 = (const uint8_t*)w0;
    a.w1 = (const uint8_t*)w1;
    a.ids = ids;
    a.pscale = sc;
    a.x = x;
    a.xq = xq;
    a.xd = xd;
    a.t = (int)t;
    a.n_used = (int)n_used;
    a.n_expert = (int)n_expert;
    a.in_f = (int)in_f;
    a.n_ff = (int)n_ff;
    a.rb = (int)rb;
    a.act_pair = act_pair;
    a.limit = limit;
    return a;
}

void launch_moe(float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                const float* x, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                int64_t n_ff, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(g, u, wg, wu, ids, sc, x, nullptr, nullptr, t, n_used, n_expert, in_f, n_ff, rb, 0, 0.f);
    QMM_QT_SWITCH(qt, (launch_moe_mode<Q, false, MOE_PLANES>(a, 2, tune, st)))
}

void launch_moe_act(float* act, const void* wg, const void* wu, const int* ids, const float* sc, const float* x,
                    int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int qt, int64_t rb,
                    float limit, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(act, nullptr, wg, wu, ids, sc, x, nullptr, nullptr, t, n_used, n_expert, in_f, n_ff,
                               rb, 0, limit);
    QMM_QT_SWITCH(qt, (launch_moe_mode<Q, false, MOE_ACT>(a, 1, tune, st)))
}

void launch_moe_probe(int arm, float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                      const float* x, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff,
                      int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(g, u, wg, wu, ids, sc, x, nullptr, nullptr, t, n_used, n_expert, in_f, n_ff, rb, 0, 0.f);
    if (qt == QT_NVFP4) {
        if (arm == 1) launch_moe_mode<QT_NVFP4, false, MOE_LOADONLY>(a, 2, tune, st);
        else launch_moe_mode<QT_NVFP4, false, MOE_MATHONLY>(a, 2, tune, st);
    } else if (qt == QT_NVFP4_V2) {
        if (arm == 1) launch_moe_mode<QT_NVFP4_V2, false, MOE_LOADONLY>(a, 2, tune, st);
        else launch_moe_mode<QT_NVFP4_V2, false, MOE_MATHONLY>(a, 2, tune, st);
    }
}

// ------------------------------------------------------------------ Q8_1 activations
int64_t moe_q8_lds_bytes(int64_t in_f) { return q8lds_bytes(MOE_NT, (int)in_f); }

void launch_moe_q8(float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                   const int8_t* xq, const float* xd, int64_t t, int64_t n_used, int64_t n_expert,
                   int64_t in_f, int64_t n_ff, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(g, u, wg, wu, ids, sc, nullptr, xq, xd, t, n_used, n_expert, in_f, n_ff, rb, 0, 0.f);
    if (qt == QT_NVFP4) launch_moe_mode<QT_NVFP4, true, MOE_PLANES>(a, 2, tune, st);
    else if (qt == QT_NVFP4_V2) launch_moe_mode<QT_NVFP4_V2, true, MOE_PLANES>(a, 2, tune, st);
}

void launch_moe_act_q8(float* act, const void* wg, const void* wu, const int* ids, const float* sc,
                       const int8_t* xq, const float* xd, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                       int64_t n_ff, int qt, int64_t rb, float limit, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(act, nullptr, wg, wu, ids, sc, nullptr, xq, xd, t, n_used, n_expert, in_f, n_ff, rb, 0,
                               limit);
    if (qt == QT_NVFP4) launch_moe_mode<QT_NVFP4, true, MOE_ACT>(a, 1, tune, st);
    else if (qt == QT_NVFP4_V2) launch_moe_mode<QT_NVFP4_V2, true, MOE_ACT>(a, 1, tune, st);
}

// Q8_1 quantization, one thread per block of 32 activations: d = max|x| /
// 127 and q = round-half-away(x * (1/d)) (0 when d = 0), in f32.
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(int8_t* __restrict__ q, float* __restrict__ d,
                                                            const float* __restrict__ x, int64_t nblk) {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
        const f32x4* xp = (const f32x4*)(x + 32 * b);
        f32x4 v[8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = xp[i];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        }
        const float dd = amax / 127.0f;
        const float id = dd != 0.0f ? 1.0f / dd : 0.0f;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c0 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].x * id);
            const uint32_t c1 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].y * id);
            const uint32_t c2 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].z * id);
            const uint32_t c3 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].w * id);
            w[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        }
        *(u32x4*)(q + 32 * b) = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4*)(q + 32 * b + 16) = u32x4{w[4], w[5], w[6], w[7]};
        d[b] = dd;
    }
}

void launch_quantize_q8_1(int8_t* q, float* d, const float* x, int64_t nblk, hipStream_t st) {
    int64_t blocks = (nblk + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    quantize_q8_1_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(q, d, x, nblk);
}

// ------------------------------------------------------------------ MoE down
// y[tau*d + r] = sum over s < n_used, in order, of pair_out[(tau*n_used + s)*d + r].
// One thread per four consecutive outputs when d is a multiple of 4.
template <int V>
__global__ __launch_bounds__(256) void moe_slot_sum_kernel(float* __restrict__ y,
                                                           const float* __restrict__ pair_out,
                                                           int64_t t, int n_used, int64_t d) {
    const int64_t nv = t * d / V;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
        const int64_t tau = i * V / d, r = i * V - tau * d;
        const float* src = pair_out + tau * n_used * d + r;
        // slots in order 0, 1, ...; the loads of up to 8 slots are issued
        // before their sums, so their latencies overlap
        using T = typename std::conditional<V == 4, f32x4, float>::type;
        T acc = *(const T*)src;
        for (int s0 = 1; s0 < n_used; s0 += 8) {
            T v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n_used) v[u] = *(const T*)(src + (int64_t)(s0 + u) * d);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n_used) acc += v[u];
        }
        *(T*)(y + i * V) = acc;
    }
}

static void launch_slot_sum(float* y, float* pair_out, int64_t t, int64_t n_used, int64_t d_model, hipStream_t st) {
    const bool v4 = (d_model & 3) == 0 && ((uintptr_t)y & 15) == 0 && ((uintptr_t)pair_out & 15) == 0;
    const int64_t nv = t * d_model / (v4 ? 4 : 1);
    int64_t blocks = (nv + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (v4)
        moe_slot_sum_kernel<4><<<dim3((unsigned)blocks), 256, 0, st>>>(y, pair_out, t, (int)n_used, d_model);
    else
        moe_slot_sum_kernel<1><<<dim3((unsigned)blocks), 256, 0, st>>>(y, pair_out, t, (int)n_used, d_model);
}

void launch_moe_down(float* y, float* pair_out, const void* wd, const int* ids, const float* sc,
                     const float* act, int64_t t, int64_t n_used, int64_t n_expert, int64_t n_ff,
                     int64_t d_model, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(pair_out, pair_out, wd, wd, ids, sc, act, nullptr, nullptr, t, n_used, n_expert, n_ff,
                               d_model, rb, 1, 0.f);
    QMM_QT_SWITCH(qt, (launch_moe_mode<Q, false, MOE_PLANES>(a, 1, tune, st)))
    launch_slot_sum(y, pair_out, t, n_used, d_model, st);
}

void launch_moe_down_q8(float* y, float* pair_out, const void* wd, const int* ids, const float* sc,
                        const int8_t* aq, const float* ad, int64_t t, int64_t n_used, int64_t n_expert, int64_t n_ff,
                        int64_t d_model, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const MoeArgs a = moe_args(pair_out, pair_out, wd, wd, ids, sc, nullptr, aq, ad, t, n_used, n_expert, n_ff,
                               d_model, rb, 1, 0.f);
    if (qt == QT_NVFP4) launch_moe_mode<QT_NVFP4, true, MOE_PLANES>(a, 1, tune, st);
    else if (qt == QT_NVFP4_V2) launch_moe_mode<QT_NVFP4_V2, true, MOE_PLANES>(a, 1, tune, st);
    launch_slot_sum(y, pair_out, t, n_used, d_model, st);
}

// ------------------------------------------------------------------ V2 repack
// NVFP4 rows -> NVFP4 V2 rows.  Item (row, G): the 36 bytes of group G are
// its scale word and 32 quant bytes; the quant bytes go to 32G and the scale
// word to k/2 + 4G of the same row (9 dword loads, 9 dword stores).
__global__ __launch_bounds__(256) void nvfp4_repack_v2_kernel(uint32_t* __restrict__ dst,
                                                              const uint32_t* __restrict__ src,
                                                              int64_t rows, int64_t k) {
    const int64_t groups = k / 64, rw = groups * 9;  // dwords per row
    const int64_t items = rows * groups;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < items; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / groups, G = i - r * groups;
        const uint32_t* s = src + r * rw + 9 * G;
        uint32_t* d = dst + r * rw;
        uint32_t v[9];
#pragma unroll
        for (int j = 0; j < 9; ++j) v[j] = s[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) d[8 * G + j] = v[1 + j];
        d[8 * groups + G] = v[0];
    }
}

void launch_nvfp4_repack_v2(void* dst, const void* src, int64_t rows, int64_t k, hipStream_t st) {
    const int64_t items = rows * (k / 64);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    nvfp4_repack_v2_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src,
                                                                   rows, k);
}

}  // namespace qmm
