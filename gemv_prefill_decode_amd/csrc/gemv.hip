// Decode path: the f32 GEMV for small n (on f32 FMAs, or for several
// activation rows on the matrix-core stream) and its load-only twin (the
// streaming cores, units and activation staging are in stream.hpp and
// mstream.hpp).
#include "mstream.hpp"

namespace qmm {

// grid: x = work groups (their 4 waves stride over the row groups), y = token
// groups of NT.  XL: activations staged in LDS (dynamic shared memory of
// xlds_floats(NT, k, RUNS > 0) floats).
template <int QT, int NT, int R, int D, bool XL, int WPG = 4>
__global__ __launch_bounds__(64 * WPG) void gemv_kernel(float* __restrict__ dst,
                                                        const uint8_t* __restrict__ w,
                                                        const float* __restrict__ x, int m, int k,
                                                        int n, int rb, int lpr_log2, int n_rg, int ldx,
                                                        int ldd) {
    const int wave = wave_id();
    const int tok0 = blockIdx.y * NT;
    const int ntok = min(NT, n - tok0);
    // token rows ldx floats apart; the window ends with the last row's k floats
    const rsrc_t xr = make_rsrc(x + (int64_t)tok0 * ldx,
                                ((uint32_t)(ntok - 1) * (uint32_t)ldx + (uint32_t)k) * 4u);
    uint32_t xoff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xoff[j] = (uint32_t)(j < ntok ? j : 0) * (uint32_t)ldx * 4u;
    const StreamGeom g{w, m, rb, k, lpr_log2};
    float* out = dst + (int64_t)tok0 * ldd;
    auto store = [&](int64_t row, int j, float v) {
        if (row < m && j < ntok) out[(int64_t)j * ldd + row] = v;
    };
    if constexpr (XL) {
        constexpr bool SM = GUnit<QT>::RUNS > 0;
        const XLds<NT, SM> xs{qmm_dyn_lds, xpad_len(k), qmm_dyn_lds + NT * xpad_len(k), k >> 4};
        gemv_stream<QT, NT, R, D>(g, blockIdx.x * WPG + wave, gridDim.x * WPG, n_rg, xs, store,
                                  make_xstage<NT, SM, 64 * WPG>(qmm_dyn_lds, xr, xoff, k));
    } else {
        XGlobal<NT> xs;
        xs.xr = xr;
#pragma unroll
        for (int j = 0; j < NT; ++j) xs.xoff[j] = xoff[j];
        gemv_stream<QT, NT, R, D>(g, blockIdx.x * WPG + wave, gridDim.x * WPG, n_rg, xs, store);
    }
}

// The matrix-core stream: grid x = work groups of WPG waves, y = token
// groups of 4 * TT rows, staged in LDS in the quad layout (qlds_floats(4 *
// TT, k, lm, MTraits::RUN) floats, row stride mld), then the KW-wave partial
// sums (2 * WPG * 16 R TT floats).  The work group's WPG / KW row-group
// slots take row groups blockIdx.x * (WPG / KW) + slot + j * gridDim.x *
// (WPG / KW).
template <int QT, int TT, int R, int D, int KW, int WPG>
__global__ __launch_bounds__(64 * WPG) void gemv_mfma_kernel(float* __restrict__ dst, const uint8_t* __restrict__ w,
                                                             const float* __restrict__ x, int m, int k, int n,
                                                             int rb, int n_rg, int ldx, int ldd, int mld) {
    constexpr int NTOK = 4 * TT, S = WPG / KW;
    const int wave = wave_id();
    const int tok0 = blockIdx.y * NTOK;
    const int ntok = min(NTOK, n - tok0);
    const rsrc_t xr = make_rsrc(x + (int64_t)tok0 * ldx,
                                ((uint32_t)(ntok - 1) * (uint32_t)ldx + (uint32_t)k) * 4u);
    uint32_t xoff[NTOK];
#pragma unroll
    for (int j = 0; j < NTOK; ++j) xoff[j] = (uint32_t)(j < ntok ? j : 0) * (uint32_t)ldx * 4u;
    const StreamGeom g{w, m, rb, k, 4};
    float* out = dst + (int64_t)tok0 * ldd;
    auto store = [&](int64_t row, int j, float v) {
        if (row < m && j < ntok) out[(int64_t)j * ldd + row] = v;
    };
    float* sx = qmm_dyn_lds;
    const XQuad<TT> xq = make_xquad<TT>(sx, mld, k, ntok);
    float* red = sx + qlds_floats(NTOK, k, MTraits<QT>::LM, MTraits<QT>::RUN);
    const int wg_first = (int)blockIdx.x * S, stride = (int)gridDim.x * S;
    const int n_iter = wg_first < n_rg ? (n_rg - wg_first + stride - 1) / stride : 0;  // the same for every wave
    mfma_stream<QT, TT, R, D, KW>(g, wg_first + wave / KW, stride, n_rg, n_iter, wave % KW, red, xq, store,
                                  make_qstage<NTOK, MTraits<QT>::RUN, 64 * WPG>(sx, xr, xoff, k, mld, ntok));
}

// ------------------------------------------------------------------ load-only twin
// (raw_xor, the checksum of a unit's raw words, is in stream.hpp)
template <int QT, int R, int D>
__global__ __launch_bounds__(256) void loadonly_kernel(uint32_t* __restrict__ sink,
                                                       const uint8_t* __restrict__ w, int m, int k,
                                                       int rb, int lpr_log2, int n_rg) {
    using UT = GUnit<QT>;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const StreamGeom g{w, m, rb, k, lpr_log2};
    const int lpr = 1 << lpr_log2;
    const int gl = lane & (lpr - 1), slot = lane >> lpr_log2;
    const int RG = (64 >> lpr_log2) * R;
    const int U = (k + UT::UE - 1) / UT::UE;
    const int upl = (U + lpr - 1) >> lpr_log2;
    const int first_rg = blockIdx.x * 4 + wave, rg_stride = gridDim.x * 4;
    const int n_items = first_rg < n_rg ? (n_rg - first_rg + rg_stride - 1) / rg_stride * upl : 0;
    const typename UT::Lane ln = UT::lane(gl);
    const uint32_t lane_row_off = (uint32_t)(slot * R) * (uint32_t)rb;
    const int e_step = lpr * UT::UE;
    uint32_t acc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) acc[rr] = 0;
    auto finish = [&](int q) {
        for (int off = lpr >> 1; off > 0; off >>= 1)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) acc[rr] ^= __shfl_xor(acc[rr], off, 64);
        if (gl == 0)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const int64_t row = (int64_t)(first_rg + q * rg_stride) * RG + slot * R + rr;
                if (row < m) sink[row] = acc[rr];
            }
#pragma unroll
        for (int rr = 0; rr < R; ++rr) acc[rr] = 0;
    };
    UT ring[D][R];
    if (n_items <= D) {  // short stream, as in gemv_stream
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < n_items) {
                const int q = d / upl, uu = d - q * upl;
                issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + q * rg_stride, uu,
                                  ln.e + uu * e_step, true);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < n_items) {
                const int q = d / upl, uu = d - q * upl;
                if (gl + lpr * uu < U)
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) acc[rr] ^= raw_xor(ring[d][rr]);
                if (uu == upl - 1) finish(q);
            }
        }
        return;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int q = d / upl, uu = d - q * upl;
        issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + q * rg_stride, uu,
                          ln.e + uu * e_step, true);
    }
    ItemPos cur{0, 0}, nxt{D / upl, D - (D / upl) * upl};
    for (int base = 0; base < n_items; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = base + d;
            const bool live = it < n_items;
            const int q = cur.q, uu = cur.uu;
            if (live && gl + lpr * uu < U)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) acc[rr] ^= raw_xor(ring[d][rr]);
            issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + nxt.q * rg_stride, nxt.uu,
                              ln.e + nxt.uu * e_step, it + D < n_items);
            if (live && uu == upl - 1) finish(q);
            cur.next(upl);
            nxt.next(upl);
        }
    }
}

// ------------------------------------------------------------------ launchers

int gemv_unit_elems(int qt) { return unit_elems_of(qt); }

int64_t gemv_max_window_bytes(int qt, int64_t k, int64_t rb) {
    // the smaller lane groups give the taller row groups
    return rg_rows(lpr_for(qt, k, LPR_CAP_MIN), 2) * rb + 16;
}

template <int QT, int NT>
static void launch_gemv_nt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k,
                           int64_t n, int64_t rb, int64_t ldx, int64_t ldd, const GemvTuning& tune,
                           hipStream_t st) {
    with_rd<NT>(tune, [&](auto Rc, auto Dc) {
        constexpr int R = decltype(Rc)::value, D = decltype(Dc)::value;
        int l = lpr_for(QT, k, LPR_CAP_SINGLE);
        if (n > 2) {
            const int lmin = lpr_for(QT, k, LPR_CAP_MULTI);
            while (l > lmin && (m + rg_rows(l - 1, R) - 1) / rg_rows(l - 1, R) >= 4 * (int64_t)tune.num_cu) --l;
        }
        const int64_t n_rg = (m + rg_rows(l, R) - 1) / rg_rows(l, R);
        const int64_t gy = (n + NT - 1) / NT;
        const int64_t lds = (int64_t)xlds_floats(NT, (int)k, GUnit<QT>::RUNS > 0) * 4;
        if (lds <= tune.lds_per_wg) {
            const GemvTuning lt = lds_limited(tune, lds);
            if (lt.wg_per_cu <= 2) {
                // one or two work groups per CU: 8 waves share the staged rows
                const dim3 grid(stream_grid(n_rg, gy, lt, 8), (unsigned)gy);
                gemv_kernel<QT, NT, R, D, true, 8><<<grid, 512, (size_t)lds, st>>>(
                    dst, w, x, (int)m, (int)k, (int)n, (int)rb, l, (int)n_rg, (int)ldx, (int)ldd);
            } else {
                const dim3 grid(stream_grid(n_rg, gy, lt), (unsigned)gy);
                gemv_kernel<QT, NT, R, D, true><<<grid, 256, (size_t)lds, st>>>(
                    dst, w, x, (int)m, (int)k, (int)n, (int)rb, l, (int)n_rg, (int)ldx, (int)ldd);
            }
        } else {
            const dim3 grid(stream_grid(n_rg, gy, tune), (unsigned)gy);
            gemv_kernel<QT, NT, R, D, false><<<grid, 256, 0, st>>>(
                dst, w, x, (int)m, (int)k, (int)n, (int)rb, l, (int)n_rg, (int)ldx, (int)ldd);
        }
    });
}

// Launch shape of the matrix-core stream with token groups of 4 * TT rows
// and R rows per lane.  With at least four row groups per CU, one wave per
// row group (KW = 1), 8-wave work groups where the LDS holds at most two per
// CU, else 4-wave ones.  With fewer row groups and rows of at least 4 unit
// iterations, KW = 4 or 8 waves share a row group (one row group per work
// group at KW = 8), which costs a barrier per row group but fills the CUs:
// 1024x4608 Q4_0, n = 4: 17.7 -> 7.8 us; on 14336x4096 and 4608x1024 the
// barriers made it slower than KW = 1.  iters: row-group passes of the
// busiest work group.
struct MStreamLaunch {
    int64_t lds, n_rg, gy, iters;
    int kw, wpg, mld;
    unsigned grid;
};

template <int QT, int TT, int R>
static MStreamLaunch mstream_launch(int64_t m, int64_t k, int64_t n, const GemvTuning& tune) {
    MStreamLaunch p{};
    const int lm = MTraits<QT>::LM;
    p.lds = ((int64_t)qlds_floats(4 * TT, (int)k, lm, MTraits<QT>::RUN) + 2 * 8 * 16 * R * TT) * 4;  // partial sums sized for 8 waves
    p.mld = qld((int)k, lm);
    p.n_rg = (m + 4 * R - 1) / (4 * R);
    p.gy = (n + 4 * TT - 1) / (4 * TT);
    const GemvTuning lt = lds_limited(tune, p.lds);
    const int64_t units = (k + GUnit<QT>::UE - 1) / GUnit<QT>::UE;
    const int64_t upl = (units + 15) / 16;
    p.kw = p.n_rg >= 4 * (int64_t)lt.num_cu || upl < 4 ? 1 : (upl < 8 ? 4 : 8);
    p.wpg = p.kw > 1 || lt.wg_per_cu <= 2 ? 8 : 4;
    const int64_t slots = p.wpg / p.kw;
    p.grid = stream_grid(p.n_rg, p.gy, lt, (int)slots);
    p.iters = (p.n_rg + (int64_t)p.grid * slots - 1) / ((int64_t)p.grid * slots);
    return p;
}

// false if the launch does not fit one work group's LDS
template <int QT, int TT, int R>
static bool launch_gemv_mfma_r(const MStreamLaunch& p, float* dst, const uint8_t* w, const float* x, int64_t m,
                               int64_t k, int64_t n, int64_t rb, int64_t ldx, int64_t ldd, const GemvTuning& tune,
                               hipStream_t st) {
    constexpr int D = 2;
    if (p.lds > tune.lds_per_wg) return false;
    auto go = [&](auto KWc, auto WPGc) {
        constexpr int KW = decltype(KWc)::value, WPG = decltype(WPGc)::value;
        gemv_mfma_kernel<QT, TT, R, D, KW, WPG><<<dim3(p.grid, (unsigned)p.gy), 64 * WPG, (size_t)p.lds, st>>>(
            dst, w, x, (int)m, (int)k, (int)n, (int)rb, (int)p.n_rg, (int)ldx, (int)ldd, p.mld);
    };
    using I1 = std::integral_constant<int, 1>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    if (p.kw == 4) go(I4{}, I8{});
    else if (p.kw == 8) go(I8{}, I8{});
    else if (p.wpg == 8) go(I1{}, I8{});
    else go(I1{}, I4{});
    return true;
}

// Rows per lane R: one for Q6_K (row groups of 4 rows: twice the work
// groups, and its scaled sub-units keep more registers per row), two for f32
// rows.  For the other formats one row only where it shortens the rows the
// busiest wave streams (its row-group passes times R) to under three
// quarters of the two-row figure, and never with four or more row groups of
// 8 rows per CU.  Measured (graph replays, one row against two): 14336x4096
// Q6_K n = 8 / 32: 28.4 / 75.7 against 30.3 / 89.1 us; 4608x1024 Q4_K
// n = 16: 9.0 against 10.4; 1024x4608 Q4_0 n = 4: 6.4 against 7.8, but
// n = 8 / 32, with as many passes: 8.1 / 18.7 against 7.8 / 16.5; 4608x1024
// Q4_K n = 24, two passes against one: 13.4 against 10.5; 14336x4096 Q4_K
// n = 16: 55.4 against 46.8; f32 3072x1024 n = 32: 18.6 against 12.6.
template <int QT, int TT>
static bool launch_gemv_mfma(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k, int64_t n,
                             int64_t rb, int64_t ldx, int64_t ldd, const GemvTuning& tune, hipStream_t st) {
    if constexpr (QT == QT_Q6_K) {
        const MStreamLaunch p1 = mstream_launch<QT, TT, 1>(m, k, n, tune);
        return launch_gemv_mfma_r<QT, TT, 1>(p1, dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
    } else {
        const MStreamLaunch p2 = mstream_launch<QT, TT, 2>(m, k, n, tune);
        if constexpr (QT != QT_F32) {
            const MStreamLaunch p1 = mstream_launch<QT, TT, 1>(m, k, n, tune);
            if ((m + 7) / 8 < 4 * (int64_t)tune.num_cu && 4 * p1.iters < 3 * 2 * p2.iters)
                return launch_gemv_mfma_r<QT, TT, 1>(p1, dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
        }
        return launch_gemv_mfma_r<QT, TT, 2>(p2, dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
    }
}

// Token groups of the matrix-core stream: 8 rows where they fit (half the
// passes over the weights) and n > 4, else 4 where they fit, else 0.
// GEMV_AUTO takes it from n = gemv_mfma_min; below n = 8 only where it
// measured faster than the FMA stream: at least four row groups of 8 rows
// per CU (14336x4096, n = 4: 19.2 against 20.0 us) or rows of at least 4
// unit iterations, which several waves then share (1024x4608 Q4_0: 7.8
// against 9.4 us); on short rows with few row groups the FMA stream stays
// (4608x1024 Q4_K, n = 4: 5.8 against 6.2 us).
int gemv_matrix_tokens(int64_t m, int64_t k, int64_t n, int qt, int kind, const GemvTuning& tune) {
    const int64_t n_rg = (m + 7) / 8;
    const int64_t upl = ((k + unit_elems_of(qt) - 1) / unit_elems_of(qt) + 15) / 16;
    const bool wide = n >= 8 || n_rg >= 4 * (int64_t)tune.num_cu || upl >= 4;
    const bool use = kind == GEMV_MATRIX ||
                     (kind == GEMV_AUTO && tune.gemv_mfma_min > 0 && n >= tune.gemv_mfma_min && wide);
    if (!use) return 0;
    const int lm = mtraits_lm(qt);
    const bool sums = qt_runs(qt);
    // the staged rows and the partial sums of launch_gemv_mfma (R = 2)
    auto lds = [&](int tt) { return ((int64_t)qlds_floats(4 * tt, (int)k, lm, sums) + 2 * 8 * 16 * 2 * tt) * 4; };
    if (n > 4 && tune.gemv_mfma_tt >= 2 && lds(2) <= tune.lds_per_wg) return 8;
    if (lds(1) <= tune.lds_per_wg) return 4;
    return 0;
}

template <int QT>
static void launch_gemv_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k,
                           int64_t n, int64_t rb, int64_t ldx, int64_t ldd, int kind, const GemvTuning& tune,
                           hipStream_t st) {
    const int tok = gemv_matrix_tokens(m, k, n, QT, kind, tune);
    if (tok == 8 && launch_gemv_mfma<QT, 2>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st)) return;
    if (tok == 4 && launch_gemv_mfma<QT, 1>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st)) return;
    const bool fits8 = (int64_t)xlds_floats(8, (int)k, GUnit<QT>::RUNS > 0) * 4 <= tune.lds_per_wg;
    const bool fits4 = (int64_t)xlds_floats(4, (int)k, GUnit<QT>::RUNS > 0) * 4 <= tune.lds_per_wg;
    if (n == 1) launch_gemv_nt<QT, 1>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
    else if (n == 2) launch_gemv_nt<QT, 2>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
    else if (n <= 4 || (!fits8 && fits4))  // groups of 4 staged rows beat 8 rows read from L2
        launch_gemv_nt<QT, 4>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
    else launch_gemv_nt<QT, 8>(dst, w, x, m, k, n, rb, ldx, ldd, tune, st);
}

void launch_gemv(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                 int qt, int64_t rb, int64_t ldx, int64_t ldd, int kind, const GemvTuning& tune, hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    QMM_QT_SWITCH(qt, (launch_gemv_qt<Q>(dst, wb, x, m, k, n, rb, ldx, ldd, kind, tune, st)))
}

template <int QT>
static void launch_lo_qt(uint32_t* sink, const uint8_t* w, int64_t m, int64_t k, int64_t rb,
                         const GemvTuning& tune, hipStream_t st) {
    with_rd<1>(tune, [&](auto Rc, auto Dc) {
        constexpr int R = decltype(Rc)::value, D = decltype(Dc)::value;
        const int l = lpr_for(QT, k, LPR_CAP_SINGLE);
        const int64_t n_rg = (m + rg_rows(l, R) - 1) / rg_rows(l, R);
        loadonly_kernel<QT, R, D><<<dim3(stream_grid(n_rg, 1, tune)), 256, 0, st>>>(
            sink, w, (int)m, (int)k, (int)rb, l, (int)n_rg);
    });
}

void launch_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k, int qt, int64_t rb,
                     const GemvTuning& tune, hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    QMM_QT_SWITCH(qt, (launch_lo_qt<Q>(sink, wb, m, k, rb, tune, st)))
}

}  // namespace qmm
