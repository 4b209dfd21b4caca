// The matrix-core variant of the streaming core, for streams that apply each
// weight to several activation rows (the GEMV at n > 2, the MoE experts with
// several tokens).  The weights stream and decode exactly as in stream.hpp
// (the same units, loads and decoders); the products with the activations
// run on v_mfma_f32_4x4x1f32 instead of f32 FMAs, in f32 throughout: every
// product w*x is formed and summed in f32, as the FMA stream does.
//
// v_mfma_f32_4x4x1f32 computes 16 independent 4x4 outer products: lane
// 4b + i supplies A[i] of block b, lane 4b + j supplies B[j], and lane 4b + j
// holds D[i][j] of block b in its accumulator register i.  Here A is four
// activation rows (tokens) and B four weight rows at one k: the lanes of a
// quad (the four lanes 4b..4b+3) decode the same unit position of four rows,
// each lane its own row, and supply the same k of four tokens, each lane its
// own token.  A lane's register i then accumulates its own row against token
// i, so per-row scale factors are the lane's own.  The 16 quads take 16
// units of their rows at a time (a row has 16 lanes, like a lane group of 16
// in the FMA stream), and the quads' sums are added by a butterfly at the
// end of each row group.
//
// Rounding chains.  Each unit's products accumulate in fresh registers (a
// run of one scale factor, at most 64 terms, or the whole unit) before
// joining the lane's running sum, so every f32 chain has at most
// 64 + k/(16*UE) + 4 terms, the bound the FMA stream keeps.
#pragma once
#include "stream.hpp"

namespace qmm {

// ------------------------------------------------------------------ activations
// Token-major rows with 4 floats of padding after every 32 and a row stride
// of lm (mod 32) floats: the 8 lanes of an LDS phase (two quads: four tokens
// at two neighbouring units) then read distinct 16-byte bank groups, with
// lm = 8 for formats whose neighbouring units are 32 weights apart and
// lm = 4 for those 16 apart.  A block of QZERO zero floats follows the rows:
// quads whose unit lies past the row's end read it.
__host__ __device__ constexpr int qpad(int e) { return e + ((e >> 5) << 2); }
__host__ __device__ constexpr int qld(int k, int lm) {
    const int b = qpad((k + 31) & ~31);
    return b + ((lm - b % 32) % 32 + 32) % 32;
}
constexpr int QZERO = 128;
// LDS floats of nt staged rows, the zero block and, for the offset formats
// (sums), the rows' run sums (k/16 per row, four rows interleaved).
__host__ __device__ constexpr int qlds_floats(int nt, int k, int lm, bool sums) {
    return nt * qld(k, lm) + QZERO + (sums ? nt * (k >> 4) : 0);
}

// Offset of k = e + rel from k = e in the padded layout.  Every unit starts
// at e with e % 32 + rel % 32 + 4 <= 32 for the offsets it reads, so the
// padding crossed depends on rel alone (qrel_ok checks it for each format at
// compile time over the residues e % 32 its units start at).
__host__ __device__ constexpr int qrel(int rel) { return rel + 4 * (rel >> 5); }

// Per format: LM (the row stride residue above), CH (chains per sub-unit: 2
// when its two halves carry different scale factors), EM1 (the second residue
// e % 32 that units start at, besides 0), flush(s) (whether a run of one
// scale factor, or the unit, ends with sub-unit s).
// Q4_0 and Q4_K (w = A_r*q - B_r per run of 16, 4-bit q) stream q itself,
// exact, and finish each run with A_r*sum(q*x) - B_r*sum(x) (RUN); q
// converts through v_cvt_pk_f32_fp8 as the E4M3 codes 0..15, whose values
// are exactly q * 2^-9, so QS = 2^9 goes into A_r.  Q6_K keeps w = q - 32
// with its scale per run: its 6-bit q converts through ubyte_f32, whose
// inline asm hides the register write from the compiler's hazard checks,
// and a matrix-core operand must not be such a write (the subtract between
// them is an ordinary VALU instruction).
template <int QT> struct MTraits;
template <> struct MTraits<QT_F32> { static constexpr bool RUN = false; static constexpr float QS = 1.0f; static constexpr int LM = 4, CH = 1, EM1 = 16; static constexpr bool flush(int s) { return s == 1; } };
template <> struct MTraits<QT_Q4_0> { static constexpr bool RUN = true; static constexpr float QS = 512.0f; static constexpr int LM = 8, CH = 1, EM1 = 0; static constexpr bool flush(int s) { return s == 3; } };
template <> struct MTraits<QT_Q8_0> { static constexpr bool RUN = false; static constexpr float QS = 1.0f; static constexpr int LM = 8, CH = 1, EM1 = 0; static constexpr bool flush(int s) { return s == 3; } };
template <> struct MTraits<QT_Q4_K> { static constexpr bool RUN = true; static constexpr float QS = 512.0f; static constexpr int LM = 4, CH = 1, EM1 = 16; static constexpr bool flush(int s) { return s == 3; } };
// Q6_K: a scale factor per quarter (sub-units 2g, 2g + 1)
template <> struct MTraits<QT_Q6_K> { static constexpr bool RUN = false; static constexpr float QS = 1.0f; static constexpr int LM = 4, CH = 1, EM1 = 16; static constexpr bool flush(int s) { return (s & 1) == 1; } };
// NVFP4: the two halves of a sub-unit belong to the unit's two scale groups
template <> struct MTraits<QT_NVFP4> { static constexpr bool RUN = false; static constexpr float QS = 1.0f; static constexpr int LM = 8, CH = 2, EM1 = 0; static constexpr bool flush(int s) { return s == 3; } };
template <> struct MTraits<QT_NVFP4_V2> { static constexpr bool RUN = false; static constexpr float QS = 1.0f; static constexpr int LM = 8, CH = 2, EM1 = 0; static constexpr bool flush(int s) { return s == 3; } };

// The four activations at e + rel .. e + rel + 3 are contiguous at
// qpad(e) + qrel(rel) for every sub-unit offset and unit start residue.
template <int QT>
constexpr bool qrel_ok() {
    using UT = GUnit<QT>;
    for (int i = 0; i < 2; ++i) {
        const int e = i == 0 ? 0 : MTraits<QT>::EM1;
        for (int s = 0; s < UT::S; ++s)
            for (int h = 0; h < 2; ++h) {
                const int rel = h == 0 ? UT::rel0(s) : UT::rel1(s);
                for (int q = 0; q < 4; ++q)
                    if (qpad(e + rel + q) - qpad(e) != qrel(rel) + q) return false;
            }
    }
    return true;
}
static_assert(qrel_ok<QT_F32>() && qrel_ok<QT_Q4_0>() && qrel_ok<QT_Q8_0>() && qrel_ok<QT_Q4_K>() &&
                  qrel_ok<QT_Q6_K>() && qrel_ok<QT_NVFP4>() && qrel_ok<QT_NVFP4_V2>(),
              "a unit's activations cross the quad layout's padding");

// The formats whose matrix-core stream needs the run sums (MTraits::RUN).
inline bool qt_runs(int qt) { return qt == QT_Q4_0 || qt == QT_Q4_K; }
static_assert(MTraits<QT_Q4_0>::RUN && MTraits<QT_Q4_K>::RUN && !MTraits<QT_Q6_K>::RUN && !MTraits<QT_F32>::RUN &&
                  !MTraits<QT_Q8_0>::RUN && !MTraits<QT_NVFP4>::RUN && !MTraits<QT_NVFP4_V2>::RUN,
              "qt_runs lists the formats with MTraits::RUN");
static_assert(GUnit<QT_Q4_0>::RUNS > 0 && GUnit<QT_Q4_K>::RUNS > 0, "RUN formats have runs");

inline int mtraits_lm(int qt) {
    switch (qt) {
        case QT_F32: return MTraits<QT_F32>::LM;
        case QT_Q4_0: return MTraits<QT_Q4_0>::LM;
        case QT_Q8_0: return MTraits<QT_Q8_0>::LM;
        case QT_Q4_K: return MTraits<QT_Q4_K>::LM;
        case QT_Q6_K: return MTraits<QT_Q6_K>::LM;
        case QT_NVFP4: return MTraits<QT_NVFP4>::LM;
        case QT_NVFP4_V2: return MTraits<QT_NVFP4_V2>::LM;
    }
    return 8;
}

// Activation rows of TT tiles of four tokens in the quad layout: row[t] is
// this lane's token row in tile t (token lane & 3 of the tile), zero the
// zero block.
template <int TT>
struct XQuad {
    const float* row[TT];
    const float* zero;
    const float* sums[TT];  // offset formats: run sums of tile t, [k/16][4 tokens]
};

// Stage rows xoff[j] (j < nreal <= NTOK) of x into LDS in the quad layout
// (two-phase, as XStage), clear the zero block and, with SUMS, write the run
// sums of the staged rows: token j's sum over k = 16r .. 16r + 15 at
// sums[((j >> 2) * (k >> 4) + r) * 4 + (j & 3)], added in a fixed order.
// Rows j >= nreal are not staged: the lanes of absent tokens read row 0.
template <int NTOK, bool SUMS, int TPB = 256>
struct QStage {
    static constexpr int U = NTOK >= 8 ? 1 : 8 / NTOK;  // float4 columns per thread per batch
    float* sx;
    rsrc_t xr;
    uint32_t xoff[NTOK];
    int k, ld, nreal;
    f32x4 v[NTOK][U];

    __device__ __forceinline__ void load(int c0) {
        const int per = k >> 2;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + TPB * u;
#pragma unroll
            for (int j = 0; j < NTOK; ++j)
                if (j < nreal)
                    v[j][u] = __builtin_bit_cast(f32x4, ld128(xr, c < per ? xoff[j] + 16u * (uint32_t)c : OOB_OFF));
        }
    }
    __device__ __forceinline__ void store(int c0) {
        const int per = k >> 2;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + TPB * u;
            if (c < per)
#pragma unroll
                for (int j = 0; j < NTOK; ++j)
                    if (j < nreal) *(f32x4*)(sx + j * ld + qpad(4 * c)) = v[j][u];
        }
    }
    __device__ __forceinline__ void issue() { load((int)threadIdx.x); }
    __device__ __forceinline__ void finish() {
        store((int)threadIdx.x);
        for (int c0 = (int)threadIdx.x + TPB * U; c0 < (k >> 2); c0 += TPB * U) {
            load(c0);
            store(c0);
        }
        for (int i = (int)threadIdx.x; i < QZERO; i += TPB) sx[NTOK * ld + i] = 0.0f;
        __syncthreads();
        if constexpr (SUMS) {
            const int nrun = k >> 4;
            float* sums = sx + NTOK * ld + QZERO;
            for (int t = threadIdx.x; t < nreal * nrun; t += TPB) {
                const int j = t / nrun, r = t - j * nrun;
                const float* p = sx + j * ld + qpad(16 * r);  // 16 contiguous floats
                const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
                const f32x4 c = *(const f32x4*)(p + 8), d = *(const f32x4*)(p + 12);
                const float sa = (a.x + a.y) + (a.z + a.w), sb = (b.x + b.y) + (b.z + b.w);
                const float sc = (c.x + c.y) + (c.z + c.w), sd = (d.x + d.y) + (d.z + d.w);
                sums[((j >> 2) * nrun + r) * 4 + (j & 3)] = (sa + sb) + (sc + sd);
            }
            __syncthreads();
        }
    }
};

template <int NTOK, bool SUMS, int TPB = 256>
__device__ __forceinline__ QStage<NTOK, SUMS, TPB> make_qstage(float* sx, rsrc_t xr, const uint32_t (&xoff)[NTOK],
                                                               int k, int ld, int nreal) {
    QStage<NTOK, SUMS, TPB> st;
    st.sx = sx;
    st.xr = xr;
#pragma unroll
    for (int j = 0; j < NTOK; ++j) st.xoff[j] = xoff[j];
    st.k = k;
    st.ld = ld;
    st.nreal = nreal;
    return st;
}

// The quad-layout view of NTOK = 4 TT staged rows at sx (row stride ld) for
// this lane: tile t's token 4t + (lane & 3), row 0 for tokens >= nreal.
template <int TT>
__device__ __forceinline__ XQuad<TT> make_xquad(float* sx, int ld, int k, int nreal) {
    XQuad<TT> xq;
    const int i = (int)(threadIdx.x & 3);
    xq.zero = sx + 4 * TT * ld;
    const float* sums = xq.zero + QZERO;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int j = 4 * t + i;
        xq.row[t] = sx + (j < nreal ? j : 0) * ld;
        xq.sums[t] = sums + t * (k >> 4) * 4;
    }
    return xq;
}

// ------------------------------------------------------------------ core
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// Sub-unit S_ of every row rr and tile t: 8 products per lane into chain(s)
// P; at the format's flush points the chains join acc (times the run's scale
// factor for the SCALED formats).
template <int QT, int TT, int R, int S_>
__device__ __forceinline__ void msub(const GUnit<QT> (&un)[R], const float* const (&xp)[TT], int k, int e,
                                     f32x4 (&P)[R][TT][MTraits<QT>::CH], f32x4 (&acc)[R][TT]) {
    using UT = GUnit<QT>;
    using MT = MTraits<QT>;
    float w[R][8], f0[R], f1[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) un[rr].sub(S_, w[rr], f0[rr], f1[rr]);
    f32x4 xa[TT], xb[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        xa[t] = *(const f32x4*)(xp[t] + qrel(UT::rel0(S_)));
        xb[t] = *(const f32x4*)(xp[t] + qrel(UT::rel1(S_)));
        if constexpr (QT == QT_F32) {  // runs past k belong to the next row
            if (e + UT::rel0(S_) >= k) xa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (e + UT::rel1(S_) >= k) xb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // independent chains interleaved (rows, tiles and, with two chains, the
    // halves), so that no product waits for the one before it
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                P[rr][t][0] = mfma4(xa[t][q], w[rr][q], P[rr][t][0]);
                if constexpr (MT::CH == 2) P[rr][t][1] = mfma4(xb[t][q], w[rr][4 + q], P[rr][t][1]);
            }
    if constexpr (MT::CH == 1)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) P[rr][t][0] = mfma4(xb[t][q], w[rr][4 + q], P[rr][t][0]);
    if constexpr (MT::flush(S_)) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int c = 0; c < MT::CH; ++c) {
                    const float f = c == 0 ? f0[rr] : f1[rr];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (UT::SCALED) acc[rr][t][i] = __builtin_fmaf(f, P[rr][t][c][i], acc[rr][t][i]);
                        else acc[rr][t][i] += P[rr][t][c][i];
                    }
                    P[rr][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
    }
}

template <int QT, int TT, int R, int S_ = 0>
__device__ __forceinline__ void msub_all(const GUnit<QT> (&un)[R], const float* const (&xp)[TT], int k, int e,
                                         f32x4 (&P)[R][TT][MTraits<QT>::CH], f32x4 (&acc)[R][TT]) {
    if constexpr (S_ < GUnit<QT>::S) {
        msub<QT, TT, R, S_>(un, xp, k, e, P, acc);
        msub_all<QT, TT, R, S_ + 1>(un, xp, k, e, P, acc);
    }
}

// Four nibbles (bytes 0..3 of lo) as floats q * 2^-9: v_cvt_pk_f32_fp8
// reads each byte as an E4M3 code, and the codes 0..15 are the subnormals
// m * 2^-9 (m < 8) and the normals (1 + m/8) * 2^-6 = (8 + m) * 2^-9.
__device__ __forceinline__ void nib4_f32(uint32_t v, float* q) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
    q[0] = a.x;
    q[1] = a.y;
    q[2] = b.x;
    q[3] = b.y;
}

// q of sub-unit s of an offset format as exact floats times 1/QS, in the
// order of GUnit::qsub (q[0..3] at rel0(s), q[4..7] at rel1(s)).
template <int QT>
__device__ __forceinline__ void mq(const GUnit<QT>& u, int s, float (&q)[8]) {
    static_assert(QT == QT_Q4_0 || QT == QT_Q4_K, "4-bit q only");
    uint32_t v;
    if constexpr (QT == QT_Q4_0) v = shr64(u.r[s], u.r[s + 1], u.sh + 2u);
    else v = s == 0 ? u.qs.x : (s == 1 ? u.qs.y : (s == 2 ? u.qs.z : u.qs.w));
    nib4_f32(v & 0x0F0F0F0Fu, q);
    nib4_f32((v >> 4) & 0x0F0F0F0Fu, q + 4);
}

// Sub-unit S_ of an offset format: the q*x products of each run accumulate
// in P (slot r & 1); after the run's last sub-unit, acc += A_r*QS*P -
// B_r*sum(x of the run), the sums of the lane's tile tokens read as one
// float4 (sp[t]: the run sums at the unit's first k).
template <int QT, int TT, int R, int S_>
__device__ __forceinline__ void msub_runs(const GUnit<QT> (&un)[R], const float* const (&xp)[TT],
                                          const float* const (&sp)[TT], f32x4 (&P)[R][TT][2],
                                          f32x4 (&acc)[R][TT]) {
    using UT = GUnit<QT>;
    using MT = MTraits<QT>;
    constexpr int r0 = UT::run0(S_), r1 = UT::run1(S_);
    float q[R][8];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) mq<QT>(un[rr], S_, q[rr]);
    f32x4 xa[TT], xb[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        xa[t] = *(const f32x4*)(xp[t] + qrel(UT::rel0(S_)));
        xb[t] = *(const f32x4*)(xp[t] + qrel(UT::rel1(S_)));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                P[rr][t][r0 & 1] = mfma4(xa[t][c], q[rr][c], P[rr][t][r0 & 1]);
                if constexpr (r1 != r0) P[rr][t][r1 & 1] = mfma4(xb[t][c], q[rr][4 + c], P[rr][t][r1 & 1]);
            }
    if constexpr (r1 == r0)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int t = 0; t < TT; ++t)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) P[rr][t][r0 & 1] = mfma4(xb[t][c], q[rr][4 + c], P[rr][t][r0 & 1]);
    auto flush = [&](int r) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const f32x4 sx = *(const f32x4*)(sp[t] + (UT::runrel(r) >> 4) * 4);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const float a = un[rr].runA(r) * MT::QS, b = un[rr].runB(r);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = __builtin_fmaf(a, P[rr][t][r & 1][i], acc[rr][t][i]);
                    acc[rr][t][i] = __builtin_fmaf(-b, sx[i], v);
                }
                P[rr][t][r & 1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    if constexpr (S_ == UT::lastsub(r0)) flush(r0);
    if constexpr (r1 != r0 && S_ == UT::lastsub(r1)) flush(r1);
}

template <int QT, int TT, int R, int S_ = 0>
__device__ __forceinline__ void msub_all_runs(const GUnit<QT> (&un)[R], const float* const (&xp)[TT],
                                              const float* const (&sp)[TT], f32x4 (&P)[R][TT][2],
                                              f32x4 (&acc)[R][TT]) {
    if constexpr (S_ < GUnit<QT>::S) {
        msub_runs<QT, TT, R, S_>(un, xp, sp, P, acc);
        msub_all_runs<QT, TT, R, S_ + 1>(un, xp, sp, P, acc);
    }
}

// One item: the unit at k = e of the lane's R rows against the lane's token
// in each tile; valid = false (the quad's unit lies past the row's end; its
// weights were loaded as zeros) reads the zero block instead.
template <int QT, int TT, int R>
__device__ __forceinline__ void mcompute_item(GUnit<QT> (&un)[R], const typename GUnit<QT>::Lane& ln, int e,
                                              bool valid, int k, const XQuad<TT>& xq, f32x4 (&acc)[R][TT]) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) un[rr].prep(ln);
    const float* xp[TT];
    const int pe = qpad(e);
#pragma unroll
    for (int t = 0; t < TT; ++t) xp[t] = valid ? xq.row[t] + pe : xq.zero;
    if constexpr (MTraits<QT>::RUN) {
        const float* sp[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) sp[t] = valid ? xq.sums[t] + (e >> 4) * 4 : xq.zero;
        f32x4 P[R][TT][2];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int t = 0; t < TT; ++t) P[rr][t][0] = P[rr][t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        msub_all_runs<QT, TT, R>(un, xp, sp, P, acc);
        return;
    }
    f32x4 P[R][TT][MTraits<QT>::CH];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < MTraits<QT>::CH; ++c) P[rr][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    msub_all<QT, TT, R>(un, xp, k, e, P, acc);
}

// Row groups of 4R rows (lane l takes rows (l & 3) * R + rr of the group, and
// units (l >> 2) + 16 uu of them).  KW waves share a row group: wave kq of
// the KW takes the unit iterations uu = kq, kq + KW, ... (V = ceil(upl/KW)
// items per row group, those past upl dead), and at the row group's end the
// KW partial sums meet in LDS (red: 2 * waves per work group * 16 R TT
// floats, alternate halves per row group) and the kq = 0 wave adds them in
// the order kq = 0, 1, ... and stores.  A work group's waves all run the
// same n_iter row-group iterations (row groups past n_rg are dead: no loads,
// no stores), so its barriers match.  A ring of D items of loads is in
// flight; pre.issue()/pre.finish() go around the first loads.  store(row, j,
// value) is called by lanes 0..3 for token j = 4t + i of every row of a live
// row group (rows >= m too).  A quad whose unit lies past the row's end loads
// nothing (zeros) and reads the zero block, so it adds exact zeros.
// ARM: the measurement twins as in gemv_stream (load-only: the raw words
// XORed into acc[rr][0][0]; math-only: the first item's unit for every item).
template <int QT, int TT, int R, int D, int KW, typename Store, typename Pre = NoPre, int ARM = STREAM_SERVED>
__device__ __forceinline__ void mfma_stream(const StreamGeom& g, int first_rg, int rg_stride, int n_rg, int n_iter,
                                            int kq, float* red, const XQuad<TT>& xq, Store store, Pre pre = {}) {
    using UT = GUnit<QT>;
    constexpr int LPR = 16;
    const int lane = threadIdx.x & 63;
    const int gl = lane >> 2, slot = lane & 3;
    const int RG = 4 * R;
    const int U = (g.k + UT::UE - 1) / UT::UE;
    const int upl = (U + LPR - 1) / LPR;
    const int V = (upl + KW - 1) / KW;
    const int n_items = n_iter * V;
    const typename UT::Lane ln = UT::lane(gl);
    const uint32_t lane_row_off = (uint32_t)(slot * R) * (uint32_t)g.rb;
    const int e_step = LPR * UT::UE;
    const StreamGeom g16{g.w, g.m, g.rb, g.k, 4};  // the unit step of 16-lane groups
    auto rg_live = [&](int q) { return first_rg + q * rg_stride < n_rg; };

    f32x4 acc[R][TT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[rr][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto finish = [&](int q) {
#pragma unroll
        for (int off = 4; off < 64; off <<= 1)
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rr][t][i] += __shfl_xor(acc[rr][t][i], off, 64);
        const int64_t r0 = (int64_t)(first_rg + q * rg_stride) * RG + slot * R;
        if constexpr (KW == 1) {
            if (rg_live(q) && lane < 4)
#pragma unroll
                for (int rr = 0; rr < R; ++rr)
#pragma unroll
                    for (int t = 0; t < TT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) store(r0 + rr, 4 * t + i, acc[rr][t][i]);
        } else {
            constexpr int PW = 16 * R * TT;  // floats per wave: lanes 0..3, R*TT*4 each
            const int wave = wave_id();
            float* half = red + (q & 1) * (int)(blockDim.x >> 6) * PW;
            if (lane < 4)
#pragma unroll
                for (int rr = 0; rr < R; ++rr)
#pragma unroll
                    for (int t = 0; t < TT; ++t)
                        *(f32x4*)(half + wave * PW + lane * (4 * R * TT) + (rr * TT + t) * 4) = acc[rr][t];
            __syncthreads();
            if (kq == 0 && rg_live(q) && lane < 4) {
#pragma unroll
                for (int rr = 0; rr < R; ++rr)
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        f32x4 v = *(const f32x4*)(half + wave * PW + lane * (4 * R * TT) + (rr * TT + t) * 4);
#pragma unroll
                        for (int w = 1; w < KW; ++w)
                            v += *(const f32x4*)(half + (wave + w) * PW + lane * (4 * R * TT) + (rr * TT + t) * 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) store(r0 + rr, 4 * t + i, v[i]);
                    }
            }
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[rr][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // loads of item (row-group iteration q, iteration v of this wave): unit
    // uu = kq + KW v; dead items (row group past n_rg, or uu >= upl) load
    // nothing, and a quad whose unit is past the row's end loads zeros
    auto issue = [&](UT (&slot_un)[R], int q, int v, bool exists) {
        const int uu = kq + KW * v;
        issue_item<QT, R>(slot_un, g16, RG, lane_row_off, ln, first_rg + q * rg_stride, uu, ln.e + uu * e_step,
                          exists && rg_live(q) && uu < upl, gl + LPR * uu < U);
    };

    UT ring[D][R];
    pre.issue();
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int q = d / V, v = d - q * V;
        issue(ring[d], q, v, d < n_items);
    }
    pre.finish();
    ItemPos cur{0, 0}, nxt{D / V, D - (D / V) * V};
    for (int base = 0; base < n_items; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = base + d;
            const bool exists = it < n_items;  // wave-uniform, the same for every wave of the work group
            const int q = cur.q, v = cur.uu, uu = kq + KW * v;
            if (exists && rg_live(q) && uu < upl) {
                if constexpr (ARM == STREAM_LOADONLY) {
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
                        acc[rr][0][0] = __builtin_bit_cast(
                            float, __builtin_bit_cast(uint32_t, acc[rr][0][0]) ^ raw_xor(ring[d][rr]));
                } else {
                    mcompute_item<QT, TT, R>(ring[d], ln, ln.e + uu * e_step, gl + LPR * uu < U, g.k, xq, acc);
                }
            }
            if constexpr (ARM == STREAM_MATHONLY) issue(ring[d], 0, 0, it + D < n_items);
            else issue(ring[d], nxt.q, nxt.uu, it + D < n_items);
            if (exists && v == V - 1) finish(q);
            cur.next(V);
            nxt.next(V);
        }
    }
}

}  // namespace qmm
