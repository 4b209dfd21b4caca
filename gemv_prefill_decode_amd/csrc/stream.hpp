// The streaming core shared by the decode GEMV (gemv.hip) and the MoE
// projections (moe.hip): f32 GEMV for small n, the MoE gate/up projections,
// and the load-only twin.  No matrix cores: the weights stream from HBM once, each
// lane decodes its blocks to f32 in registers and accumulates with f32 FMA;
// lanes that share a row reduce with cross-lane shuffles.
//
// Work split.  A row of k weights is cut into "units" (16..64 weights each,
// per format).  The LPR lanes of a lane group take units gl + LPR*uu
// (uu = 0, 1, ...) of the same R rows, so one wave load instruction reads LPR
// consecutive units of a row, and the activations a lane reads for a unit are
// reused for its R rows.  Because LPR is a power of two no smaller than the
// number of units per block-format period, the position of a lane's unit
// inside its block is the same for every uu: byte and k offsets are a
// per-lane constant plus uu times a uniform step, and the decode parameters
// that depend on that position are per-lane constants.
//
// Rounding chains.  Each unit's products are summed in a fresh partial (at
// most 64 terms) before joining the lane's running sum, and the LPR lane sums
// are combined by a butterfly: every f32 chain has at most
// 64 + k/(UE*LPR) + log2(LPR) terms.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

// ------------------------------------------------------------------ units
// Per format:
//   UE, S        weights per unit, sub-units of 8 weights
//   MIN_LPR      smallest lane-group size for which the unit position within
//                its block is the same for all uu
//   Lane         per-lane constants: boff (byte offset of unit gl in its row),
//                e (k index of the unit's first run)
//   ustep(lpr)   byte offset added per uu
//   load(), prep(), sub(s, w, f0, f1)
//                sub-unit s: 8 weights w[0..7]; w[0..3] pair with the 4
//                activations at k = e + rel0(s), w[4..7] with k = e + rel1(s).
//                SCALED units return unscaled weights and the factors f0, f1
//                of the two runs (the factor is common to each run).
//   prel0(s), prel1(s)
//                rel0/rel1 in the padded LDS activation layout.
//   RUNS > 0     offset formats: in each of the unit's RUNS runs of 16
//                weights, w = A_r*q - B_r with q a small non-negative
//                integer.  qsub(s, q) gives the q of sub-unit s as exact
//                floats, run0(s)/run1(s) the runs its halves belong to,
//                lastsub(r) the last sub-unit of run r, runrel(r) its first
//                k relative to e, runA/runB its factors.  With activations
//                staged in LDS the sums use sum(w*x) = A_r*sum(q*x) -
//                B_r*sum(x), the run sums of x being computed once per work
//                group: one FMA per weight and token instead of two.
//   PACKED       (offset formats) qpack(s, p) gives sub-unit s's q as four
//                dwords of two subnormal f16 halves each, cut out of the
//                packed bytes by masks: p[0] = (q0, q2), p[1] = (q1, q3),
//                p[2] = (q4, q6), p[3] = (q5, q7), each half worth
//                q / pscale(run) (a power of two).  Every product q*x then is
//                one v_fma_mix_f32, and the run's sum comes out scaled by
//                exactly 1/pscale(run) (no f32 underflow for |x| above
//                about 2^-100), which the run's end multiplies back into A_r.

template <int QT> struct GUnit;

struct LaneBase {
    uint32_t boff;
    int e;
};

template <> struct GUnit<QT_F32> {  // 16 weights, 64 bytes
    static constexpr int UE = 16, S = 2, MIN_LPR = 1;
    static constexpr bool SCALED = false;
    static constexpr int RUNS = 0;
    struct Lane : LaneBase {};
    __device__ static Lane lane(int gl) { return Lane{{(uint32_t)gl * 64u, gl * 16}}; }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)lpr * 64u; }
    static constexpr int rel0(int s) { return 8 * s; }
    static constexpr int rel1(int s) { return 8 * s + 4; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    uint32_t r[16];
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int e, int k, const Lane&) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // k % 4 == 0: a run of 4 is wholly in or out
            const u32x4 v = ld128(wr, e + 4 * i < k ? off + 16u * i : OOB_OFF);
            r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
        }
    }
    __device__ __forceinline__ void prep(const Lane&) {}
    __device__ __forceinline__ void sub(int s, float (&w)[8], float&, float&) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = __builtin_bit_cast(float, r[8 * s + i]);
    }
};

template <> struct GUnit<QT_Q4_0> {  // one 18-byte block of 32 weights
    static constexpr int UE = 32, S = 4, MIN_LPR = 1;
    static constexpr bool SCALED = false;
    static constexpr int RUNS = 2;  // w = d*q - 8d; runs: low nibbles (k 0..15), high (16..31)
    static constexpr int run0(int) { return 0; }
    static constexpr int run1(int) { return 1; }
    static constexpr int lastsub(int) { return 3; }
    static constexpr int runrel(int r) { return 16 * r; }
    struct Lane : LaneBase {};
    __device__ static Lane lane(int gl) { return Lane{{(uint32_t)gl * 18u, gl * 32}}; }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)lpr * 18u; }
    static constexpr int rel0(int s) { return 4 * s; }
    static constexpr int rel1(int s) { return 16 + 4 * s; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    uint32_t r[5], sh;
    float d, d8;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int, int, const Lane&) {
        sh = off & 3u;
        ld_span<5>(wr, off, r);
    }
    __device__ __forceinline__ void prep(const Lane&) {
        d = h2f(r[0] >> (8u * sh));
        d8 = -8.0f * d;
    }
    __device__ __forceinline__ float runA(int) const { return d; }
    __device__ __forceinline__ float runB(int) const { return -d8; }
    // low nibbles in place (q * 2^-24), high nibbles in place (q * 2^-20)
    static constexpr bool PACKED = true;
    static constexpr float pscale(int r) { return r == 0 ? 16777216.0f : 1048576.0f; }
    __device__ __forceinline__ void qpack(int s, uint32_t (&p)[4]) const {
        const uint32_t v = shr64(r[s], r[s + 1], sh + 2u), v8 = v >> 8;
        p[0] = v & 0x000F000Fu;
        p[1] = v8 & 0x000F000Fu;
        p[2] = v & 0x00F000F0u;
        p[3] = v8 & 0x00F000F0u;
    }
    __device__ __forceinline__ void qsub(int s, float (&q)[8]) const {
        const uint32_t v = shr64(r[s], r[s + 1], sh + 2u);
        const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            q[b] = ubyte_f32(lo, b);
            q[4 + b] = ubyte_f32(hi, b);
        }
    }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float&, float&) const {
        const uint32_t q = shr64(r[s], r[s + 1], sh + 2u);  // qs[4s..4s+3]
        const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = __builtin_fmaf(d, ubyte_f32(lo, b), d8);  // d*(q-8), exact
            w[4 + b] = __builtin_fmaf(d, ubyte_f32(hi, b), d8);
        }
    }
};

template <> struct GUnit<QT_Q8_0> {  // one 34-byte block of 32 weights
    static constexpr int UE = 32, S = 4, MIN_LPR = 1;
    static constexpr bool SCALED = true;  // d is common to the whole block
    static constexpr int RUNS = 0;
    struct Lane : LaneBase {};
    __device__ static Lane lane(int gl) { return Lane{{(uint32_t)gl * 34u, gl * 32}}; }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)lpr * 34u; }
    static constexpr int rel0(int s) { return 8 * s; }
    static constexpr int rel1(int s) { return 8 * s + 4; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    uint32_t r[9], sh;
    float d;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int, int, const Lane&) {
        sh = off & 3u;
        ld_span<9>(wr, off, r);
    }
    __device__ __forceinline__ void prep(const Lane&) { d = h2f(r[0] >> (8u * sh)); }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float& f0, float& f1) const {
        // int8 q as (q + 128) - 128: both exact in f32
        const uint32_t qa = shr64(r[2 * s], r[2 * s + 1], sh + 2u) ^ 0x80808080u;
        const uint32_t qb = shr64(r[2 * s + 1], r[2 * s + 2], sh + 2u) ^ 0x80808080u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = ubyte_f32(qa, b) - 128.0f;
            w[4 + b] = ubyte_f32(qb, b) - 128.0f;
        }
        f0 = d;
        f1 = d;
    }
};

// Q4_K: 16 bytes of nibbles (32 weights: 16 of sub-block 2c, 16 of 2c+1) of
// a 144-byte superblock, plus the superblock's 16-byte header.  The lane's
// nibble-chunk index c8 = gl & 7 is the same for every uu (LPR >= 8).
template <> struct GUnit<QT_Q4_K> {
    static constexpr int UE = 32, S = 4, MIN_LPR = 8;
    static constexpr bool SCALED = false;
    static constexpr int RUNS = 2;  // w = D*q - M; runs: sub-block 2c (k e..e+15), 2c+1 (e+32..)
    static constexpr int run0(int) { return 0; }
    static constexpr int run1(int) { return 1; }
    static constexpr int lastsub(int) { return 3; }
    static constexpr int runrel(int r) { return 32 * r; }
    struct Lane : LaneBase {
        uint32_t qoff;   // byte offset of the lane's 16 nibble bytes in the superblock
        int lo6;         // c < 2: the (scale, min) pairs are 6-bit fields of sc[j], sc[j+4]
        uint32_t bsh;    // bit offset of the byte of sub-block j = 2c in its dword
    };
    __device__ static Lane lane(int gl) {
        const int c8 = gl & 7, c = c8 >> 1, hh = c8 & 1;
        Lane l;
        l.boff = (uint32_t)(gl >> 3) * 144u;
        l.e = (gl >> 3) * 256 + 64 * c + 16 * hh;
        l.qoff = 16u + 16u * (uint32_t)c8;
        l.lo6 = c < 2;
        l.bsh = 16u * (uint32_t)(c & 1);
        return l;
    }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)(lpr / 8) * 144u; }
    static constexpr int rel0(int s) { return 4 * s; }
    static constexpr int rel1(int s) { return 32 + 4 * s; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    u32x4 hdr, qs;
    float D0, M0, D1, M1;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int, int, const Lane& l) {
        hdr = ld128(wr, off);
        qs = ld128(wr, off + l.qoff);
    }
    // (scale, min) of sub-blocks j = 2c (field at bit b) and 2c+1 (b + 8):
    // j < 4: scale = sc[j] & 63, min = sc[j+4] & 63;
    // j >= 4: scale = (sc[j+4] & 15) | (sc[j-4] >> 6) << 4,
    //         min   = (sc[j+4] >> 4) | (sc[j]   >> 6) << 4.
    // sc[0..3] = hdr.y, sc[4..7] = hdr.z, sc[8..11] = hdr.w.
    __device__ __forceinline__ void prep(const Lane& l) {
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        const uint32_t sa = l.lo6 ? hdr.y : hdr.w;  // holds the low 4 bits of the scale
        const uint32_t ma = l.lo6 ? hdr.z : hdr.w;  // holds the low 4 bits of the min
        const uint32_t mas = l.lo6 ? 0u : 4u;
        const uint32_t hs = l.lo6 ? 4u : 6u;        // position of the 2 high bits
        float Dv[2], Mv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t b = l.bsh + 8u * t;
            const uint32_t sc = __builtin_amdgcn_ubfe(sa, b, 4) | (__builtin_amdgcn_ubfe(hdr.y, b + hs, 2) << 4);
            const uint32_t mn = __builtin_amdgcn_ubfe(ma, b + mas, 4) | (__builtin_amdgcn_ubfe(hdr.z, b + hs, 2) << 4);
            Dv[t] = d * (float)sc;
            Mv[t] = dmin * (float)mn;
        }
        D0 = Dv[0]; M0 = Mv[0]; D1 = Dv[1]; M1 = Mv[1];
    }
    __device__ __forceinline__ float runA(int r) const { return r == 0 ? D0 : D1; }
    __device__ __forceinline__ float runB(int r) const { return r == 0 ? M0 : M1; }
    // sub-block 2c: low nibbles in place (q * 2^-24); 2c+1: high (q * 2^-20)
    static constexpr bool PACKED = true;
    static constexpr float pscale(int r) { return r == 0 ? 16777216.0f : 1048576.0f; }
    __device__ __forceinline__ void qpack(int s, uint32_t (&p)[4]) const {
        const uint32_t v = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w)), v8 = v >> 8;
        p[0] = v & 0x000F000Fu;
        p[1] = v8 & 0x000F000Fu;
        p[2] = v & 0x00F000F0u;
        p[3] = v8 & 0x00F000F0u;
    }
    __device__ __forceinline__ void qsub(int s, float (&q)[8]) const {
        const uint32_t v = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
        const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            q[b] = ubyte_f32(lo, b);
            q[4 + b] = ubyte_f32(hi, b);
        }
    }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float&, float&) const {
        const uint32_t q = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
        const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = __builtin_fmaf(D0, ubyte_f32(lo, b), -M0);
            w[4 + b] = __builtin_fmaf(D1, ubyte_f32(hi, b), -M1);
        }
    }
};

// Q6_K: 64 weights of a 210-byte superblock: half h, l in [l0, l0+16) of the
// half's four quarters.  Reads 16 bytes of ql for quarters 0/2, 16 for 1/3,
// 16 bytes of qh, the 8 scale bytes of the half and d.  (gl & 3 fixes h and
// l0 for every uu, LPR >= 4.)
template <> struct GUnit<QT_Q6_K> {
    static constexpr int UE = 64, S = 8, MIN_LPR = 4;
    static constexpr bool SCALED = true;  // d * scale is common to each 16-run
    static constexpr int RUNS = 4;  // w = D_g*q - 32*D_g; run g = quarter g (sub-units 2g, 2g+1)
    static constexpr int run0(int s) { return s >> 1; }
    static constexpr int run1(int s) { return s >> 1; }
    static constexpr int lastsub(int r) { return 2 * r + 1; }
    static constexpr int runrel(int r) { return 32 * r; }
    struct Lane : LaneBase {
        uint32_t oa, ob, oh, os;  // byte offsets (in the superblock) of the four spans
        uint32_t so;              // bit offset of the half's first used scale byte
    };
    __device__ static Lane lane(int gl) {
        const int h = (gl >> 1) & 1, l0 = 16 * (gl & 1);
        Lane l;
        l.boff = (uint32_t)(gl >> 2) * 210u;
        l.e = (gl >> 2) * 256 + 128 * h + l0;
        l.oa = 64u * h + l0;
        l.ob = 64u * h + 32u + l0;
        l.oh = 128u + 32u * h + l0;
        l.os = 192u + 8u * h;
        l.so = 8u * (uint32_t)(l0 >> 4);
        return l;
    }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)(lpr / 4) * 210u; }
    // sub-unit s: quarter g = s/2, 8 weights at l0 + 8*(s&1) of the quarter
    static constexpr int rel0(int s) { return 32 * (s >> 1) + 8 * (s & 1); }
    static constexpr int rel1(int s) { return rel0(s) + 4; }
    static constexpr int prel0(int s) { return rel0(s) + ((s >> 1) >= 2 ? 4 : 0); }
    static constexpr int prel1(int s) { return rel1(s) + ((s >> 1) >= 2 ? 4 : 0); }
    uint32_t ra[5], rb[5], rh[5], rs[3], rd, sh;
    float D[4];
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int, int, const Lane& l) {
        sh = off & 3u;
        ld_span<5>(wr, off + l.oa, ra);
        ld_span<5>(wr, off + l.ob, rb);
        ld_span<5>(wr, off + l.oh, rh);
        ld_span<3>(wr, off + l.os, rs);
        rd = ld32(wr, (off + 208u) & ~3u);
    }
    __device__ __forceinline__ void prep(const Lane& l) {
        const float d = h2f(rd >> (8u * sh));
        const uint32_t sc0 = shr64(rs[0], rs[1], sh), sc1 = shr64(rs[1], rs[2], sh);
        // quarter g uses scale byte 2g + l0/16 of the half
        D[0] = d * (float)(int8_t)(sc0 >> l.so);
        D[1] = d * (float)(int8_t)(sc0 >> (l.so + 16u));
        D[2] = d * (float)(int8_t)(sc1 >> l.so);
        D[3] = d * (float)(int8_t)(sc1 >> (l.so + 16u));
    }
    __device__ __forceinline__ float runA(int r) const { return D[r]; }
    __device__ __forceinline__ float runB(int r) const { return 32.0f * D[r]; }
    // q = low nibble | 2 high bits << 4, built in place: quarters 0/1 take
    // the low nibbles of ql (q * 2^-24), quarters 2/3 the high ones (q * 2^-20)
    static constexpr bool PACKED = true;
    static constexpr float pscale(int r) { return r < 2 ? 16777216.0f : 1048576.0f; }
    __device__ __forceinline__ void qpack(int s, uint32_t (&p)[4]) const {
        const int g = s >> 1, i8 = s & 1;
        const uint32_t L0 = (g & 1) ? rb[2 * i8] : ra[2 * i8];
        const uint32_t L1 = (g & 1) ? rb[2 * i8 + 1] : ra[2 * i8 + 1];
        const uint32_t L2 = (g & 1) ? rb[2 * i8 + 2] : ra[2 * i8 + 2];
        const uint32_t l_a = shr64(L0, L1, sh), l_b = shr64(L1, L2, sh);
        const uint32_t h_a = shr64(rh[2 * i8], rh[2 * i8 + 1], sh);
        const uint32_t h_b = shr64(rh[2 * i8 + 1], rh[2 * i8 + 2], sh);
        const int nsh = g >= 2 ? 4 : 0;
        const uint32_t ML = 0x000F000Fu << nsh, MH = 0x00300030u << nsh;
        const int up = 4 + nsh - 2 * g, dn = 4 - nsh + 2 * g;  // qh field -> bits 4+nsh of bytes 0/2, 1/3
        p[0] = (l_a & ML) | ((h_a << up) & MH);
        p[1] = ((l_a >> 8) & ML) | ((h_a >> dn) & MH);
        p[2] = (l_b & ML) | ((h_b << up) & MH);
        p[3] = ((l_b >> 8) & ML) | ((h_b >> dn) & MH);
    }
    __device__ __forceinline__ void qsub(int s, float (&q)[8]) const {
        const int g = s >> 1, i8 = s & 1;
        const uint32_t L0 = (g & 1) ? rb[2 * i8] : ra[2 * i8];
        const uint32_t L1 = (g & 1) ? rb[2 * i8 + 1] : ra[2 * i8 + 1];
        const uint32_t L2 = (g & 1) ? rb[2 * i8 + 2] : ra[2 * i8 + 2];
        const uint32_t l_a = shr64(L0, L1, sh), l_b = shr64(L1, L2, sh);
        const uint32_t h_a = shr64(rh[2 * i8], rh[2 * i8 + 1], sh);
        const uint32_t h_b = shr64(rh[2 * i8 + 1], rh[2 * i8 + 2], sh);
        const int nsh = g >= 2 ? 4 : 0;
        const uint32_t qa = ((l_a >> nsh) & 0x0F0F0F0Fu) | (((h_a >> (2 * g)) & 0x03030303u) << 4);
        const uint32_t qb = ((l_b >> nsh) & 0x0F0F0F0Fu) | (((h_b >> (2 * g)) & 0x03030303u) << 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            q[b] = ubyte_f32(qa, b);
            q[4 + b] = ubyte_f32(qb, b);
        }
    }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float& f0, float& f1) const {
        const int g = s >> 1, i8 = s & 1;
        const uint32_t L0 = (g & 1) ? rb[2 * i8] : ra[2 * i8];
        const uint32_t L1 = (g & 1) ? rb[2 * i8 + 1] : ra[2 * i8 + 1];
        const uint32_t L2 = (g & 1) ? rb[2 * i8 + 2] : ra[2 * i8 + 2];
        const uint32_t l_a = shr64(L0, L1, sh), l_b = shr64(L1, L2, sh);
        const uint32_t h_a = shr64(rh[2 * i8], rh[2 * i8 + 1], sh);
        const uint32_t h_b = shr64(rh[2 * i8 + 1], rh[2 * i8 + 2], sh);
        const int nsh = g >= 2 ? 4 : 0;
        const uint32_t qa = ((l_a >> nsh) & 0x0F0F0F0Fu) | (((h_a >> (2 * g)) & 0x03030303u) << 4);
        const uint32_t qb = ((l_b >> nsh) & 0x0F0F0F0Fu) | (((h_b >> (2 * g)) & 0x03030303u) << 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = ubyte_f32(qa, b) - 32.0f;  // q - 32, exact
            w[4 + b] = ubyte_f32(qb, b) - 32.0f;
        }
        f0 = D[g];
        f1 = D[g];
    }
};

// NVFP4: one half (32 weights) of a 36-byte group: the group's scale dword
// and 16 bytes of E2M1 nibbles.  (gl & 1 fixes the half, LPR >= 2.)
template <> struct GUnit<QT_NVFP4> {
    static constexpr int UE = 32, S = 4, MIN_LPR = 2;
    static constexpr bool SCALED = true;  // one E4M3 factor per 16-weight run
    static constexpr int RUNS = 0;
    struct Lane : LaneBase {
        uint32_t hsh;  // 16 * h: the half's two scale bytes
        uint32_t qoff;
    };
    __device__ static Lane lane(int gl) {
        const int h = gl & 1;
        Lane l;
        l.boff = (uint32_t)(gl >> 1) * 36u;
        l.e = (gl >> 1) * 64 + 32 * h;
        l.hsh = 16u * (uint32_t)h;
        l.qoff = 4u + 16u * (uint32_t)h;
        return l;
    }
    __host__ __device__ static uint32_t ustep(int lpr) { return (uint32_t)(lpr / 2) * 36u; }
    static constexpr int rel0(int s) { return 4 * s; }
    static constexpr int rel1(int s) { return 16 + 4 * s; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    uint32_t sd;
    u32x4 qs;
    float s_lo, s_hi;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int, int, const Lane& l) {
        sd = ld32(wr, off);
        qs = ld128(wr, off + l.qoff);
    }
    __device__ __forceinline__ void prep(const Lane& l) {
        s_lo = e4m3_to_f32((sd >> l.hsh) & 0xFFu);
        s_hi = e4m3_to_f32((sd >> (l.hsh + 8u)) & 0xFFu);
    }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float& f0, float& f1) const {
        const uint32_t q = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x2 v = e2m1x2_to_f32(q, b);
            w[b] = v.x;
            w[4 + b] = v.y;
        }
        f0 = s_lo;
        f1 = s_hi;
    }
};

// NVFP4 V2: the same values as NVFP4 with a row's quant bytes first and its
// scale bytes after them (k/2 + 2g holds the two scales of 32-element group
// g).  A unit is one group: 16 quant bytes at 16g and the scale dword holding
// its two scale bytes.  The weights, their order and the arithmetic are those
// of GUnit<QT_NVFP4>, so both layouts give bit-identical results.
template <> struct GUnit<QT_NVFP4_V2> {
    static constexpr int UE = 32, S = 4, MIN_LPR = 1;
    static constexpr bool SCALED = true;
    static constexpr int RUNS = 0;
    struct Lane : LaneBase {};
    __device__ static Lane lane(int gl) {
        Lane l;
        l.boff = 16u * (uint32_t)gl;
        l.e = 32 * gl;
        return l;
    }
    __host__ __device__ static uint32_t ustep(int lpr) { return 16u * (uint32_t)lpr; }
    static constexpr int rel0(int s) { return 4 * s; }
    static constexpr int rel1(int s) { return 16 + 4 * s; }
    static constexpr int prel0(int s) { return rel0(s); }
    static constexpr int prel1(int s) { return rel1(s); }
    uint32_t sd, hsh;
    u32x4 qs;
    float s_lo, s_hi;
    // off: the group's quant bytes (row start + 16g); its scale bytes are at
    // row start + k/2 + 2g = off + k/2 - 14g (rows start 4-byte aligned).
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t off, int e, int k, const Lane&) {
        const uint32_t soff = off + (uint32_t)(k >> 1) - 14u * (uint32_t)(e >> 5);
        hsh = 8u * (soff & 3u);
        sd = ld32(wr, soff & ~3u);
        qs = ld128(wr, off);
    }
    __device__ __forceinline__ void prep(const Lane&) {
        s_lo = e4m3_to_f32((sd >> hsh) & 0xFFu);
        s_hi = e4m3_to_f32((sd >> (hsh + 8u)) & 0xFFu);
    }
    __device__ __forceinline__ void sub(int s, float (&w)[8], float& f0, float& f1) const {
        const uint32_t q = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x2 v = e2m1x2_to_f32(q, b);
            w[b] = v.x;
            w[4 + b] = v.y;
        }
        f0 = s_lo;
        f1 = s_hi;
    }
};

// ------------------------------------------------------------------ activations
// NT activation rows, either staged in LDS (4 floats of padding after every
// 64 so that the lanes of a wave, which read 16 bytes at unit-strided k
// offsets, fall on distinct banks) or read from global memory.
__device__ __forceinline__ int xpad(int e) { return e + ((e >> 6) << 2); }
__host__ __device__ constexpr int xpad_len(int k) { return k + ((k + 63) / 64) * 4; }

template <int NT, bool SUMS_ = false>
struct XLds {
    static constexpr bool SUMS = SUMS_;
    const float* s;  // [NT][xpad_len(k)]
    int ld;
    const float* sums;  // SUMS: [NT][k/16] sums of runs of 16 activations
    int nrun;
    struct Base { const float* p[NT]; };
    // sum of activations k .. k+15 of token j (k a multiple of 16)
    __device__ __forceinline__ float runsum(int k, int j) const { return sums[j * nrun + (k >> 4)]; }
    __device__ __forceinline__ Base base(int e) const {
        Base b;
        const int pe = xpad(e);
#pragma unroll
        for (int j = 0; j < NT; ++j) b.p[j] = s + j * ld + pe;
        return b;
    }
    template <int REL, int PREL>
    __device__ __forceinline__ f32x4 get(const Base& b, int j) const {
        return *(const f32x4*)(b.p[j] + PREL);
    }
};

template <int NT>
struct XGlobal {
    static constexpr bool SUMS = false;
    rsrc_t xr;
    uint32_t xoff[NT];
    struct Base { uint32_t o[NT]; };
    __device__ __forceinline__ Base base(int e) const {
        Base b;
#pragma unroll
        for (int j = 0; j < NT; ++j) b.o[j] = xoff[j] + 4u * (uint32_t)e;
        return b;
    }
    template <int REL, int PREL>
    __device__ __forceinline__ f32x4 get(const Base& b, int j) const {
        return __builtin_bit_cast(f32x4, ld128(xr, b.o[j] + 4u * REL));
    }
};

// Stage rows xoff[j] (j < NT) of x (row length k) into LDS in the padded
// layout, in two phases.  issue() loads the first batch into registers (each
// thread at least 8 independent 16-byte loads); finish() writes it, stages
// the remaining batches, and ends with a barrier.  A stream issues the first
// batch before its weight loads: waits count loads in issue order, so the
// activations then land without waiting for the weights.  With SUMS, the sums
// of each run of 16 activations (k/16 per row, k a multiple of 16) follow the
// rows: ((x0+x1)+(x2+x3)) + ... in a fixed order.
template <int NT, bool SUMS = false, int TPB = 256>
struct XStage {
    static constexpr int U = NT >= 8 ? 1 : 8 / NT;  // float4 columns per thread per batch
    float* sx;
    rsrc_t xr;
    uint32_t xoff[NT];
    int k;
    f32x4 v[NT][U];

    __device__ __forceinline__ void load(int c0) {
        const int per = k >> 2;  // float4 per row
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + TPB * u;
#pragma unroll
            for (int j = 0; j < NT; ++j)
                v[j][u] = __builtin_bit_cast(f32x4, ld128(xr, c < per ? xoff[j] + 16u * (uint32_t)c : OOB_OFF));
        }
    }
    __device__ __forceinline__ void store(int c0) {
        const int ld = xpad_len(k), per = k >> 2;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + TPB * u;
            if (c < per)
#pragma unroll
                for (int j = 0; j < NT; ++j) *(f32x4*)(sx + j * ld + xpad(4 * c)) = v[j][u];
        }
    }
    __device__ __forceinline__ void issue() { load((int)threadIdx.x); }
    __device__ __forceinline__ void finish() {
        store((int)threadIdx.x);
        for (int c0 = (int)threadIdx.x + TPB * U; c0 < (k >> 2); c0 += TPB * U) {
            load(c0);
            store(c0);
        }
        __syncthreads();
        if constexpr (SUMS) {
            const int ld = xpad_len(k), nrun = k >> 4;
            float* sums = sx + NT * ld;
            for (int t = threadIdx.x; t < NT * nrun; t += TPB) {
                const int j = t / nrun, r = t - j * nrun;
                const float* p = sx + j * ld + xpad(16 * r);  // 16 contiguous floats
                const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
                const f32x4 c = *(const f32x4*)(p + 8), d = *(const f32x4*)(p + 12);
                const float sa = (a.x + a.y) + (a.z + a.w), sb = (b.x + b.y) + (b.z + b.w);
                const float sc = (c.x + c.y) + (c.z + c.w), sd = (d.x + d.y) + (d.z + d.w);
                sums[t] = (sa + sb) + (sc + sd);
            }
            __syncthreads();
        }
    }
};

template <int NT, bool SUMS = false, int TPB = 256>
__device__ __forceinline__ XStage<NT, SUMS, TPB> make_xstage(float* sx, rsrc_t xr, const uint32_t (&xoff)[NT],
                                                            int k) {
    XStage<NT, SUMS, TPB> st;
    st.sx = sx;
    st.xr = xr;
#pragma unroll
    for (int j = 0; j < NT; ++j) st.xoff[j] = xoff[j];
    st.k = k;
    return st;
}

// LDS floats of NT staged rows (and their run sums).
__host__ __device__ constexpr int xlds_floats(int nt, int k, bool sums) {
    return nt * xpad_len(k) + (sums ? nt * (k >> 4) : 0);
}

// ------------------------------------------------------------------ core

struct StreamGeom {
    const uint8_t* w;  // packed rows
    int64_t m;         // rows
    int64_t rb;        // bytes per row
    int k;             // weights per row
    int lpr_log2;      // lanes per lane group = 1 << lpr_log2
};

template <int QT, int NT, int R, typename XS, int S_>
__device__ __forceinline__ void sub_fma(const GUnit<QT> (&un)[R], const XS& xs,
                                        const typename XS::Base& xb, int k, int e,
                                        float (&part)[R][NT]) {
    using UT = GUnit<QT>;
    float wv[R][8], f0[R], f1[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) un[rr].sub(S_, wv[rr], f0[rr], f1[rr]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        f32x4 xa = xs.template get<UT::rel0(S_), UT::prel0(S_)>(xb, j);
        f32x4 xb4 = xs.template get<UT::rel1(S_), UT::prel1(S_)>(xb, j);
        if constexpr (QT == QT_F32) {  // runs past k belong to the next row
            if (e + UT::rel0(S_) >= k) xa = f32x4{0.f, 0.f, 0.f, 0.f};
            if (e + UT::rel1(S_) >= k) xb4 = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            if constexpr (UT::SCALED) {
                float p0 = wv[rr][0] * xa.x;
                p0 = __builtin_fmaf(wv[rr][1], xa.y, p0);
                p0 = __builtin_fmaf(wv[rr][2], xa.z, p0);
                p0 = __builtin_fmaf(wv[rr][3], xa.w, p0);
                float p1 = wv[rr][4] * xb4.x;
                p1 = __builtin_fmaf(wv[rr][5], xb4.y, p1);
                p1 = __builtin_fmaf(wv[rr][6], xb4.z, p1);
                p1 = __builtin_fmaf(wv[rr][7], xb4.w, p1);
                const float p = __builtin_fmaf(f0[rr], p0, part[rr][j]);
                part[rr][j] = __builtin_fmaf(f1[rr], p1, p);
            } else {
                float p = part[rr][j];
                p = __builtin_fmaf(wv[rr][0], xa.x, p);
                p = __builtin_fmaf(wv[rr][1], xa.y, p);
                p = __builtin_fmaf(wv[rr][2], xa.z, p);
                p = __builtin_fmaf(wv[rr][3], xa.w, p);
                p = __builtin_fmaf(wv[rr][4], xb4.x, p);
                p = __builtin_fmaf(wv[rr][5], xb4.y, p);
                p = __builtin_fmaf(wv[rr][6], xb4.z, p);
                p = __builtin_fmaf(wv[rr][7], xb4.w, p);
                part[rr][j] = p;
            }
        }
    }
}

// Whether the sub-units of an offset format take the packed-half form: with
// one activation row only.  Each v_fma_mix_f32 widens its half again, and
// with several rows the widened q of the float form, shared by the rows'
// FMAs, cost less (14336x4096 Q4_K at n = 4..32 ran 10-17% slower packed;
// n = 1 ran 3.5% faster).
template <typename UT, int NT>
__host__ __device__ constexpr bool packed_q() { return UT::PACKED && NT == 1; }

// A_r of run r, times the packing scale of its q when packed.
template <typename UT, bool PK>
__device__ __forceinline__ float run_a(const UT& u, int r) {
    if constexpr (PK) return u.runA(r) * UT::pscale(r);
    else return u.runA(r);
}

// Sub-unit S_ of an offset format (RUNS > 0) with run sums of x: the q*x
// products of each run accumulate in P (slot r & 1; a run's 16 FMAs form one
// chain); after the run's last sub-unit, part += A_r*P - B_r*sum(x of run).
template <int QT, int NT, int R, typename XS, int S_>
__device__ __forceinline__ void sub_runs(const GUnit<QT> (&un)[R], const XS& xs,
                                         const typename XS::Base& xb, int e, float (&P)[R][NT][2],
                                         float (&part)[R][NT]) {
    using UT = GUnit<QT>;
    constexpr int r0 = UT::run0(S_), r1 = UT::run1(S_);
    constexpr bool PK = packed_q<UT, NT>();
    float q[R][8];
    uint32_t pq[R][4];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        if constexpr (PK) un[rr].qpack(S_, pq[rr]);
        else un[rr].qsub(S_, q[rr]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const f32x4 xa = xs.template get<UT::rel0(S_), UT::prel0(S_)>(xb, j);
        const f32x4 xb4 = xs.template get<UT::rel1(S_), UT::prel1(S_)>(xb, j);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            float& pa = P[rr][j][r0 & 1];
            float& pb = P[rr][j][r1 & 1];
            if constexpr (PK) {
                pa = __builtin_fmaf(f16lo(pq[rr][0]), xa.x, pa);
                pa = __builtin_fmaf(f16lo(pq[rr][1]), xa.y, pa);
                pa = __builtin_fmaf(f16hi(pq[rr][0]), xa.z, pa);
                pa = __builtin_fmaf(f16hi(pq[rr][1]), xa.w, pa);
                pb = __builtin_fmaf(f16lo(pq[rr][2]), xb4.x, pb);
                pb = __builtin_fmaf(f16lo(pq[rr][3]), xb4.y, pb);
                pb = __builtin_fmaf(f16hi(pq[rr][2]), xb4.z, pb);
                pb = __builtin_fmaf(f16hi(pq[rr][3]), xb4.w, pb);
            } else {
                pa = __builtin_fmaf(q[rr][0], xa.x, pa);
                pa = __builtin_fmaf(q[rr][1], xa.y, pa);
                pa = __builtin_fmaf(q[rr][2], xa.z, pa);
                pa = __builtin_fmaf(q[rr][3], xa.w, pa);
                pb = __builtin_fmaf(q[rr][4], xb4.x, pb);
                pb = __builtin_fmaf(q[rr][5], xb4.y, pb);
                pb = __builtin_fmaf(q[rr][6], xb4.z, pb);
                pb = __builtin_fmaf(q[rr][7], xb4.w, pb);
            }
        }
        if constexpr (S_ == UT::lastsub(r0)) {
            const float sx = xs.runsum(e + UT::runrel(r0), j);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const float t = __builtin_fmaf(run_a<UT, PK>(un[rr], r0), P[rr][j][r0 & 1], part[rr][j]);
                part[rr][j] = __builtin_fmaf(-un[rr].runB(r0), sx, t);
                P[rr][j][r0 & 1] = 0.0f;
            }
        }
        if constexpr (r1 != r0 && S_ == UT::lastsub(r1)) {
            const float sx = xs.runsum(e + UT::runrel(r1), j);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const float t = __builtin_fmaf(run_a<UT, PK>(un[rr], r1), P[rr][j][r1 & 1], part[rr][j]);
                part[rr][j] = __builtin_fmaf(-un[rr].runB(r1), sx, t);
                P[rr][j][r1 & 1] = 0.0f;
            }
        }
    }
}

template <int QT, int NT, int R, typename XS, int S_ = 0>
__device__ __forceinline__ void sub_all(const GUnit<QT> (&un)[R], const XS& xs,
                                        const typename XS::Base& xb, int k, int e,
                                        float (&part)[R][NT]) {
    if constexpr (S_ < GUnit<QT>::S) {
        sub_fma<QT, NT, R, XS, S_>(un, xs, xb, k, e, part);
        sub_all<QT, NT, R, XS, S_ + 1>(un, xs, xb, k, e, part);
    }
}

template <int QT, int NT, int R, typename XS, int S_ = 0>
__device__ __forceinline__ void sub_all_runs(const GUnit<QT> (&un)[R], const XS& xs,
                                             const typename XS::Base& xb, int e,
                                             float (&P)[R][NT][2], float (&part)[R][NT]) {
    if constexpr (S_ < GUnit<QT>::S) {
        sub_runs<QT, NT, R, XS, S_>(un, xs, xb, e, P, part);
        sub_all_runs<QT, NT, R, XS, S_ + 1>(un, xs, xb, e, P, part);
    }
}

template <int QT, int NT, int R, typename XS>
__device__ __forceinline__ void compute_item(GUnit<QT> (&un)[R], const typename GUnit<QT>::Lane& ln,
                                             int e, int k, const XS& xs, float (&acc)[R][NT]) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) un[rr].prep(ln);
    float part[R][NT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int j = 0; j < NT; ++j) part[rr][j] = 0.0f;
    const typename XS::Base xb = xs.base(e);
    if constexpr (GUnit<QT>::RUNS > 0 && XS::SUMS) {
        float P[R][NT][2];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NT; ++j) P[rr][j][0] = P[rr][j][1] = 0.0f;
        sub_all_runs<QT, NT, R, XS>(un, xs, xb, e, P, part);
    } else {
        sub_all<QT, NT, R, XS>(un, xs, xb, k, e, part);
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[rr][j] += part[rr][j];
}

// ------------------------------------------------------------------ Q8_1 activations
// NT rows of Q8_1 activations staged in LDS: the int8 codes as f16 (exact),
// 8 halves of padding after every 32 (one quantization block, one NVFP4 unit)
// so the 16-byte reads of a wave's lanes at unit-strided offsets spread over
// the banks, then each row's k/32 block scales.
__host__ __device__ constexpr int q8pad_len(int k) { return k / 32 * 40; }
__host__ __device__ constexpr int q8lds_bytes(int nt, int k) { return nt * (q8pad_len(k) * 2 + k / 32 * 4); }

template <int NT>
struct XLdsQ8 {
    static constexpr bool SUMS = false;
    const _Float16* s;  // [NT][q8pad_len(k)]
    int ld;
    const float* d;     // [NT][k/32]
    int nblk;
};

// Stage NT Q8_1 rows: codes at byte offsets qoff[j] of qr, scales at byte
// offsets doff[j] of dr.
template <int NT>
__device__ __forceinline__ void stage_q8(_Float16* sx, rsrc_t qr, rsrc_t dr, const uint32_t (&qoff)[NT],
                                         const uint32_t (&doff)[NT], int k) {
    const int ld = q8pad_len(k), nblk = k / 32;
    float* sd = (float*)(sx + NT * ld);
    const int per = k >> 4;  // 16-code chunks per row
    // rows one after another (compile-time j: a wave-varying index into the
    // offset arrays would put them in scratch memory)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        for (int cc = threadIdx.x; cc < per; cc += 256) {
            const u32x4 v = ld128(qr, qoff[j] + 16u * (uint32_t)cc);
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
            f16x8 h0, h1;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                h0[b] = (_Float16)(float)(int8_t)(vw[b >> 2] >> (8 * (b & 3)));
                h1[b] = (_Float16)(float)(int8_t)(vw[2 + (b >> 2)] >> (8 * (b & 3)));
            }
            _Float16* dst = sx + j * ld + (cc >> 1) * 40 + (cc & 1) * 16;
            *(u32x4*)dst = __builtin_bit_cast(u32x4, h0);
            *(u32x4*)(dst + 8) = __builtin_bit_cast(u32x4, h1);
        }
        for (int b = threadIdx.x; b < nblk; b += 256)
            sd[j * nblk + b] = __builtin_bit_cast(float, ld32(dr, doff[j] + 4u * (uint32_t)b));
    }
    __syncthreads();
}

// stage_q8 as a stream's staging step (no early loads).
template <int NT>
struct Q8Stage {
    _Float16* sx;
    rsrc_t qr, dr;
    uint32_t qoff[NT], doff[NT];
    int k;
    __device__ __forceinline__ void issue() {}
    __device__ __forceinline__ void finish() { stage_q8<NT>(sx, qr, dr, qoff, doff, k); }
};

// One NVFP4 unit (32 weights: two groups of 16 with their E4M3 scales)
// against Q8_1 rows.  Each group's dot product is exact: E2M1 values and
// int8 codes are exact in f16, their products and the sums of 16 of them
// exact in f32 (v_dot2_f32_f16), as an integer dot product would be.  Then
// acc += d_block * (s_lo * dot_lo + s_hi * dot_hi).
template <int QT, int NT, int R>
__device__ __forceinline__ void compute_item(GUnit<QT> (&un)[R], const typename GUnit<QT>::Lane& ln,
                                             int e, int, const XLdsQ8<NT>& xs, float (&acc)[R][NT]) {
    static_assert(QT == QT_NVFP4 || QT == QT_NVFP4_V2, "Q8_1 activations with NVFP4 weights only");
    f16x2 wl[R][8], wh[R][8];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        un[rr].prep(ln);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t q = s == 0 ? un[rr].qs.x : (s == 1 ? un[rr].qs.y : (s == 2 ? un[rr].qs.z : un[rr].qs.w));
            // low nibbles of bytes 0,1 (2,3) into byte 0 (2): weights 4s..4s+3
            const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
            const uint32_t tl = lo | (lo >> 4), th = hi | (hi >> 4);
            wl[rr][2 * s] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(tl, 1.0f, 0);
            wl[rr][2 * s + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(tl, 1.0f, 2);
            wh[rr][2 * s] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(th, 1.0f, 0);
            wh[rr][2 * s + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(th, 1.0f, 2);
        }
    }
    const int pe = (e >> 5) * 40;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const _Float16* xp = xs.s + j * xs.ld + pe;
        f16x2 xl[8], xh[8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 a = *(const u32x4*)(xp + 8 * i);
            const u32x4 b = *(const u32x4*)(xp + 16 + 8 * i);
            // components copied to scalars first: hipcc compiles a bit_cast of
            // a vector-element expression (a.y) as one of the vector's first
            // element
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xl[4 * i + c] = __builtin_bit_cast(f16x2, av[c]);
                xh[4 * i + c] = __builtin_bit_cast(f16x2, bv[c]);
            }
        }
        const float db = xs.d[j * xs.nblk + (e >> 5)];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            float sl = 0.0f, sh = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sl = __builtin_amdgcn_fdot2(wl[rr][i], xl[i], sl, false);
                sh = __builtin_amdgcn_fdot2(wh[rr][i], xh[i], sh, false);
            }
            acc[rr][j] = __builtin_fmaf(db, __builtin_fmaf(un[rr].s_lo, sl, un[rr].s_hi * sh), acc[rr][j]);
        }
    }
}

// Issue the loads of item (row group rg, unit iteration uu) into un[].
// Callers issue every ring refill, also for items past the end (live =
// false), so that the number of loads issued after any item is the same on
// every path and the compiler's wait before an item counts only that item's
// loads, not all of those in flight.
// The descriptor covers the row group's rows from the 16-byte boundary at or
// below its first byte (wave-uniform, scalar registers); a lane's offset is
// its per-lane row/unit constant plus the group's sub-16 remainder and uu
// times the format's step.  lane_ok = false sends this lane's loads past
// the descriptor's end (zeros) while the descriptor stays wave-uniform.
template <int QT, int R>
__device__ __forceinline__ void issue_item(GUnit<QT> (&un)[R], const StreamGeom& g, int RG,
                                           uint32_t lane_row_off, const typename GUnit<QT>::Lane& ln,
                                           int rg, int uu, int e, bool live, bool lane_ok = true) {
    const int64_t row0 = (int64_t)rg * RG;
    const int64_t byte0 = row0 * g.rb;
    // an item past the end gets an empty descriptor: its loads return zeros
    const int64_t base = live ? byte0 & ~(int64_t)15 : 0;
    const int64_t end = live ? imin64(g.m, row0 + RG) * g.rb : 0;
    const rsrc_t wr = make_rsrc(g.w + base, (uint32_t)((end - base + 15) & ~(int64_t)15));
    const uint32_t off = lane_row_off + (uint32_t)(byte0 & 15) + ln.boff +
                         (uint32_t)uu * GUnit<QT>::ustep(1 << g.lpr_log2);
    const uint32_t off0 = lane_ok ? off : OOB_OFF;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) un[rr].load(wr, off0 + (uint32_t)(rr * g.rb), e, g.k, ln);
}

// ------------------------------------------------------------------ measurement twins
// XOR of a unit's raw words: the load-only twins keep their loads live
// with it in place of the decode and FMAs.
template <typename UT>
__device__ __forceinline__ uint32_t raw_xor(const UT& un);

template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_F32>& u) {
    uint32_t v = 0;
    for (int i = 0; i < 16; ++i) v ^= u.r[i];
    return v;
}
template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_Q4_0>& u) {
    return u.r[0] ^ u.r[1] ^ u.r[2] ^ u.r[3] ^ u.r[4];
}
template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_Q8_0>& u) {
    uint32_t v = 0;
    for (int i = 0; i < 9; ++i) v ^= u.r[i];
    return v;
}
template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_Q4_K>& u) {
    return u.hdr.x ^ u.hdr.y ^ u.hdr.z ^ u.hdr.w ^ u.qs.x ^ u.qs.y ^ u.qs.z ^ u.qs.w;
}
template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_Q6_K>& u) {
    uint32_t v = u.rd ^ u.rs[0] ^ u.rs[1] ^ u.rs[2];
    for (int i = 0; i < 5; ++i) v ^= u.ra[i] ^ u.rb[i] ^ u.rh[i];
    return v;
}
template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_NVFP4>& u) {
    return u.sd ^ u.qs.x ^ u.qs.y ^ u.qs.z ^ u.qs.w;
}

template <> __device__ __forceinline__ uint32_t raw_xor(const GUnit<QT_NVFP4_V2>& u) {
    return u.sd ^ u.qs.x ^ u.qs.y ^ u.qs.z ^ u.qs.w;
}

// Row groups first_rg, first_rg + rg_stride, ... < n_rg.  A row group is the
// RG = (64/LPR)*R rows that the wave's lane groups cover at once.  Items are
// numbered it = 0, 1, ...: row group first_rg + (it / upl) * rg_stride, unit
// iteration it % upl.  D items of weight loads are kept in flight in a ring
// of register sets (slot it % D, indexed at compile time); a slot is refilled
// with item it + D right after item it is consumed.  store(row, j, value) is
// called by lane gl == 0 of each lane group for every row (rows >= m too).
struct NoPre {
    __device__ void issue() {}
    __device__ void finish() {}
};

// pre.issue() is called by every wave before the ring's first loads and
// pre.finish() once they are issued (the work group's activation staging,
// with its barrier, goes there so that it overlaps the first weight loads).
// Position (row-group step q, unit uu) of a stream item, advanced by one
// item without the integer division it / upl (a division is about thirty
// scalar and vector instructions; the loops below advance two positions per
// item).
struct ItemPos {
    int q, uu;
    __device__ __forceinline__ void next(int upl) {
        if (++uu == upl) {
            uu = 0;
            ++q;
        }
    }
};

// ARM selects a measurement twin of the stream (the memra page's ceiling
// probe arms): STREAM_SERVED computes; STREAM_LOADONLY issues the same loads
// and folds the raw words into acc[rr][0] by XOR instead of decoding;
// STREAM_MATHONLY loads the first item's unit for every item (so every load
// hits the cache) and runs the full arithmetic on it.
enum : int { STREAM_SERVED = 0, STREAM_LOADONLY = 1, STREAM_MATHONLY = 2 };

template <int QT, int NT, int R, int D, typename XS, typename Store, typename Pre = NoPre,
          int ARM = STREAM_SERVED>
__device__ __forceinline__ void gemv_stream(const StreamGeom& g, int first_rg, int rg_stride,
                                            int n_rg, const XS& xs, Store store, Pre pre = {}) {
    using UT = GUnit<QT>;
    const int lane = threadIdx.x & 63;
    const int lpr = 1 << g.lpr_log2;
    const int gl = lane & (lpr - 1), slot = lane >> g.lpr_log2;
    const int RG = (64 >> g.lpr_log2) * R;
    const int U = (g.k + UT::UE - 1) / UT::UE;
    const int upl = (U + lpr - 1) >> g.lpr_log2;
    const int n_items = first_rg < n_rg ? (n_rg - first_rg + rg_stride - 1) / rg_stride * upl : 0;
    const typename UT::Lane ln = UT::lane(gl);
    const uint32_t lane_row_off = (uint32_t)(slot * R) * (uint32_t)g.rb;
    const int e_step = lpr * UT::UE;

    float acc[R][NT];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[rr][j] = 0.0f;

    // row group of item it complete: lane-group reduction, store, reset
    auto finish = [&](int q) {
        for (int off = lpr >> 1; off > 0; off >>= 1)
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[rr][j] += __shfl_xor(acc[rr][j], off, 64);
        if (gl == 0) {
            const int64_t r0 = (int64_t)(first_rg + q * rg_stride) * RG + slot * R;
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int j = 0; j < NT; ++j) store(r0 + rr, j, acc[rr][j]);
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[rr][j] = 0.0f;
    };

    UT ring[D][R];
    if (n_items <= D) {
        // Short stream: every item's loads are in flight before the first
        // is consumed.
        pre.issue();
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < n_items) {
                const int q = d / upl, uu = d - q * upl;
                issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + q * rg_stride, uu,
                                  ln.e + uu * e_step, true);
            }
        }
        pre.finish();
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < n_items) {
                const int q = d / upl, uu = d - q * upl;
                if (gl + lpr * uu < U) {
                    if constexpr (ARM == STREAM_LOADONLY) {
#pragma unroll
                        for (int rr = 0; rr < R; ++rr)
                            acc[rr][0] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, acc[rr][0]) ^
                                                                       raw_xor(ring[d][rr]));
                    } else {
                        compute_item<QT, NT, R>(ring[d], ln, ln.e + uu * e_step, g.k, xs, acc);
                    }
                }
                if (uu == upl - 1) finish(q);
            }
        }
        return;
    }
    // Long stream: a ring of D items.  Every refill is issued, also for items
    // past the end (they read nothing), so the wait before an item counts
    // only the loads issued after it on every path.
    pre.issue();
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int q = d / upl, uu = d - q * upl;
        issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + q * rg_stride, uu,
                          ln.e + uu * e_step, true);
    }
    pre.finish();
    ItemPos cur{0, 0}, nxt{D / upl, D - (D / upl) * upl};
    for (int base = 0; base < n_items; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = base + d;
            const bool live = it < n_items;  // wave-uniform
            const int q = cur.q, uu = cur.uu;
            if (live && gl + lpr * uu < U) {
                if constexpr (ARM == STREAM_LOADONLY) {
#pragma unroll
                    for (int rr = 0; rr < R; ++rr)
                        acc[rr][0] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, acc[rr][0]) ^
                                                                   raw_xor(ring[d][rr]));
                } else {
                    compute_item<QT, NT, R>(ring[d], ln, ln.e + uu * e_step, g.k, xs, acc);
                }
            }
            if constexpr (ARM == STREAM_MATHONLY)
                issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg, 0, ln.e, it + D < n_items);
            else
                issue_item<QT, R>(ring[d], g, RG, lane_row_off, ln, first_rg + nxt.q * rg_stride, nxt.uu,
                                  ln.e + nxt.uu * e_step, it + D < n_items);
            if (live && uu == upl - 1) finish(q);
            cur.next(upl);
            nxt.next(upl);
        }
    }
}

extern __shared__ __attribute__((aligned(16))) float qmm_dyn_lds[];

// ------------------------------------------------------------------ launch helpers

inline int unit_elems_of(int qt) {
    switch (qt) {
        case QT_F32: return GUnit<QT_F32>::UE;
        case QT_Q4_0: return GUnit<QT_Q4_0>::UE;
        case QT_Q8_0: return GUnit<QT_Q8_0>::UE;
        case QT_Q4_K: return GUnit<QT_Q4_K>::UE;
        case QT_Q6_K: return GUnit<QT_Q6_K>::UE;
        case QT_NVFP4: return GUnit<QT_NVFP4>::UE;
        case QT_NVFP4_V2: return GUnit<QT_NVFP4_V2>::UE;
    }
    return 0;
}

static inline int min_lpr(int qt) {
    switch (qt) {
        case QT_Q4_K: return GUnit<QT_Q4_K>::MIN_LPR;
        case QT_Q6_K: return GUnit<QT_Q6_K>::MIN_LPR;
        case QT_NVFP4: return GUnit<QT_NVFP4>::MIN_LPR;
        case QT_NVFP4_V2: return GUnit<QT_NVFP4_V2>::MIN_LPR;
    }
    return 1;
}

// log2 of the lane-group size: the largest power of two <= min(units, 64),
// and at least the format's MIN_LPR (a row then leaves lanes of its group
// idle rather than breaking the per-lane constant unit position).
// Lane groups down to 1 << LPR_CAP_MULTI lanes for the streams that apply
// each weight to several activation rows (GEMV n > 2, the MoE): a lane then
// takes more units of its row between two lane-group reductions, and a wave
// more rows at once.  Measured on 14336x4096 (q4_k / q6_k): n = 8 from
// 43.5 / 48.1 to 31.4 / 35.2 us, n = 32 from 125 / 128 to 98 / 96 us, the MoE
// gate/up at t = 16 from 210 to 188 us and the down projection from 119 to
// 97 us; at n = 1 whole-wave groups stay (q6_k 16.4 against 17.7 us).  The
// GEMV shrinks its groups only while the rows still give one row group per
// SIMD (on 1024x4608 q4_0, n = 4, 16-lane groups left 128 waves for 1024
// SIMDs: 17.3 against 9.3 us).
constexpr int LPR_CAP_SINGLE = 6;  // LPR_CAP_MULTI, LPR_CAP_MIN: kernels.hpp

static inline int lpr_for(int qt, int64_t k, int cap_log2) {
    const int ue = unit_elems_of(qt);
    const int64_t units = (k + ue - 1) / ue;
    int l = 0;
    while (l < cap_log2 && (int64_t(2) << l) <= units) ++l;
    while ((1 << l) < min_lpr(qt)) ++l;
    return l;
}

// Row-group size in rows for R rows per lane group.
static inline int64_t rg_rows(int lpr_log2, int R) { return (int64_t)(64 >> lpr_log2) * R; }


// Work groups for a stream of n_rg row groups shared by `sets` independent
// streams: about num_cu * wg_per_cu work groups in total, never more than one
// wave per row group.
static inline unsigned stream_grid(int64_t n_rg, int64_t sets, const GemvTuning& tune, int wpg = 4) {
    // rounded down: a few work groups past what is resident at once would run
    // as a second round (the whole time of a round again)
    int64_t target = (int64_t)tune.num_cu * tune.wg_per_cu / (sets > 0 ? sets : 1);
    if (target < 1) target = 1;
    const int64_t need = (n_rg + wpg - 1) / wpg;
    return (unsigned)(need < target ? need : target);
}

// Activations are staged in LDS when NT rows of them fit what one work group
// may allocate; the MoE kernel keeps to 64 KB.
constexpr int64_t XLDS_MAX_BYTES = 64 * 1024;

// The tuning with wg_per_cu lowered to the work groups of `lds` bytes each
// that fit in one CU's LDS at once.
static inline GemvTuning lds_limited(const GemvTuning& t, int64_t lds) {
    GemvTuning r = t;
    if (lds > 0) {
        const int64_t fit = t.lds_per_cu / lds;
        r.wg_per_cu = (int)(fit < 1 ? 1 : (fit < t.wg_per_cu ? fit : t.wg_per_cu));
    }
    return r;
}

// (R, D) variants compiled: NT <= 2: (1,4) (1,8) (2,2) (2,4); NT >= 4: (1,2) (1,4) (2,2).
template <int NT, typename F>
static void with_rd(const GemvTuning& t, F&& f) {
    if constexpr (NT <= 2) {
        if (t.rows >= 2) {
            if (t.depth >= 4) f(std::integral_constant<int, 2>{}, std::integral_constant<int, 4>{});
            else f(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
        } else {
            if (t.depth >= 8) f(std::integral_constant<int, 1>{}, std::integral_constant<int, 8>{});
            else f(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{});
        }
    } else {
        if (t.rows >= 2) f(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
        else if (t.depth >= 4) f(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{});
        else f(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    }
}

// Call CALL with the format as the compile-time constant Q.
#define QMM_QT_SWITCH(qt, CALL)                                     \
    switch (qt) {                                                   \
        case QT_F32: { constexpr int Q = QT_F32; CALL; break; }     \
        case QT_Q4_0: { constexpr int Q = QT_Q4_0; CALL; break; }   \
        case QT_Q8_0: { constexpr int Q = QT_Q8_0; CALL; break; }   \
        case QT_Q4_K: { constexpr int Q = QT_Q4_K; CALL; break; }   \
        case QT_Q6_K: { constexpr int Q = QT_Q6_K; CALL; break; }   \
        case QT_NVFP4: { constexpr int Q = QT_NVFP4; CALL; break; } \
        case QT_NVFP4_V2: { constexpr int Q = QT_NVFP4_V2; CALL; break; } \
    }

}  // namespace qmm
