// Prefill path, LDS-ring form: the packed weight bytes and the f16
// activations of each 64-k step are streamed straight from memory into a
// ring of NS LDS stages by buffer-to-LDS loads (buffer_load_dwordx4 ... lds),
// issued NS-1 steps ahead of their use.  No register holds data in flight,
// so the ring can be deep, and the k loop is a single rolled step.
//
// One work group of 4 waves computes a BM x BNT tile of dst (BM = 4*WR
// weight rows, BNT = 64, 128 or 256 tokens).  Wave w owns weight rows
// [w*WR, w*WR + WR) and all the tile's tokens; 256-token tiles halve the
// decode work per matrix-core op.  Per step it decodes its rows' packed bytes from the LDS
// stage straight into the A operands of v_mfma_f32_16x16x32_f16 (no decoded
// weight tile is written back to LDS), reads the B operands (f16 activations)
// from the stage, and runs (WR/16) x (BNT/16) x 2 matrix-core ops with f32
// accumulators.
//
// Operand layout of v_mfma_f32_16x16x32_f16: lane l holds A row l % 16 and B
// column l % 16, each at the 8 k slots 8*(l / 16) .. +7 of the op's 32; the
// result D[r][c] sits in lane (r / 4) * 16 + c, element r % 4.  A 64-k step
// is two such ops (ks = 0, 1) per 16 x 16 block, so lane (r16, g) of a wave
// needs, per weight row, the 16 weights in slots 32*ks + 8*g + i (i < 8).
// Each format assigns k values to slots so that these 16 weights come from a
// few adjacent packed bytes of the row (slot_k below); the activations are
// laid out in the same slot order by the f16 pre-pass, so the contraction
// over the step's 64 k values is unchanged.
//
// Step k sets: a step is k in [64 kt, 64 kt + 64), except Q6_K, whose step kt
// covers the two 32-runs of super-block kt/4 whose codes share one set of ql
// bytes (the ggml Q6_K layout: low and high nibbles of ql[l] belong to
// elements l and l + 64 of a 128-half).
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

typedef __attribute__((address_space(3))) void lds_void_t;

namespace lds_ring {

constexpr int LDS_BYTES = 160 * 1024;

// 16-byte chunks one weight row occupies in a stage (a pad chunk where it
// spreads rows over the LDS banks), and how a step's bytes are fetched.
template <int QT> struct Fmt;
template <> struct Fmt<QT_F32> { static constexpr int CPR = 16; };   // chunks XOR-swizzled per row
template <> struct Fmt<QT_Q4_0> { static constexpr int CPR = 3; };   // 36 B from a dword-aligned start
template <> struct Fmt<QT_Q8_0> { static constexpr int CPR = 5; };   // 68 B from a dword-aligned start
template <> struct Fmt<QT_Q4_K> { static constexpr int CPR = 3; };   // header 16 B + 32 B of qs
template <> struct Fmt<QT_Q6_K> { static constexpr int CPR = 9; };   // ql 32, qh 32, scales+d 18, pad
template <> struct Fmt<QT_NVFP4> { static constexpr int CPR = 3; };  // 36 B group

// KG k groups of 4 waves: group g computes the steps s0 + g, s0 + g + KG,
// ... of the item, so a CU holding one work group runs KG waves per SIMD.
// The ring holds NS stages, KG per round of steps.
template <int QT, int WR, int BNT, int KG, bool XF = false> struct Geo {
    static constexpr int BM = 4 * WR;
    // one stage's activations: BNT tokens x 64 f16 (XF: written by the work
    // group itself from the caller's f32 rows, rounded to f16 once)
    static constexpr int B_STAGE = BNT * 128;
    static constexpr int CPR = Fmt<QT>::CPR;
    static constexpr int A_ROWS_CHUNKS = BM * CPR;
    // the A loads of a stage cover whole rounds of 4 waves x 64 chunks; the
    // chunks past the rows' land in a tail of the stage nobody reads
    static constexpr int A_CHUNKS = (A_ROWS_CHUNKS + 255) / 256 * 256;
    static constexpr int A_STAGE = A_CHUNKS * 16;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int NR_FIT = LDS_BYTES / (KG * STAGE);     // rounds of KG stages that fit
    static constexpr int NR_HALF = LDS_BYTES / 2 / (KG * STAGE);  // ... in half the CU's LDS
    static constexpr int NR_MAX = KG == 1 && BNT == 128 && !XF ? 4 : 3;
    // Two work groups per CU (two waves per SIMD, one hiding the other's
    // load and LDS latency) beat one work group with a deeper ring by 20-45%
    // wherever a ring of two rounds fits in half the LDS: take the deepest
    // such ring, else the deepest ring of one work group.
    static constexpr int NR_PICK = NR_HALF >= 2 ? NR_HALF : NR_FIT;
    static constexpr int NR = NR_PICK > NR_MAX ? NR_MAX : NR_PICK;
    static constexpr int PER_CU = LDS_BYTES / (NR * KG * STAGE) >= 2 ? 2 : 1;  // work groups an LDS holds
    static constexpr int NS = NR * KG;
    static constexpr int DA = A_CHUNKS / 256;          // A loads per wave per step (64 chunks each)
    static constexpr int DB = XF ? 0 : B_STAGE / 4096;  // B loads to LDS per wave per step
    static constexpr int XC = XF ? BNT / 32 : 0;        // XF: 8-slot units a thread converts per step
    static constexpr int XL = 2 * XC;                   // XF: its 16-byte f32 loads per step
    // runnable: a ring of at least 2 rounds, its waits within vmcnt's range,
    // (KG = 2) room for group 1's accumulators in the ring's LDS, and (XF)
    // 64- or 128-token tiles with at most 3 rounds (the waits below assume them)
    static constexpr bool OK = NR >= 2 && (NR - 2) * (DA + DB + XL) <= 63 &&
                               (KG == 1 || NS * STAGE >= BM * BNT * 4) &&
                               (!XF || ((BNT == 128 || BNT == 64) && NR <= 3));
};

// k of slot s = 32*ks + 8*g + i of step kt (see the file comment).
template <int QT>
__host__ __device__ __forceinline__ int slot_k(int kt, int ks, int g, int i) {
    if constexpr (QT == QT_Q4_0 || QT == QT_NVFP4) {
        // byte 4g+b of a 32-run (16 packed bytes) holds elements 4g+b (low
        // nibble) and 16+4g+b (high nibble)
        return 64 * kt + 32 * ks + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
    } else if constexpr (QT == QT_Q6_K) {
        return 256 * (kt >> 2) + 128 * ((kt >> 1) & 1) + 64 * ks + 32 * (kt & 1) + 8 * g + i;
    } else {
        return 64 * kt + 32 * ks + 8 * g + i;  // identity
    }
}

// Byte offset (from the weight window's base) of chunk c of a row whose first
// byte is at rowoff, for step kt (pad chunks are masked by the caller).
template <int QT>
__device__ __forceinline__ uint32_t a_chunk_off(uint32_t rowoff, int c, int kt) {
    if constexpr (QT == QT_F32) {
        return rowoff + 256u * (uint32_t)kt + 16u * (uint32_t)c;
    } else if constexpr (QT == QT_Q4_0) {
        return ((rowoff + 36u * (uint32_t)kt) & ~3u) + 16u * (uint32_t)c;
    } else if constexpr (QT == QT_Q8_0) {
        return ((rowoff + 68u * (uint32_t)kt) & ~3u) + 16u * (uint32_t)c;
    } else if constexpr (QT == QT_Q4_K) {
        const uint32_t o = rowoff + 144u * ((uint32_t)kt >> 2);
        return c == 0 ? o : o + 16u + 32u * ((uint32_t)kt & 3u) + 16u * (uint32_t)(c - 1);
    } else if constexpr (QT == QT_Q6_K) {
        // c = 3*piece + chunk: pieces ql (64hh + 32kh), qh (128 + 32hh) and
        // scales + d (192), each from the dword at or below its first byte
        const uint32_t o = rowoff + 210u * ((uint32_t)kt >> 2);
        const uint32_t hh = ((uint32_t)kt >> 1) & 1u, kh = (uint32_t)kt & 1u;
        const int p = c >= 6 ? 2 : (c >= 3 ? 1 : 0);
        const uint32_t pb = p == 0 ? 64u * hh + 32u * kh : (p == 1 ? 128u + 32u * hh : 192u);
        return ((o + pb) & ~3u) + 16u * (uint32_t)(c - 3 * p);
    } else {  // NVFP4: 36-byte groups, rows a multiple of 4 bytes
        return rowoff + 36u * (uint32_t)kt + 16u * (uint32_t)c;
    }
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) { return *(const uint32_t*)p; }

// f16x8 A operand from four packed f16 pairs
__device__ __forceinline__ f16x8 frag4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(f16x8, v);
}

// (1024 + byte) as binary16 for bytes b0 and b0+1 of v, as one f16x2: one
// v_perm_b32 puts the two bytes under the exponent byte 0x64 (selectors 0-3
// pick bytes of v, 4 the constant's)
__device__ __forceinline__ f16x2 mpair(uint32_t v, int b0) {
    const uint32_t sel = b0 == 0 ? 0x04010400u : 0x04030402u;
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, v, sel));
}

// In-step slot of the first of the 4 consecutive k in f32 chunk c (slots
// 4c .. 4c+3) and its k offset from the step's base k (step_k0 below): every
// format's 64 slots are runs of 4 (or 8) consecutive k.
template <int QT>
__device__ __forceinline__ int chunk_rel_k(int c) {
    const int ks = c >> 3, g = (c >> 1) & 3, i = 4 * (c & 1);
    if constexpr (QT == QT_Q6_K)
        return 64 * ks + 8 * g + i;
    else
        return slot_k<QT>(0, ks, g, i);
}
template <int QT>
__device__ __forceinline__ int step_k0(int kt) {
    if constexpr (QT == QT_Q6_K)
        return 256 * (kt >> 2) + 128 * ((kt >> 1) & 1) + 32 * (kt & 1);
    else
        return 64 * kt;
}

// ------------------------------------------------------------ row decoders
// Decode one weight row's 16 weights of lane group g for the step into the
// two A operands (ks = 0, 1).  row: the row's bytes in the LDS stage;
// rowoff: its byte offset in the weight window (alignment of unaligned
// formats); kt: the step.

template <int QT> struct Dec;

template <> struct Dec<QT_F32> {
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t, int, int g, int rsw,
                                               f16x8& a0, f16x8& a1) {
        // chunk c of the row sits at chunk c ^ rsw (rsw = row & 15)
        auto ld = [&](int c) { return *(const f32x4*)(row + 16 * (c ^ rsw)); };
        const f32x4 p0 = ld(2 * g), p1 = ld(2 * g + 1), q0 = ld(8 + 2 * g), q1 = ld(9 + 2 * g);
        a0 = frag4(pack_f2h(p0.x, p0.y), pack_f2h(p0.z, p0.w), pack_f2h(p1.x, p1.y), pack_f2h(p1.z, p1.w));
        a1 = frag4(pack_f2h(q0.x, q0.y), pack_f2h(q0.z, q0.w), pack_f2h(q1.x, q1.y), pack_f2h(q1.z, q1.w));
    }
};

template <> struct Dec<QT_Q4_0> {
    // block ks (18 bytes) at byte sh + 18 ks of the stage row, sh = rowoff & 3
    __device__ __forceinline__ static f16x8 blk(const uint8_t* row, int sh, int ks, int g) {
        const int db = sh + 18 * ks;                    // d
        const uint32_t dw = lds_u32(row + (db & ~3));
        const _Float16 d = bits_h(dw >> (8 * (db & 3)));
        const int qb = db + 2 + 4 * g;                  // qs[4g .. 4g+3]
        const uint32_t q = __builtin_amdgcn_alignbyte(lds_u32(row + (qb & ~3) + 4), lds_u32(row + (qb & ~3)),
                                                      (uint32_t)(qb & 3));
        const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
        const f16x2 dd = {d, d}, off = {(_Float16)1032.0f, (_Float16)1032.0f};
        // (1024 + q) - 1032 = q - 8 exactly; one f16 rounding in the product
        return frag4(__builtin_bit_cast(uint32_t, (mpair(lo, 0) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(lo, 2) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(hi, 0) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(hi, 2) - off) * dd));
    }
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t rowoff, int, int g, int,
                                               f16x8& a0, f16x8& a1) {
        const int sh = (int)(rowoff & 3u);
        a0 = blk(row, sh, 0, g);
        a1 = blk(row, sh, 1, g);
    }
};

template <> struct Dec<QT_Q8_0> {
    __device__ __forceinline__ static f16x8 blk(const uint8_t* row, int sh, int ks, int g) {
        const int db = sh + 34 * ks;
        const uint32_t dw = lds_u32(row + (db & ~3));
        const _Float16 d = bits_h(dw >> (8 * (db & 3)));
        const int qb = db + 2 + 8 * g;                  // qs[8g .. 8g+7]
        const uint8_t* p = row + (qb & ~3);
        const uint32_t s = (uint32_t)(qb & 3);
        const uint32_t w0 = lds_u32(p), w1 = lds_u32(p + 4), w2 = lds_u32(p + 8);
        // int8 q -> byte q + 128 -> 1024 + q + 128 in f16, minus 1152 = q exactly
        const uint32_t qa = __builtin_amdgcn_alignbyte(w1, w0, s) ^ 0x80808080u;
        const uint32_t qc = __builtin_amdgcn_alignbyte(w2, w1, s) ^ 0x80808080u;
        const f16x2 dd = {d, d}, off = {(_Float16)1152.0f, (_Float16)1152.0f};
        return frag4(__builtin_bit_cast(uint32_t, (mpair(qa, 0) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(qa, 2) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(qc, 0) - off) * dd),
                     __builtin_bit_cast(uint32_t, (mpair(qc, 2) - off) * dd));
    }
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t rowoff, int, int g, int,
                                               f16x8& a0, f16x8& a1) {
        const int sh = (int)(rowoff & 3u);
        a0 = blk(row, sh, 0, g);
        a1 = blk(row, sh, 1, g);
    }
};

// 8 weights D*q - M from codes held as f16 halves (affine4h): e0, o0 the
// halves of codes 0..3, e1, o1 of codes 4..7; D24 = D * 2^24.
__device__ __forceinline__ f16x8 affine8h(uint32_t e0, uint32_t o0, uint32_t e1, uint32_t o1, float D24,
                                          float Mneg) {
    uint32_t p[4];
    affine4h(e0, o0, D24, Mneg, p[0], p[1]);
    affine4h(e1, o1, D24, Mneg, p[2], p[3]);
    return frag4(p[0], p[1], p[2], p[3]);
}

template <> struct Dec<QT_Q4_K> {
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t, int kt, int g, int,
                                               f16x8& a0, f16x8& a1) {
        const u32x4 hdr = *(const u32x4*)row;
        const u32x2 q = *(const u32x2*)(row + 16 + 8 * g);
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        // sub-blocks j0 = 2c (low nibbles) and j1 = 2c + 1 (high nibbles) of
        // chunk c = kt & 3.  With jj = j & 3, the packing uses the bytes
        // A = sc[jj], B = sc[jj + 4], C = sc[jj + 8]: for j < 4 the scale is
        // A & 63 and the min B & 63; for j >= 4 the scale is
        // (C & 15) | (A >> 6) << 4 and the min (C >> 4) | (B >> 6) << 4.
        const int c = kt & 3;  // the same for the whole wave
        const uint32_t sh0 = 16u * (uint32_t)(c & 1);  // byte jj0 = 2(c & 1), jj1 = jj0 + 1
        const uint32_t A = hdr.y >> sh0, B = hdr.z >> sh0, C = hdr.w >> sh0;
        uint32_t s0, m0, s1, m1;
        if (c < 2) {
            s0 = A & 63u;
            m0 = B & 63u;
            s1 = (A >> 8) & 63u;
            m1 = (B >> 8) & 63u;
        } else {
            s0 = (C & 15u) | (((A >> 6) & 3u) << 4);
            m0 = ((C >> 4) & 15u) | (((B >> 6) & 3u) << 4);
            s1 = ((C >> 8) & 15u) | (((A >> 14) & 3u) << 4);
            m1 = ((C >> 12) & 15u) | (((B >> 14) & 3u) << 4);
        }
        const float d24 = d * TWO24;
        const float D0 = d24 * (float)s0, M0 = dmin * (float)m0;
        const float D1 = d24 * (float)s1, M1 = dmin * (float)m1;
        // low nibbles: elements 0..7 of the step's first 32; high: of its second
        constexpr uint32_t N2 = 0x000F000Fu;
        a0 = affine8h(q.x & N2, (q.x >> 8) & N2, q.y & N2, (q.y >> 8) & N2, D0, -M0);
        a1 = affine8h((q.x >> 4) & N2, (q.x >> 12) & N2, (q.y >> 4) & N2, (q.y >> 12) & N2, D1, -M1);
    }
};

template <> struct Dec<QT_Q6_K> {
    // stage row: chunks 0-2 ql piece, 3-5 qh piece, 6-7 scales + d piece;
    // every piece starts at the dword at or below its first byte, sh = the
    // super-block's offset & 3 (0 or 2)
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t rowoff, int kt, int g, int,
                                               f16x8& a0, f16x8& a1) {
        const uint32_t sh = (rowoff + 210u * ((uint32_t)kt >> 2)) & 3u;
        const int hh = (kt >> 1) & 1, kh = kt & 1;
        const uint8_t* L = row + 8 * g;
        const uint8_t* H = row + 48 + 8 * g;
        const uint8_t* S = row + 96;
        const uint32_t l0 = __builtin_amdgcn_alignbyte(lds_u32(L + 4), lds_u32(L), sh);
        const uint32_t l1 = __builtin_amdgcn_alignbyte(lds_u32(L + 8), lds_u32(L + 4), sh);
        const uint32_t h0 = __builtin_amdgcn_alignbyte(lds_u32(H + 4), lds_u32(H), sh);
        const uint32_t h1 = __builtin_amdgcn_alignbyte(lds_u32(H + 8), lds_u32(H + 4), sh);
        const int i0 = (int)sh + 8 * hh + 2 * kh + (g >> 1), i1 = i0 + 4;  // scale bytes
        const int8_t sc0 = (int8_t)(lds_u32(S + (i0 & ~3)) >> (8 * (i0 & 3)));
        const int8_t sc1 = (int8_t)(lds_u32(S + (i1 & ~3)) >> (8 * (i1 & 3)));
        const float d = h2f(lds_u32(S + 16) >> (8 * sh));  // bytes sh+16, sh+17
        const float Dl = d * (float)sc0, Dh = d * (float)sc1;
        const int hs = 2 * kh;
        const uint32_t ql0 = (l0 & 0x0F0F0F0Fu) | (((h0 >> hs) & 0x03030303u) << 4);
        const uint32_t ql1 = (l1 & 0x0F0F0F0Fu) | (((h1 >> hs) & 0x03030303u) << 4);
        const uint32_t qh0 = ((l0 >> 4) & 0x0F0F0F0Fu) | (((h0 >> (hs + 4)) & 0x03030303u) << 4);
        const uint32_t qh1 = ((l1 >> 4) & 0x0F0F0F0Fu) | (((h1 >> (hs + 4)) & 0x03030303u) << 4);
        // one 6-bit code per byte: even bytes by a mask, odd ones by a permute
        constexpr uint32_t B2 = 0x00FF00FFu;
        a0 = affine8h(ql0 & B2, odd_bytes(ql0), ql1 & B2, odd_bytes(ql1), Dl * TWO24, -32.0f * Dl);
        a1 = affine8h(qh0 & B2, odd_bytes(qh0), qh1 & B2, odd_bytes(qh1), Dh * TWO24, -32.0f * Dh);
    }
};

template <> struct Dec<QT_NVFP4> {
    __device__ __forceinline__ static f16x8 half(uint32_t q, float sl, float sh_) {
        float lo[4], hi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x2 v = e2m1x2_to_f32(q, b);
            lo[b] = v.x * sl;   // exact: at most 5 significant bits, within f16 range
            hi[b] = v.y * sh_;
        }
        return frag4(pack_f2h(lo[0], lo[1]), pack_f2h(lo[2], lo[3]), pack_f2h(hi[0], hi[1]), pack_f2h(hi[2], hi[3]));
    }
    __device__ __forceinline__ static void run(const uint8_t* row, uint32_t, int, int g, int,
                                               f16x8& a0, f16x8& a1) {
        const uint32_t s = lds_u32(row);
        const uint32_t q0 = lds_u32(row + 4 + 4 * g), q1 = lds_u32(row + 20 + 4 * g);
        a0 = half(q0, e4m3_to_f32(s & 0xFFu), e4m3_to_f32((s >> 8) & 0xFFu));
        a1 = half(q1, e4m3_to_f32((s >> 16) & 0xFFu), e4m3_to_f32(s >> 24));
    }
};

// s_waitcnt with vmcnt(vm), lgkmcnt(lg), expcnt left free (gfx9 encoding)
template <int VM, int LG>
__device__ __forceinline__ void waitcnt() {
    static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "waitcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LG << 8));
}

}  // namespace lds_ring

// ------------------------------------------------------------ f16 pre-pass
// x16[j][64 kt + s] = f16(x[j][slot_k(kt, s)]) (round to nearest even), zero
// past k.  One thread per 8-slot unit (16 bytes out).
template <int QT>
__global__ __launch_bounds__(256) void x16_slot_kernel(uint16_t* __restrict__ x16, const float* __restrict__ x,
                                                       int n, int k, int kp, int ldx) {
    const int units = kp >> 3;
    const int64_t total = (int64_t)n * units;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int j = (int)(i / units), u = (int)(i - (int64_t)j * units);
        const int kt = u >> 3, ks = (u >> 2) & 1, g = u & 3;
        const int ka = lds_ring::slot_k<QT>(kt, ks, g, 0), kb = lds_ring::slot_k<QT>(kt, ks, g, 4);
        const float* xr = x + (int64_t)j * ldx;
        const f32x4 a = ka < k ? *(const f32x4*)(xr + ka) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 b = kb < k ? *(const f32x4*)(xr + kb) : f32x4{0.f, 0.f, 0.f, 0.f};
        *(u32x4*)(x16 + (int64_t)j * kp + 8 * (int64_t)u) =
            u32x4{pack_f2h(a.x, a.y), pack_f2h(a.z, a.w), pack_f2h(b.x, b.y), pack_f2h(b.z, b.w)};
    }
}

// ------------------------------------------------------------ the GEMM kernel
// Work items (k split z, tile) are dealt to the 8 XCDs in contiguous runs,
// weight-row tile fastest (as in the other prefill kernels).  Item z covers
// steps [z*sps, min(nk, (z+1)*sps)); with n_split > 1 it writes its partial
// tile to partial + z*splitk_stride(n, m), summed by splitk_sum_kernel.
// XF: the activations are the caller's f32 rows x (ldx floats apart) instead
// of the f16 pre-pass's rows x16 (kp halves apart).  Each thread of a k group
// loads XC 8-slot units of its group's step into registers one round ahead,
// and after the round's barrier writes them, rounded to f16 (nearest even),
// where the buffer-to-LDS loads would have put the pre-pass's rows: every
// activation is converted once per work group and no pre-pass runs.
// TG = 2 (8 waves, one k group): the two halves of the tile's tokens go to
// two sets of 4 waves that share every stage; wave w of each set decodes the
// same rows [w*WR, w*WR + WR) for its own BNT/2 tokens, and only the first
// set issues the stage loads.  With 256-row tiles this halves the activation
// bytes each weight row costs (LDS reads and L2 traffic) against 128-row
// tiles, for twice the decode per matrix-core op.
template <int QT, int WR, int BNT, int KG, bool XF, int TG>
__device__ __forceinline__ void gemm_lds_body(float* __restrict__ dst, const uint8_t* __restrict__ w,
                                              const uint16_t* __restrict__ x16, const float* __restrict__ x,
                                              int ldx, int m, int k, int n, int rb, int kp, int n_mb, int n_nb,
                                              int n_split, int sps, float* __restrict__ partial, int ldd,
                                              int nb_fast) {
    using G = lds_ring::Geo<QT, WR, BNT, KG, XF>;
    static_assert(G::OK, "no LDS ring of this shape fits");
    static_assert(TG == 1 || (TG == 2 && KG == 1 && !XF), "token groups: one k group, f16 activations");
    constexpr int BM = G::BM, BN = BNT, CPR = G::CPR, NR = G::NR, DA = G::DA, DB = G::DB;
    constexpr int RI = WR / 16, NJ = BN / 16 / TG;  // 16-row and 16-token blocks per wave
    __shared__ __attribute__((aligned(1024))) uint8_t lds[G::NS * G::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave_all = wave_id();
    const int grp = KG == 1 ? 0 : wave_all >> 2, wave = wave_all & 3;  // k group, wave in the group
    const int tg = TG == 1 ? 0 : wave_all >> 2;                        // token group
    const int jb = tg * NJ;                                            // its first token block
    const int r16 = lane & 15, g = lane >> 4;

    const int T = n_mb * n_nb, NI = T * n_split, L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3, per = NI >> 3, rem = NI & 7;
    const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int z = item / T, tile = item - z * T;
    // nb_fast: an XCD's run of items holds all token tiles of a few weight
    // tiles (each weight tile read into one L2), else all weight tiles of a
    // token tile; the host picks the order with the smaller total of bytes
    // that several XCDs read
    const int nb = nb_fast ? tile % n_nb : tile / n_mb;
    const int mb = nb_fast ? tile / n_nb : tile - nb * n_mb;
    const int64_t m0 = (int64_t)mb * BM, n0 = (int64_t)nb * BN;

    int64_t base;
    const rsrc_t wr = row_window(w, m0, BM, m, rb, base);
    const int ntok = (int)imin64(BN, n - n0);
    // token rows: x16 rows of kp halves, or x rows ldx floats apart (the
    // window ends with the last row's k floats)
    const rsrc_t xr = XF ? make_rsrc(x + n0 * ldx, ((uint32_t)(ntok - 1) * (uint32_t)ldx + (uint32_t)k) * 4u)
                         : make_rsrc(x16 + n0 * kp, (uint32_t)ntok * (uint32_t)kp * 2u);
    const uint32_t rowoff0 = (uint32_t)(m0 * rb - base);  // byte offset of the tile's first row

    const int nk_all = k >> 6;
    const int s0 = z * sps;
    const int nk = min(nk_all, s0 + sps);

    // This lane's chunks of the buffer-to-LDS loads of its group's stages:
    // A load u covers chunks (wave*DA + u)*64 + lane, B load u chunks
    // (wave*DB + u)*64 + lane.
    uint32_t a_rowoff[DA], a_dead[DA];
    int a_c[DA];
#pragma unroll
    for (int u = 0; u < DA; ++u) {
        const int q = (wave * DA + u) * 64 + lane;
        const int r = q / CPR, c = q - r * CPR;
        a_rowoff[u] = rowoff0 + (uint32_t)r * (uint32_t)rb;
        // F32 rows: physical chunk q % 16 holds logical chunk c ^ (r & 15)
        a_c[u] = QT == QT_F32 ? (c ^ (r & 15)) : c;
        // chunks of the stage's tail and Q6_K's pad chunk load zeros: their
        // offsets get bit 31 (past every window)
        a_dead[u] = (q >= G::A_ROWS_CHUNKS || (QT == QT_Q6_K && c == 8)) ? OOB_OFF : 0u;
    }
    // f16 rows: B load u covers token t = 8*(wave*DB + u) + lane/8, physical
    // chunk lane % 8 holding logical chunk (lane % 8) ^ (t % 8); the per-load
    // part of the offset is wave-uniform (a scalar offset).
    const uint32_t b_off0 = (uint32_t)(8 * wave * DB + (lane >> 3)) * (uint32_t)kp * 2u +
                            16u * (uint32_t)((lane & 7) ^ ((lane >> 3) & 7));
    // round r: group grp's step s0 + KG*r + grp into stage KG*slot + grp
    auto issue = [&](int r, int slot) {
        if (TG > 1 && tg != 0) return;  // the first token group loads the shared stages
        const int kt = s0 + KG * r + grp;
        uint8_t* sa = lds + (KG * slot + grp) * G::STAGE;
        uint8_t* sb = sa + G::A_STAGE;
        // steps past the item's end load zeros (bit 31: past every window)
        const uint32_t dead = kt < nk ? 0u : OOB_OFF;
#pragma unroll
        for (int u = 0; u < DA; ++u) {
            const uint32_t off = lds_ring::a_chunk_off<QT>(a_rowoff[u], a_c[u], kt) | a_dead[u] | dead;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)(sa + (wave * DA + u) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < DB; ++u) {
            const uint32_t soff = kt < nk ? 16u * (uint32_t)u * (uint32_t)kp + 128u * (uint32_t)kt : OOB_OFF;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(sb + (wave * DB + u) * 1024), 16, b_off0,
                                                     soff, 0, 0);
        }
    };

    // XF: thread lt of the group converts unit xc8 (slots 8*xc8 .. +7) of
    // tokens xt0 + 32q, q < XC: two 16-byte loads each (slots 8*xc8 .. +3 and
    // +4 .. +7, each 4 consecutive k), written as 16 bytes of f16 at the
    // unit's swizzled place in the token's 128-byte stage row.  The token and
    // the out-of-range bit sit in the vector offset (range-checked), the
    // step's first k in the scalar one.
    const int xlt = tid & 255, xc8 = xlt & 7, xt0 = xlt >> 3;
    const uint32_t xva = ((uint32_t)xt0 * (uint32_t)ldx + (uint32_t)lds_ring::chunk_rel_k<QT>(2 * xc8)) * 4u;
    const uint32_t xvb = ((uint32_t)xt0 * (uint32_t)ldx + (uint32_t)lds_ring::chunk_rel_k<QT>(2 * xc8 + 1)) * 4u;
    const uint32_t xwo = (uint32_t)xt0 * 128u + 16u * (uint32_t)(xc8 ^ (xt0 & 7));
    constexpr int XC1 = G::XC > 0 ? G::XC : 1;
    u32x4 xa[XC1], xb[XC1];
    auto xload = [&](int r) {
        if constexpr (XF) {
            const int kt = s0 + KG * r + grp;
            const uint32_t dead = kt < nk ? 0u : OOB_OFF;
            const uint32_t soff = kt < nk ? 4u * (uint32_t)lds_ring::step_k0<QT>(kt) : 0u;
#pragma unroll
            for (int q = 0; q < G::XC; ++q) {
                const uint32_t tq = 128u * (uint32_t)q * (uint32_t)ldx;  // 32q token rows
                xa[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (xva + tq) | dead, soff, 0);
                xb[q] = __builtin_amdgcn_raw_buffer_load_b128(xr, (xvb + tq) | dead, soff, 0);
            }
        }
    };
    auto xstore = [&](int slot) {
        if constexpr (XF) {
            uint8_t* sb = lds + (KG * slot + grp) * G::STAGE + G::A_STAGE;
#pragma unroll
            for (int q = 0; q < G::XC; ++q) {
                const f32x4 a = __builtin_bit_cast(f32x4, xa[q]), b = __builtin_bit_cast(f32x4, xb[q]);
                *(u32x4*)(sb + xwo + 4096u * (uint32_t)q) =
                    u32x4{pack_f2h(a.x, a.y), pack_f2h(a.z, a.w), pack_f2h(b.x, b.y), pack_f2h(b.z, b.w)};
            }
        }
    };

    f32x4 acc[RI][NJ];
#pragma unroll
    for (int i = 0; i < RI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this lane's weight rows in a stage, and their offsets in the window
    const int rbase = wave * WR + r16;
    const int bsw = 16 * (g ^ (r16 & 7));  // B chunk of slots [8g, 8g+8) of run ks = 0 (ks = 1: ^4 -> +64)
    // the B operand of token row bt for run ks: 8 f16
    auto bfrag = [&](const uint8_t* bt, int ks) -> f16x8 { return *(const f16x8*)(bt + (ks ? bsw ^ 64 : bsw)); };
    constexpr int BROW = 128;  // bytes of one token row of a stage

#pragma unroll
    for (int p = 0; p < NR - 1; ++p) issue(p, p);
    if constexpr (XF) {
        // round 0's activations in flight with the first rounds' weights
        // (their store waits for all of them), then round 1's
        xload(0);
        xstore(0);
        xload(1);
    }

    const int nrounds = (nk - s0 + KG - 1) / KG;
    int cur = 0;
    for (int r = 0; r < nrounds; ++r) {
        // this wave's loads of round r have landed (later rounds' stay in
        // flight), its LDS reads of round r-1 and writes of round r's
        // activations are done; then every wave's.  Loads issued after round
        // r's weights: rounds r+1 .. r+NR-2 of them, and (XF) the activations
        // of rounds r+2 .. r+NR-1, except at r = 0, where the first rounds'
        // weights and round 0's activations have landed before round 0's
        // activation store.
        if (XF && r == 0)
            lds_ring::waitcnt<G::XL, 0>();
        else
            lds_ring::waitcnt<(NR - 2) * (DA + DB + G::XL), 0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (XF) {
            // round r+1's activations into the stage round r+1-NR used (every
            // wave is past it), then round r+2's loads
            xstore(cur == NR - 1 ? 0 : cur + 1);
            xload(r + 2);
        }
        // refill the stages round r-1 used, NR-1 rounds ahead
        issue(r + NR - 1, cur == 0 ? NR - 1 : cur - 1);

        const int kt = s0 + KG * r + grp;
        const uint8_t* sa = lds + (KG * cur + grp) * G::STAGE;
        const uint8_t* sb = sa + G::A_STAGE;
        cur = cur == NR - 1 ? 0 : cur + 1;
        if (KG > 1 && kt >= nk) continue;  // this group's step of the last round is past the item's end
        if constexpr (NJ == 8) {
            // all B operands of the step in registers, rows decoded one by one
            f16x8 b0[8], b1[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint8_t* bt = sb + (16 * (jb + j) + r16) * BROW;
                b0[j] = bfrag(bt, 0);
                b1[j] = bfrag(bt, 1);
            }
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const int rr = rbase + 16 * i;
                f16x8 a0, a1;
                lds_ring::Dec<QT>::run(sa + rr * CPR * 16, rowoff0 + (uint32_t)rr * (uint32_t)rb, kt, g, rr & 15,
                                       a0, a1);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1[j], acc[i][j], 0, 0, 0);
                }
            }
        } else {
            // all rows' A operands in registers, B operands read per token block
            f16x8 a0[RI], a1[RI];
#pragma unroll
            for (int i = 0; i < RI; ++i) {
                const int rr = rbase + 16 * i;
                lds_ring::Dec<QT>::run(sa + rr * CPR * 16, rowoff0 + (uint32_t)rr * (uint32_t)rb, kt, g, rr & 15,
                                       a0[i], a1[i]);
            }
            // B operands PF token blocks ahead in a register ring, so each
            // block's LDS reads are in flight behind the matrix-core ops of
            // the blocks before it (with two work groups per CU; with one,
            // PF = 1 reads each block just before its use, as measured
            // faster there: Q6_K 14336x4096x2048 386 against 401 us)
            constexpr int PF = G::PER_CU == 2 ? 4 : 1;
            f16x8 bq0[PF], bq1[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                const uint8_t* bt = sb + (16 * (jb + j) + r16) * BROW;
                bq0[j] = bfrag(bt, 0);
                bq1[j] = bfrag(bt, 1);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f16x8 b0 = bq0[j % PF], b1 = bq1[j % PF];
                if (j + PF < NJ) {
                    const uint8_t* bt = sb + (16 * (jb + j + PF) + r16) * BROW;
                    bq0[j % PF] = bfrag(bt, 0);
                    bq1[j % PF] = bfrag(bt, 1);
                }
#pragma unroll
                for (int i = 0; i < RI; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[i], b0, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[i], b1, acc[i][j], 0, 0, 0);
                }
                // a scheduling fence per block: the scheduler would otherwise
                // sink each prefetch read down to its use
                if constexpr (PF > 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // drain the loads past the last step before the ring is reused or the
    // work group ends
    lds_ring::waitcnt<0, 0>();

    if constexpr (KG == 2) {
        // group 1 hands its accumulators to group 0 through the ring's LDS
        // (value v of lane tid at v*256 + tid); group 0 adds them to its own
        // (group 0's + group 1's: a fixed order)
        float* red = reinterpret_cast<float*>(lds);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // every wave is done with the ring
        asm volatile("" ::: "memory");
        const int lt = tid & 255;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < RI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[((i * NJ + j) * 4 + e) * 256 + lt] = acc[i][j][e];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int i = 0; i < RI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] += red[((i * NJ + j) * 4 + e) * 256 + lt];
    }

    float* out = n_split > 1 ? partial + (int64_t)z * splitk_stride(n, m) : dst;
    const int64_t ldo = n_split > 1 ? m : ldd;  // partials are dense
#pragma unroll
    for (int i = 0; i < RI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t mrow = m0 + wave * WR + i * 16 + g * 4;
            const int64_t tok = n0 + (jb + j) * 16 + r16;
            if (tok < n) {
                float* p = out + tok * ldo + mrow;
                const f32x4 v = acc[i][j];
                if ((ldo & 3) == 0 && mrow + 4 <= m) {
                    *(f32x4*)p = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (mrow + e < m) p[e] = v[e];
                }
            }
        }
    }
}

template <int QT, int WR, int BNT, int KG, bool XF>
__global__ __launch_bounds__(256 * KG, 1) void gemm_lds_kernel(float* __restrict__ dst, const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ x16,
                                                               const float* __restrict__ x, int ldx, int m, int k,
                                                               int n, int rb, int kp, int n_mb, int n_nb, int n_split,
                                                               int sps, float* __restrict__ partial, int ldd,
                                                               int nb_fast) {
    gemm_lds_body<QT, WR, BNT, KG, XF, 1>(dst, w, x16, x, ldx, m, k, n, rb, kp, n_mb, n_nb, n_split, sps, partial,
                                          ldd, nb_fast);
}

// 8 waves in two token groups (TG = 2 above) on f16 activations, one k group
template <int QT, int WR, int BNT>
__global__ __launch_bounds__(512, 1) void gemm_lds_tg_kernel(float* __restrict__ dst, const uint8_t* __restrict__ w,
                                                             const uint16_t* __restrict__ x16, int m, int k, int n,
                                                             int rb, int kp, int n_mb, int n_nb, int n_split, int sps,
                                                             float* __restrict__ partial, int ldd, int nb_fast) {
    gemm_lds_body<QT, WR, BNT, 1, false, 2>(dst, w, x16, nullptr, 0, m, k, n, rb, kp, n_mb, n_nb, n_split, sps,
                                            partial, ldd, nb_fast);
}

template <int QT>
static void launch_lds_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k, int64_t n,
                          int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd, hipStream_t st) {
    const int64_t kp = x16_row_halves(k);
    const bool xf = pl.x16 == 4 || pl.x16 == 6;  // f32 activations straight into the ring: no pre-pass
    uint16_t* x16 = (uint16_t*)ws;
    float* part = xf ? (float*)ws : (float*)((uint8_t*)ws + x16_bytes(n, k));
    if (!xf) {
        const int64_t total = n * (kp / 8);
        int64_t blocks = (total + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        x16_slot_kernel<QT><<<dim3((unsigned)blocks), 256, 0, st>>>(x16, x, (int)n, (int)k, (int)kp, (int)ldx);
    }
    const int bm = 64 * pl.wm, bn = pl.x16 == 3 || pl.x16 == 7 ? 256 : (pl.x16 == 5 || pl.x16 == 6 ? 64 : 128);
    const int n_mb = (int)((m + bm - 1) / bm), n_nb = (int)((n + bn - 1) / bn);
    const dim3 grid((unsigned)(n_mb * n_nb * pl.n_split));
    // Item order: with the weight tile fastest, every token tile's XCDs read
    // all the weights (about n_nb reads of w in all); with the token tile
    // fastest, every XCD reads about all the activations (min(8, n_mb)
    // reads of them).  Take the order that reads fewer bytes.
    const double w_bytes = (double)m * (double)rb, x_bytes = (double)n * (double)kp * (xf ? 4.0 : 2.0);
    const int nb_fast = (double)(n_nb - 1) * w_bytes > (double)((n_mb < 8 ? n_mb : 8) - 1) * x_bytes;
    // only shapes lds_ring_fits() accepts are planned
    const int bnt = bn, wr = pl.x16 == 3 ? 32 : 16 * pl.wm;
#define QMM_LDS_LAUNCH(WR_, BN_, KG_, XF_)                                                                      \
    if constexpr (lds_ring::Geo<QT, WR_, BN_, KG_, XF_>::OK) {                                                  \
        if (wr == WR_ && bnt == BN_ && pl.kg == KG_ && xf == XF_)                                               \
            gemm_lds_kernel<QT, WR_, BN_, KG_, XF_><<<grid, 256 * KG_, 0, st>>>(                                \
                dst, w, x16, x, (int)ldx, (int)m, (int)k, (int)n, (int)rb, (int)kp, n_mb, n_nb, pl.n_split,     \
                pl.sps, part, (int)ldd, nb_fast);                                                               \
    }
    if (pl.x16 == 7) {
        // 256 x 256 tiles, two token groups of 4 waves
        if constexpr (lds_ring::Geo<QT, 64, 256, 1, false>::OK)
            gemm_lds_tg_kernel<QT, 64, 256><<<grid, 512, 0, st>>>(dst, w, x16, (int)m, (int)k, (int)n, (int)rb,
                                                                 (int)kp, n_mb, n_nb, pl.n_split, pl.sps, part,
                                                                 (int)ldd, nb_fast);
    } else {
    QMM_LDS_LAUNCH(16, 64, 1, false)
    QMM_LDS_LAUNCH(16, 64, 2, false)
    QMM_LDS_LAUNCH(16, 64, 1, true)
    QMM_LDS_LAUNCH(16, 64, 2, true)
    QMM_LDS_LAUNCH(16, 128, 1, false)
    QMM_LDS_LAUNCH(16, 128, 2, false)
    QMM_LDS_LAUNCH(16, 128, 1, true)
    QMM_LDS_LAUNCH(16, 128, 2, true)
    QMM_LDS_LAUNCH(32, 128, 1, false)
    QMM_LDS_LAUNCH(64, 128, 1, false)
    QMM_LDS_LAUNCH(32, 256, 1, false)
    QMM_LDS_LAUNCH(32, 128, 2, false)
    QMM_LDS_LAUNCH(32, 256, 2, false)
    QMM_LDS_LAUNCH(32, 128, 1, true)
    QMM_LDS_LAUNCH(32, 128, 2, true)
    }
#undef QMM_LDS_LAUNCH
    if (pl.n_split > 1) launch_splitk_sum(dst, part, n * m, splitk_stride(n, m), pl.n_split, m, ldd, st);
}

template <int QT>
static int per_cu_qt(int wr, int bnt, int kg, bool xf) {
    using namespace lds_ring;
#define QMM_LDS_PER_CU(WR_, BN_, KG_, XF_) \
    if (xf == XF_ && wr == WR_ && bnt == BN_ && kg == KG_) return Geo<QT, WR_, BN_, KG_, XF_>::OK ? Geo<QT, WR_, BN_, KG_, XF_>::PER_CU : 0;
    QMM_LDS_PER_CU(16, 64, 1, false)
    QMM_LDS_PER_CU(16, 64, 2, false)
    QMM_LDS_PER_CU(16, 64, 1, true)
    QMM_LDS_PER_CU(16, 64, 2, true)
    QMM_LDS_PER_CU(16, 128, 1, false)
    QMM_LDS_PER_CU(16, 128, 2, false)
    QMM_LDS_PER_CU(16, 128, 1, true)
    QMM_LDS_PER_CU(16, 128, 2, true)
    QMM_LDS_PER_CU(32, 128, 1, false)
    QMM_LDS_PER_CU(64, 128, 1, false)
    QMM_LDS_PER_CU(32, 256, 1, false)
    QMM_LDS_PER_CU(32, 128, 2, false)
    QMM_LDS_PER_CU(32, 256, 2, false)
    QMM_LDS_PER_CU(64, 256, 1, false)
    QMM_LDS_PER_CU(32, 128, 1, true)
    QMM_LDS_PER_CU(32, 128, 2, true)
#undef QMM_LDS_PER_CU
    return 0;
}

int lds_ring_per_cu(int qt, int tile_rows, int tile_tokens, int kg, bool xf) {
    const int wr = tile_rows / 4;
    switch (qt) {
        case QT_F32: return per_cu_qt<QT_F32>(wr, tile_tokens, kg, xf);
        case QT_Q4_0: return per_cu_qt<QT_Q4_0>(wr, tile_tokens, kg, xf);
        case QT_Q8_0: return per_cu_qt<QT_Q8_0>(wr, tile_tokens, kg, xf);
        case QT_Q4_K: return per_cu_qt<QT_Q4_K>(wr, tile_tokens, kg, xf);
        case QT_Q6_K: return per_cu_qt<QT_Q6_K>(wr, tile_tokens, kg, xf);
        case QT_NVFP4: return per_cu_qt<QT_NVFP4>(wr, tile_tokens, kg, xf);
    }
    return 0;
}

bool lds_ring_fits(int qt, int tile_rows, int tile_tokens, int kg, bool xf) {
    return lds_ring_per_cu(qt, tile_rows, tile_tokens, kg, xf) > 0;
}

void launch_gemm_lds(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n, int qt,
                     int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd, hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_lds_qt<QT_F32>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_0: launch_lds_qt<QT_Q4_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q8_0: launch_lds_qt<QT_Q8_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_K: launch_lds_qt<QT_Q4_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q6_K: launch_lds_qt<QT_Q6_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_NVFP4: launch_lds_qt<QT_NVFP4>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
    }
}

}  // namespace qmm
