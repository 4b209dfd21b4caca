// Weight-tile loaders shared by the prefill kernels: per format, the packed
// bytes of half a row of a 64-k step are loaded into registers and decoded to
// 32 f16 values (round to nearest even, once) in the step's k order.
//
// k order inside an LDS row.  The contraction is over k, so any permutation
// of the 64 k values of a step gives the same result, provided the weight
// and activation tiles use the same one.  Each format uses the permutation
// under which one thread's 4 packed bytes expand into 8 consecutive LDS
// slots: slot 8s+i holds k = g*2H + 4s' + i (i<4) or g*2H + H + 4s' + i-4
// (i>=4), where s = g*H/4 + s' and H is the distance between the two weights
// that share a packed byte (16 for Q4_0 and NVFP4, 32 for Q4_K, 64 for Q6_K;
// 4, the identity, for F32 and Q8_0).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride in halves (16-byte pad: conflict-free b128 reads)

template <int QT> struct Perm { static constexpr int H = 4; };
template <> struct Perm<QT_Q4_0> { static constexpr int H = 16; };
template <> struct Perm<QT_Q4_K> { static constexpr int H = 32; };
template <> struct Perm<QT_Q6_K> { static constexpr int H = 64; };
template <> struct Perm<QT_NVFP4> { static constexpr int H = 16; };

// f16x2 from two bytes (lo, hi) of v at byte positions b0, b0+1, each given
// as 1024 + byte by the binary16 pattern 0x6400 | byte.
__device__ __forceinline__ f16x2 magic_pair(uint32_t v, int b0) {
    const uint32_t bits = ((v >> (8 * b0)) & 0xFFu) | (((v >> (8 * b0 + 8)) & 0xFFu) << 16) | 0x64006400u;
    return __builtin_bit_cast(f16x2, bits);
}

// ------------------------------------------------------------ weight tiles
// Thread (row, p) covers the 32 slots [32p, 32p+32) of its row's k-step kt.
// decode() fills o[4u..4u+3] with the 8 halves of slot unit u (slot order).

template <int QT> struct ALoad;

template <> struct ALoad<QT_F32> {
    u32x4 r[8];
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int k, int) {
        const int e = kt * 64 + 32 * p;
#pragma unroll
        for (int i = 0; i < 8; ++i)  // runs past k read zeros (out-of-range offset)
            r[i] = ld128(wr, e + 4 * i < k ? row_off + 4u * (uint32_t)(e + 4 * i) : OOB_OFF);
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = __builtin_bit_cast(f32x4, r[i]);
            o[2 * i] = pack_f2h(v.x, v.y);
            o[2 * i + 1] = pack_f2h(v.z, v.w);
        }
    }
};

template <> struct ALoad<QT_Q4_0> {
    uint32_t r[5], sh;
    // a block past k reads zeros (out-of-range offset): d = 0, every weight 0
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int k, int) {
        const int b = 2 * kt + p;
        const uint32_t o = b * 32 < k ? row_off + (uint32_t)b * 18u : OOB_OFF;
        sh = o & 3u;
        ld_span<5>(wr, o, r);
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
        const _Float16 d = bits_h(r[0] >> (8u * sh));
        const f16x2 dd = {d, d}, off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t q = shr64(r[u], r[u + 1], sh + 2u);
            const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
            // (1024 + q) - 1032 = q - 8 exactly; one f16 rounding in the product
            o[4 * u + 0] = __builtin_bit_cast(uint32_t, (magic_pair(lo, 0) - off) * dd);
            o[4 * u + 1] = __builtin_bit_cast(uint32_t, (magic_pair(lo, 2) - off) * dd);
            o[4 * u + 2] = __builtin_bit_cast(uint32_t, (magic_pair(hi, 0) - off) * dd);
            o[4 * u + 3] = __builtin_bit_cast(uint32_t, (magic_pair(hi, 2) - off) * dd);
        }
    }
};

template <> struct ALoad<QT_Q8_0> {
    uint32_t r[9], sh;
    // a block past k reads zeros (out-of-range offset): d = 0, every weight 0
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int k, int) {
        const int b = 2 * kt + p;
        const uint32_t o = b * 32 < k ? row_off + (uint32_t)b * 34u : OOB_OFF;
        sh = o & 3u;
        ld_span<9>(wr, o, r);
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
        const _Float16 d = bits_h(r[0] >> (8u * sh));
        const f16x2 dd = {d, d}, off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // int8 q -> byte q+128 -> 1024 + q + 128 in f16, minus 1152 = q exactly
            const uint32_t qa = shr64(r[2 * u], r[2 * u + 1], sh + 2u) ^ 0x80808080u;
            const uint32_t qb = shr64(r[2 * u + 1], r[2 * u + 2], sh + 2u) ^ 0x80808080u;
            o[4 * u + 0] = __builtin_bit_cast(uint32_t, (magic_pair(qa, 0) - off) * dd);
            o[4 * u + 1] = __builtin_bit_cast(uint32_t, (magic_pair(qa, 2) - off) * dd);
            o[4 * u + 2] = __builtin_bit_cast(uint32_t, (magic_pair(qb, 0) - off) * dd);
            o[4 * u + 3] = __builtin_bit_cast(uint32_t, (magic_pair(qb, 2) - off) * dd);
        }
    }
};

template <> struct ALoad<QT_Q4_K> {
    u32x4 hdr, qs;
    int c;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int, int nk) {
        const uint32_t sb = (uint32_t)kt >> 2;
        c = kt & 3;
        const uint32_t o = kt < nk ? row_off + sb * 144u : OOB_OFF;
        hdr = ld128(wr, o);
        qs = ld128(wr, o + 16u + 32u * (uint32_t)c + 16u * (uint32_t)p);
    }
    __device__ __forceinline__ static uint32_t scb(u32x4 h, int i) {
        const uint32_t v = i < 4 ? h.y : (i < 8 ? h.z : h.w);
        return (v >> (8 * (i & 3))) & 0xFFu;
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        // sub-blocks j0 = 2c, j1 = 2c+1: 6-bit scale and min, unpacked for
        // both halves of the packing and selected (no branch, so the decode
        // stays in the basic block of the matrix-core work it interleaves with)
        const int j0 = 2 * c, j1 = 2 * c + 1;
        const uint32_t b0 = scb(hdr, j0 & 7), b1 = scb(hdr, j1 & 7);            // sc[j]   (j < 4: scale)
        const uint32_t b4 = scb(hdr, j0 + 4), b5 = scb(hdr, j1 + 4);            // sc[j+4]
        const uint32_t bm0 = scb(hdr, (j0 - 4) & 7), bm1 = scb(hdr, (j1 - 4) & 7);  // sc[j-4]
        // all ones for the first half of the packing (c < 2), else zero
        const uint32_t lo = (uint32_t)(-(int)(c < 2));
        auto blend = [lo](uint32_t a, uint32_t b) { return (a & lo) | (b & ~lo); };
        const uint32_t s0 = blend(b0 & 63u, (b4 & 15u) | ((bm0 >> 6) << 4));
        const uint32_t m0 = blend(b4 & 63u, (b4 >> 4) | ((b0 >> 6) << 4));
        const uint32_t s1 = blend(b1 & 63u, (b5 & 15u) | ((bm1 >> 6) << 4));
        const uint32_t m1 = blend(b5 & 63u, (b5 >> 4) | ((b1 >> 6) << 4));
        const float d24 = d * TWO24;
        const float D0 = d24 * (float)s0, M0 = dmin * (float)m0;
        const float D1 = d24 * (float)s1, M1 = dmin * (float)m1;
        // the nibbles as f16 halves: low nibbles of bytes 0, 2 and 1, 3, then
        // the high ones
        constexpr uint32_t N2 = 0x000F000Fu;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t q = u == 0 ? qs.x : (u == 1 ? qs.y : (u == 2 ? qs.z : qs.w));
            affine4h(q & N2, (q >> 8) & N2, D0, -M0, o[4 * u + 0], o[4 * u + 1]);
            affine4h((q >> 4) & N2, (q >> 12) & N2, D1, -M1, o[4 * u + 2], o[4 * u + 3]);
        }
    }
};

// Q6_K step kt: superblock kt/4, half (kt/2)&1, L bytes [32*(kt&1) + 16p, +16)
// of the half's 64 ql bytes, qh bytes [16p, +16) of the half's 32, two scales.
template <> struct ALoad<QT_Q6_K> {
    uint32_t ra[5], rh[5], rs0, rs1, rd, sh;
    int kh;
    uint32_t pos0, pos1;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int, int nk) {
        const uint32_t sb = (uint32_t)kt >> 2;
        const uint32_t hh = ((uint32_t)kt >> 1) & 1u;
        kh = kt & 1;
        const uint32_t o = kt < nk ? row_off + sb * 210u : OOB_OFF;
        sh = o & 3u;
        ld_span<5>(wr, o + 64u * hh + 32u * (uint32_t)kh + 16u * (uint32_t)p, ra);
        ld_span<5>(wr, o + 128u + 32u * hh + 16u * (uint32_t)p, rh);
        const uint32_t i0 = 8u * hh + 2u * (uint32_t)kh + (uint32_t)p;
        const uint32_t a0 = o + 192u + i0, a1 = a0 + 4u;
        pos0 = a0 & 3u;
        pos1 = a1 & 3u;
        rs0 = ld32(wr, a0 & ~3u);
        rs1 = ld32(wr, a1 & ~3u);
        rd = ld32(wr, (o + 208u) & ~3u);
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
        const float d = h2f(rd >> (8u * sh));
        const float Dl = d * (float)(int8_t)(rs0 >> (8u * pos0));
        const float Dh = d * (float)(int8_t)(rs1 >> (8u * pos1));
        const float Dl32 = -32.0f * Dl, Dh32 = -32.0f * Dh;
        const int hs = 2 * kh;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t L = shr64(ra[u], ra[u + 1], sh);
            const uint32_t H = shr64(rh[u], rh[u + 1], sh);
            const uint32_t ql = (L & 0x0F0F0F0Fu) | (((H >> hs) & 0x03030303u) << 4);
            const uint32_t qhv = ((L >> 4) & 0x0F0F0F0Fu) | (((H >> (hs + 4)) & 0x03030303u) << 4);
            // one 6-bit code per byte: even bytes by a mask, odd ones by a permute
            affine4h(ql & 0x00FF00FFu, odd_bytes(ql), Dl * TWO24, Dl32, o[4 * u + 0], o[4 * u + 1]);
            affine4h(qhv & 0x00FF00FFu, odd_bytes(qhv), Dh * TWO24, Dh32, o[4 * u + 2], o[4 * u + 3]);
        }
    }
};

template <> struct ALoad<QT_NVFP4> {
    uint32_t sd;
    u32x4 qs;
    int p_;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int, int nk) {
        const uint32_t o = kt < nk ? row_off + (uint32_t)kt * 36u : OOB_OFF;
        p_ = p;
        sd = ld32(wr, o);
        qs = ld128(wr, o + 4u + 16u * (uint32_t)p);
    }
    __device__ __forceinline__ void decode(uint32_t (&o)[16]) const {
        const float sl = e4m3_to_f32((sd >> (16 * p_)) & 0xFFu);
        const float sh_ = e4m3_to_f32((sd >> (16 * p_ + 8)) & 0xFFu);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t q = u == 0 ? qs.x : (u == 1 ? qs.y : (u == 2 ? qs.z : qs.w));
            float lo[4], hi[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const f32x2 v = e2m1x2_to_f32(q, b);
                lo[b] = v.x * sl;   // exact: at most 5 significant bits, within f16 range
                hi[b] = v.y * sh_;
            }
            o[4 * u + 0] = pack_f2h(lo[0], lo[1]);
            o[4 * u + 1] = pack_f2h(lo[2], lo[3]);
            o[4 * u + 2] = pack_f2h(hi[0], hi[1]);
            o[4 * u + 3] = pack_f2h(hi[2], hi[3]);
        }
    }
};

// Scheduling hint for one half-iteration of the k loop (one basic block):
// the global loads two steps ahead, then all 16 LDS reads of the step's
// fragments (so the matrix-core ops wait on LDS latency once, not once per
// read), then each of the 32 matrix-core ops followed by a slice of the
// other buffer's decode (VALU), so the decode runs while the matrix cores
// work instead of after them.
__device__ __forceinline__ void interleave_hint() {
    __builtin_amdgcn_sched_group_barrier(0x020, 20, 0);  // VMEM read
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // DS read
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
    }
}

}  // namespace qmm
