// Device helpers shared by the qmm kernels (gfx950 / CDNA4).
//
// Packed weights are read through buffer resource descriptors: every load is
// range-checked by the hardware against the descriptor's byte count, and a
// load past it returns zero instead of faulting.  Blocks of 18, 34 and 210
// bytes start at 2-byte-aligned offsets, so the kernels load the enclosing
// dword-aligned span and shift bytes into place in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum : int { QT_F32 = 0, QT_Q4_0 = 1, QT_Q8_0 = 2, QT_Q4_K = 3, QT_Q6_K = 4, QT_NVFP4 = 5, QT_NVFP4_V2 = 6 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Raw (stride 0) buffer descriptor over [base, base + nbytes).  Word 3 is
// the gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                             0x00020000);
}

__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// An offset no descriptor reaches: every descriptor the kernels build covers
// fewer than 2^31 bytes (checked on the host), so a load at OOB_OFF (plus a
// small immediate) returns zero.  Masking an address this way, instead of
// zeroing the loaded value, keeps the load asynchronous: a select on the
// loaded data would make the wave wait for it right after issuing it.
constexpr uint32_t OOB_OFF = 0x80000000u;

// Load N dwords starting at the dword-aligned offset (off & ~3).
template <int N>
__device__ __forceinline__ void ld_span(rsrc_t r, uint32_t off, uint32_t (&v)[N]) {
    const uint32_t a = off & ~3u;
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        u32x4 t = ld128(r, a + 4 * i);
        v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
    }
    if constexpr (N % 4 >= 2) {
        u32x2 t = ld64(r, a + 4 * (N / 4 * 4));
        v[N / 4 * 4] = t.x;
        v[N / 4 * 4 + 1] = t.y;
    }
    if constexpr (N % 2 == 1) {
        v[N - 1] = ld32(r, a + 4 * (N - 1));
    }
}

// Bytes [sh, sh+4) of the 8-byte little-endian pair (lo, hi), sh in 0..4
// (v_alignbyte_b32 for 0..3; a 64-bit shift of adjacent array elements would
// be turned into an unaligned 64-bit load and push the array to scratch).
__device__ __forceinline__ uint32_t shr64(uint32_t lo, uint32_t hi, uint32_t sh) {
    const uint32_t a = __builtin_amdgcn_alignbyte(hi, lo, sh & 3u);
    return sh >= 4u ? hi : a;
}

__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ _Float16 bits_h(uint32_t bits) {
    return __builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
    f16x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f2h(float a, float b) {
    return pack_h2((_Float16)a, (_Float16)b);
}

// The low / high half of a dword read as f16 and widened to f32 (exact).
// A small integer q in a half's mantissa field, exponent field zero, is the
// subnormal q * 2^-24; a multiply-add with f32 operands on such a half
// compiles to one v_fma_mix_f32 (widening, product and sum rounded once).
__device__ __forceinline__ float f16lo(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p).x; }
__device__ __forceinline__ float f16hi(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p).y; }

__device__ __forceinline__ uint32_t byte_of(uint32_t v, int b) { return (v >> (8 * b)) & 0xFFu; }

// Bytes 1 and 3 of v as the low bytes of two halves (high bytes zero): one
// v_perm_b32 (selector 0x0c gives a zero byte).  With v & 0x00FF00FF for
// bytes 0 and 2, four byte-wide codes become the halves of two dwords.
__device__ __forceinline__ uint32_t odd_bytes(uint32_t v) { return __builtin_amdgcn_perm(0u, v, 0x0c030c01u); }

constexpr float TWO24 = 16777216.0f;

// Four weights D*q - M as two packed f16 pairs (codes 0,1 and 2,3), the
// codes given as f16 halves holding q itself (the subnormal q * 2^-24,
// exact): e = codes 0 and 2, o = codes 1 and 3.  D24 = D * 2^24, so the
// product D24 * (q * 2^-24) is D * q exactly and each weight, one
// v_fma_mix*_f16 reading its half directly, is rounded once to f16.
__device__ __forceinline__ void affine4h(uint32_t e, uint32_t o, float D24, float Mneg, uint32_t& p01,
                                         uint32_t& p23) {
    const f16x2 a = __builtin_bit_cast(f16x2, e), b = __builtin_bit_cast(f16x2, o);
    const f16x2 lo = {(_Float16)__builtin_fmaf(D24, (float)a[0], Mneg), (_Float16)__builtin_fmaf(D24, (float)b[0], Mneg)};
    const f16x2 hi = {(_Float16)__builtin_fmaf(D24, (float)a[1], Mneg), (_Float16)__builtin_fmaf(D24, (float)b[1], Mneg)};
    p01 = __builtin_bit_cast(uint32_t, lo);
    p23 = __builtin_bit_cast(uint32_t, hi);
}

// Byte B of v as f32: v_cvt_f32_ubyte{0..3}, select and convert in one
// instruction.  There is no builtin for it, and the plain expression
// (float)((v >> 8B) & 0xFF) on a nibble-masked v compiles to v_bfe_u32 plus
// v_cvt_f32_ubyte0 (20 more VALU instructions per Q4_K LDS-ring step): the
// masks' known bits turn the byte select into a 4-bit field extract.  The
// result only ever feeds VALU instructions (the f32 or f16 multiply-adds of
// the decoders), never a matrix-core operand, so no MFMA hazard depends on
// the compiler seeing this instruction.
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
    float r;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

__device__ __forceinline__ float ubyte_f32(uint32_t v, int b) {
    switch (b) {
        case 0: return ubyte_f32<0>(v);
        case 1: return ubyte_f32<1>(v);
        case 2: return ubyte_f32<2>(v);
        default: return ubyte_f32<3>(v);
    }
}

// Index of the calling wave in its work group, as a wave-uniform (scalar)
// value: buffer descriptors derived from it stay in SGPRs.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }

// OCP FP8 E4M3FN code in the low byte of b -> f32 (exact; upper bits
// ignored): v_cvt_f32_fp8 with byte select 0.  On gfx950 it decodes OCP
// E4M3FN (sign, 4-bit exponent bias 7, 3-bit mantissa, exponent 0
// subnormal, S.1111.111 NaN, no infinities), checked for all 256 codes.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// Two OCP FP4 E2M1 codes in byte `sel` of v -> f32 (low nibble first), exact.
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t v, int sel) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
    }
}

// E2M1 code (4 bits) -> f16 bit pattern of the code placed so that the f16
// value times 2^14 is the E2M1 value: magnitude bits land in f16 bits 9..11
// (a 2-bit exponent field whose bias differs from binary16's by 14, with
// exponent 0 landing in the binary16 subnormal range), sign in bit 15.
__device__ __forceinline__ uint32_t e2m1_f16_bits_unscaled(uint32_t c) {
    return ((c & 7u) << 9) | ((c & 8u) << 12);
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Descriptor over the packed rows [row0, row0+rows) clipped to m, based at the
// 16-byte boundary at or below the first row (returned in `base`); its byte
// count is rounded up to 16, so a dword-aligned span that ends inside the
// last row's final bytes never has its covering dword range-checked away.
// (Reads past the end of w stay within its last 16-byte granule.)
__device__ __forceinline__ rsrc_t row_window(const uint8_t* w, int64_t row0, int64_t rows,
                                             int64_t m, int64_t rb, int64_t& base) {
    base = (row0 * rb) & ~(int64_t)15;
    const int64_t end = imin64(m, row0 + rows) * rb;
    const int64_t bytes = end > base ? ((end - base + 15) & ~(int64_t)15) : 0;
    return make_rsrc(w + base, (uint32_t)bytes);
}

}  // namespace qmm
