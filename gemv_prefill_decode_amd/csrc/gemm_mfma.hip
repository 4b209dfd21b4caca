// Prefill path: dequant-fused GEMM on the gfx950 matrix cores.
//
// One work group (256 threads, 4 waves in a 2x2 grid) computes a 128 x 128
// tile of dst (128 weight rows x 128 tokens) over k in steps of 64.  Per step
// every thread loads the packed bytes of half a row of the weight tile and
// half a row of the activation tile into registers, decodes the weights to
// f16 (round to nearest even, once) and rounds the activations to f16, and
// stores both into LDS.  The waves then run v_mfma_f32_16x16x32_f16 on 64 x 64
// sub-tiles with f32 accumulators.  LDS is double buffered and the next
// step's global loads are issued before the current step's MFMAs, so the
// loads, the decode and the matrix-core work overlap.
//
// k order inside an LDS row.  The contraction is over k, so any permutation
// of the 64 k values of a step gives the same result, provided the weight
// and activation tiles use the same one.  Each format uses the permutation
// under which one thread's 4 packed bytes expand into 8 consecutive LDS
// slots: slot 8s+i holds k = g*2H + 4s' + i (i<4) or g*2H + H + 4s' + i-4
// (i>=4), where s = g*H/4 + s' and H is the distance between the two weights
// that share a packed byte (16 for Q4_0 and NVFP4, 32 for Q4_K, 64 for Q6_K;
// 4, the identity, for F32 and Q8_0).
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

constexpr int BM = MFMA_BM, BN = MFMA_BN, BK = 64;
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
    bool valid;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int k, int) {
        const int b = 2 * kt + p;
        const uint32_t o = b * 32 < k ? row_off + (uint32_t)b * 18u : OOB_OFF;
        sh = o & 3u;
        valid = b * 32 < k;
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
        if (!valid)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = 0u;
    }
};

template <> struct ALoad<QT_Q8_0> {
    uint32_t r[9], sh;
    bool valid;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int kt, int p, int k, int) {
        const int b = 2 * kt + p;
        const uint32_t o = b * 32 < k ? row_off + (uint32_t)b * 34u : OOB_OFF;
        sh = o & 3u;
        valid = b * 32 < k;
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
        if (!valid)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = 0u;
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
        uint32_t s0, m0, s1, m1;
        if (c < 2) {
            s0 = scb(hdr, 2 * c) & 63u;     m0 = scb(hdr, 2 * c + 4) & 63u;
            s1 = scb(hdr, 2 * c + 1) & 63u; m1 = scb(hdr, 2 * c + 5) & 63u;
        } else {
            const int j0 = 2 * c, j1 = 2 * c + 1;
            s0 = (scb(hdr, j0 + 4) & 15u) | ((scb(hdr, j0 - 4) >> 6) << 4);
            m0 = (scb(hdr, j0 + 4) >> 4) | ((scb(hdr, j0) >> 6) << 4);
            s1 = (scb(hdr, j1 + 4) & 15u) | ((scb(hdr, j1 - 4) >> 6) << 4);
            m1 = (scb(hdr, j1 + 4) >> 4) | ((scb(hdr, j1) >> 6) << 4);
        }
        const float D0 = d * (float)s0, M0 = dmin * (float)m0;
        const float D1 = d * (float)s1, M1 = dmin * (float)m1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t q = u == 0 ? qs.x : (u == 1 ? qs.y : (u == 2 ? qs.z : qs.w));
            float lo[4], hi[4];
            const uint32_t ql = q & 0x0F0F0F0Fu, qh = (q >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                lo[b] = __builtin_fmaf(D0, ubyte_f32(ql, b), -M0);
                hi[b] = __builtin_fmaf(D1, ubyte_f32(qh, b), -M1);
            }
            o[4 * u + 0] = pack_f2h(lo[0], lo[1]);
            o[4 * u + 1] = pack_f2h(lo[2], lo[3]);
            o[4 * u + 2] = pack_f2h(hi[0], hi[1]);
            o[4 * u + 3] = pack_f2h(hi[2], hi[3]);
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
            float lo[4], hi[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                lo[b] = __builtin_fmaf(Dl, ubyte_f32(ql, b), Dl32);
                hi[b] = __builtin_fmaf(Dh, ubyte_f32(qhv, b), Dh32);
            }
            o[4 * u + 0] = pack_f2h(lo[0], lo[1]);
            o[4 * u + 1] = pack_f2h(lo[2], lo[3]);
            o[4 * u + 2] = pack_f2h(hi[0], hi[1]);
            o[4 * u + 3] = pack_f2h(hi[2], hi[3]);
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

// ------------------------------------------------------------ activation tiles
// Thread t loads 16 bytes (a run of 4 consecutive k) of token row
// 16*i + t/16 (i = 0..7): lane chunk c = t % 16 is run c & 1 of slot unit
// c / 2 of the step, i.e. k = g*2H + 4s' + (c & 1)*H for the step's global
// slot unit U = 8*kt + c/2, g = U / (H/4), s' = U % (H/4).  The 16 lanes of a
// token together read whole 128-byte segments of its row.  Each run is
// rounded to f16 and stored at slots 8*(c/2) + 4*(c&1) .. +3.
struct XLoad {
    u32x4 r[8];
    // k: row length (stride); kend: loads at k positions >= kend read zeros
    template <int H>
    __device__ __forceinline__ void load(rsrc_t xr, int k, int kend, int kt, int tid) {
        const int c = tid & 15, row = tid >> 4;
        const int U = 8 * kt + (c >> 1);
        const int g = U / (H / 4), sp = U % (H / 4);
        const int e = g * 2 * H + 4 * sp + (c & 1) * H;
        const uint32_t off = 4u * ((uint32_t)row * (uint32_t)k + (uint32_t)e);
        const bool in = e < kend;  // past k lies the next token's row: read zeros instead
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = ld128(xr, in ? off + 4u * 16u * (uint32_t)i * (uint32_t)k : OOB_OFF);
    }
    __device__ __forceinline__ void store(_Float16* sB, int tid) const {
        const int c = tid & 15, row = tid >> 4;
        const int slot = 8 * (c >> 1) + 4 * (c & 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 v = __builtin_bit_cast(f32x4, r[i]);
            *(u32x2*)&sB[(16 * i + row) * LDK + slot] = u32x2{pack_f2h(v.x, v.y), pack_f2h(v.z, v.w)};
        }
    }
};

// ------------------------------------------------------------ kernel

// Split k (n_split > 1): work item (z, tile) covers the k steps
// [z*sps, min(nk, (z+1)*sps)) of one tile (sps even) and writes its partial
// tile to partial + z*splitk_stride(n, m) in dst's layout.  splitk_sum_kernel
// then adds the n_split partials in the order z = 0, 1, ... into dst; it is a
// second launch on the same stream, so the partials are visible to it without
// any fence, and the sum does not depend on the order the work items ran in.
template <int QT>
__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(float* __restrict__ dst,
                                                           const uint8_t* __restrict__ w,
                                                           const float* __restrict__ x, int m,
                                                           int k, int n, int rb, int n_mb,
                                                           int n_nb, int n_split, int sps,
                                                           float* __restrict__ partial) {
    __shared__ __attribute__((aligned(16))) _Float16 sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) _Float16 sB[2][BN * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Work groups are dealt round-robin to the 8 XCDs (id % 8); give each XCD
    // a contiguous run of work items so the tiles that share weight rows (and
    // the same k range) share an L2.
    const int T = n_mb * n_nb, NI = T * n_split, L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3, per = NI >> 3, rem = NI & 7;
    const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int z = item / T, tile = item - z * T;
    const int mb = tile / n_nb, nb = tile - mb * n_nb;
    const int64_t m0 = (int64_t)mb * BM, n0 = (int64_t)nb * BN;

    int64_t base;
    const rsrc_t wr = row_window(w, m0, BM, m, rb, base);
    const int ntok = (int)imin64(BN, n - n0);
    const rsrc_t xr = make_rsrc(x + n0 * k, (uint32_t)ntok * (uint32_t)k * 4u);
    const int arow = tid >> 1, part = tid & 1;
    const uint32_t roff = (uint32_t)((m0 + arow) * rb - base);
    const int nk_all = (k + BK - 1) / BK;
    const int s0 = z * sps;
    const int nk = min(nk_all, s0 + sps);     // steps at or past nk read zeros
    const int kend = min(k, nk * BK);         // so do k positions at or past kend
    const int lds_a = arow * LDK + part * 32;
    constexpr int H = Perm<QT>::H;

    // Two register sets of raw step data: while the matrix cores work on step
    // kt, the loads of step kt+2 are in flight and step kt+1 is decoded.
    ALoad<QT> al0, al1;
    XLoad xl0, xl1;
    uint32_t tmp[16];
    auto stage = [&](const ALoad<QT>& al, const XLoad& xl, int buf) {
        al.decode(tmp);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *(u32x4*)&sA[buf][lds_a + 8 * u] = u32x4{tmp[4 * u], tmp[4 * u + 1], tmp[4 * u + 2], tmp[4 * u + 3]};
        xl.store(sB[buf], tid);
    };

    // Every load is unconditional (steps at or past nk read zeros through
    // out-of-range offsets, and their staged tiles are never used), so the
    // loop body is straight-line and the compiler's load counters let the
    // loads of step kt+2 stay in flight while step kt computes.
    al0.load(wr, roff, s0, part, kend, nk);
    xl0.template load<H>(xr, k, kend, s0, tid);
    al1.load(wr, roff, s0 + 1, part, kend, nk);
    xl1.template load<H>(xr, k, kend, s0 + 1, tid);
    stage(al0, xl0, 0);
    __syncthreads();

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave >> 1, wn = wave & 1;
    const int frag = (lane & 15) * LDK + (lane >> 4) * 8;
    auto mfma_step = [&](int buf) {
        const _Float16* A = &sA[buf][wm * 64 * LDK + frag];
        const _Float16* B = &sB[buf][wn * 64 * LDK + frag];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = *(const f16x8*)(A + i * 16 * LDK + ks * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = *(const f16x8*)(B + j * 16 * LDK + ks * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // An odd step count runs one extra step whose weight and activation tiles
    // are all zeros (out-of-range loads): it adds exactly 0 to every sum and
    // keeps a single loop exit, so the accumulators stay in place.
    const int nk2 = s0 + ((nk - s0 + 1) & ~1);
    for (int kt = s0; kt < nk2; kt += 2) {
        // step kt: buffer 0; set 1 holds step kt+1, set 0 takes kt+2
        al0.load(wr, roff, kt + 2, part, kend, nk);
        xl0.template load<H>(xr, k, kend, kt + 2, tid);
        mfma_step(0);
        stage(al1, xl1, 1);
        __syncthreads();
        // step kt+1: buffer 1; set 0 holds step kt+2, set 1 takes kt+3
        al1.load(wr, roff, kt + 3, part, kend, nk);
        xl1.template load<H>(xr, k, kend, kt + 3, tid);
        mfma_step(1);
        stage(al0, xl0, 0);
        __syncthreads();
    }


    // D[row][col] of a 16x16 tile sits in lane (row/4)*16 + col, element row%4:
    // rows are weight rows (contiguous in dst), cols are tokens.
    float* out = n_split > 1 ? partial + (int64_t)z * splitk_stride(n, m) : dst;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t mrow = m0 + wm * 64 + i * 16 + (lane >> 4) * 4;
            const int64_t tok = n0 + wn * 64 + j * 16 + (lane & 15);
            if (tok < n) {
                float* p = out + tok * m + mrow;
                const f32x4 v = acc[i][j];
                if ((m & 3) == 0 && mrow + 4 <= m) {
                    *(f32x4*)p = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (mrow + r < m) p[r] = v[r];
                }
            }
        }
    }
}

// dst[i] = part[0][i] + part[1][i] + ... + part[n_split-1][i], in that
// order, for i < count; part[z] starts at z * splitk_stride (16-byte aligned).
__global__ __launch_bounds__(256) void splitk_sum_kernel(float* __restrict__ dst,
                                                         const float* __restrict__ part,
                                                         int64_t count, int64_t zstride, int n_split) {
    const int64_t n4 = count >> 2;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        f32x4 v = reinterpret_cast<const f32x4*>(part)[i];
        for (int z = 1; z < n_split; ++z) v += reinterpret_cast<const f32x4*>(part + z * zstride)[i];
        reinterpret_cast<f32x4*>(dst)[i] = v;
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
        float v = part[i];
        for (int z = 1; z < n_split; ++z) v += part[z * zstride + i];
        dst[i] = v;
    }
}

template <int QT>
static void launch_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int64_t rb, const MfmaPlan& pl, void* ws, hipStream_t st) {
    const int n_mb = (int)((m + BM - 1) / BM), n_nb = (int)((n + BN - 1) / BN);
    gemm_mfma_kernel<QT><<<dim3((unsigned)(n_mb * n_nb * pl.n_split)), 256, 0, st>>>(
        dst, w, x, (int)m, (int)k, (int)n, (int)rb, n_mb, n_nb, pl.n_split, pl.sps, (float*)ws);
    if (pl.n_split > 1) {
        const int64_t count = n * m;
        int64_t blocks = (count / 4 + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        if (blocks < 1) blocks = 1;
        splitk_sum_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(dst, (const float*)ws, count,
                                                                 splitk_stride(n, m), pl.n_split);
    }
}

MfmaPlan plan_gemm_mfma(int64_t m, int64_t k, int64_t n, int num_cu) {
    MfmaPlan best;
    const int64_t T = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    const int nk = (int)((k + BK - 1) / BK);
    best.n_split = 1;
    best.sps = nk + (nk & 1);
    best.ws_bytes = 0;
    if (T >= num_cu || nk < 4) return best;
    // Estimated time in k steps of one work group: (rounds of work groups
    // over the CUs) x (steps per item), plus for a split the second launch
    // and the partials' traffic (written once, read once; dst written once).
    constexpr double STEP_US = 1.3, LAUNCH_US = 2.0, BYTES_PER_US = 4.0e6;
    const double out_bytes = 4.0 * (double)n * (double)m;
    double best_cost = 1e30;
    for (int S = 1; S <= 16 && S <= nk / 2; ++S) {
        const int sps = ((nk + S - 1) / S + 1) & ~1;
        const int se = (nk + sps - 1) / sps;
        if (S > 1 && se < 2) continue;
        const int64_t rounds = (T * se + num_cu - 1) / num_cu;
        const double extra = se > 1 ? (LAUNCH_US + (2.0 * se + 1.0) * out_bytes / BYTES_PER_US) / STEP_US : 0.0;
        const double cost = (double)rounds * sps + extra;
        if (cost < best_cost) {
            best_cost = cost;
            best.n_split = se;
            best.sps = sps;
        }
    }
    if (best.n_split > 1)
        best.ws_bytes = (int64_t)best.n_split * splitk_stride(n, m) * 4;
    else
        best.sps = nk + (nk & 1);
    return best;
}

void launch_gemm_mfma(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int qt, int64_t rb, const MfmaPlan& pl, void* ws, hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_qt<QT_F32>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
        case QT_Q4_0: launch_qt<QT_Q4_0>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
        case QT_Q8_0: launch_qt<QT_Q8_0>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
        case QT_Q4_K: launch_qt<QT_Q4_K>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
        case QT_Q6_K: launch_qt<QT_Q6_K>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
        case QT_NVFP4: launch_qt<QT_NVFP4>(dst, wb, x, m, k, n, rb, pl, ws, st); break;
    }
}

}  // namespace qmm
