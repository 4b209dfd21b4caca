// Decode path: f32 GEMV for small n, the MoE gate/up projections, and the
// load-only twin.  No matrix cores: the weights stream from HBM once, each
// lane decodes its blocks to f32 in registers and accumulates with f32 FMA;
// lanes that share a row reduce with cross-lane shuffles.
//
// Work split.  A row of k weights is cut into "units" (16..64 weights each,
// per format).  The LPR lanes of a lane group take units gl, gl+LPR, ... of
// the same R rows, so one wave load instruction reads LPR consecutive units
// of a row (coalesced), and the activations a lane loads for its units are
// reused for all R rows.  Each unit's products are summed in a fresh partial
// (at most 64 terms) before joining the lane's running sum, and the LPR lane
// partials are combined by a butterfly, which keeps every f32 rounding chain
// short (64 + k/(UE*LPR) + log2(LPR) terms).
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

// ------------------------------------------------------------------ units
// load(): fetch one unit of one row (row_off = byte offset of the row inside
// the weight descriptor).  prep(): per-unit scales.  sub(s): weights of
// sub-unit s (8 weights) plus the k indices e0, e1 of the two runs of 4
// consecutive weights they are (w[0..3] <-> k e0..e0+3, w[4..7] <-> e1..e1+3).

template <int QT> struct GUnit;

template <> struct GUnit<QT_F32> {  // 16 weights, 64 bytes
    static constexpr int UE = 16, S = 2;
    uint32_t r[16];
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int k) {
        ld_span<16>(wr, row_off + (uint32_t)u * 64u, r);
#pragma unroll
        for (int i = 0; i < 4; ++i)  // k % 4 == 0: a run of 4 is wholly in or out
            if (u * 16 + 4 * i >= k) r[4 * i] = r[4 * i + 1] = r[4 * i + 2] = r[4 * i + 3] = 0u;
    }
    __device__ __forceinline__ void prep() {}
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = __builtin_bit_cast(float, r[8 * s + i]);
        e0 = u * 16 + 8 * s;
        e1 = e0 + 4;
    }
};

template <> struct GUnit<QT_Q4_0> {  // one 18-byte block of 32 weights
    static constexpr int UE = 32, S = 4;
    uint32_t r[5], sh;
    float d, d8;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int) {
        const uint32_t o = row_off + (uint32_t)u * 18u;
        sh = o & 3u;
        ld_span<5>(wr, o, r);
    }
    __device__ __forceinline__ void prep() {
        d = h2f(r[0] >> (8u * sh));
        d8 = -8.0f * d;
    }
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
        const uint32_t q = shr64(r[s], r[s + 1], sh + 2u);  // qs[4s..4s+3]
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = __builtin_fmaf(d, (float)((q >> (8 * b)) & 15u), d8);
            w[4 + b] = __builtin_fmaf(d, (float)((q >> (8 * b + 4)) & 15u), d8);
        }
        e0 = u * 32 + 4 * s;
        e1 = e0 + 16;
    }
};

template <> struct GUnit<QT_Q8_0> {  // one 34-byte block of 32 weights
    static constexpr int UE = 32, S = 4;
    uint32_t r[9], sh;
    float d;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int) {
        const uint32_t o = row_off + (uint32_t)u * 34u;
        sh = o & 3u;
        ld_span<9>(wr, o, r);
    }
    __device__ __forceinline__ void prep() { d = h2f(r[0] >> (8u * sh)); }
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
        const uint32_t qa = shr64(r[2 * s], r[2 * s + 1], sh + 2u);
        const uint32_t qb = shr64(r[2 * s + 1], r[2 * s + 2], sh + 2u);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = d * (float)(int8_t)(qa >> (8 * b));
            w[4 + b] = d * (float)(int8_t)(qb >> (8 * b));
        }
        e0 = u * 32 + 8 * s;
        e1 = e0 + 4;
    }
};

// Q4_K: 16 bytes of nibbles (32 weights) of one 144-byte superblock, plus the
// superblock's 16-byte header (d, dmin, 12 bytes of 6-bit scales/mins).
template <> struct GUnit<QT_Q4_K> {
    static constexpr int UE = 32, S = 4;
    u32x4 hdr, qs;
    float D0, M0, D1, M1;
    int c8;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int) {
        const uint32_t sb = (uint32_t)u >> 3;
        c8 = u & 7;
        const uint32_t o = row_off + sb * 144u;
        hdr = ld128(wr, o);
        qs = ld128(wr, o + 16u + 16u * (uint32_t)c8);
    }
    __device__ __forceinline__ static uint32_t scb(u32x4 h, int i) {  // scale byte i (0..11)
        const uint32_t v = i < 4 ? h.y : (i < 8 ? h.z : h.w);
        return (v >> (8 * (i & 3))) & 0xFFu;
    }
    __device__ __forceinline__ void prep() {
        const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
        const int c = c8 >> 1;
        uint32_t s0, m0, s1, m1;
        if (c < 2) {  // pairs j = 2c, 2c+1 < 4
            s0 = scb(hdr, 2 * c) & 63u;     m0 = scb(hdr, 2 * c + 4) & 63u;
            s1 = scb(hdr, 2 * c + 1) & 63u; m1 = scb(hdr, 2 * c + 5) & 63u;
        } else {      // j >= 4: low 4 bits in sc[j+4], high 2 bits in sc[j-4] / sc[j]
            const int j0 = 2 * c, j1 = 2 * c + 1;
            s0 = (scb(hdr, j0 + 4) & 15u) | ((scb(hdr, j0 - 4) >> 6) << 4);
            m0 = (scb(hdr, j0 + 4) >> 4) | ((scb(hdr, j0) >> 6) << 4);
            s1 = (scb(hdr, j1 + 4) & 15u) | ((scb(hdr, j1 - 4) >> 6) << 4);
            m1 = (scb(hdr, j1 + 4) >> 4) | ((scb(hdr, j1) >> 6) << 4);
        }
        D0 = d * (float)s0; M0 = dmin * (float)m0;
        D1 = d * (float)s1; M1 = dmin * (float)m1;
    }
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
        const uint32_t q = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = __builtin_fmaf(D0, (float)((q >> (8 * b)) & 15u), -M0);
            w[4 + b] = __builtin_fmaf(D1, (float)((q >> (8 * b + 4)) & 15u), -M1);
        }
        const int sb = u >> 3, c = c8 >> 1, hh = c8 & 1;
        e0 = sb * 256 + 64 * c + 16 * hh + 4 * s;
        e1 = e0 + 32;
    }
};

// Q6_K: 64 weights of one 210-byte superblock: half h, l in [l0, l0+16) of
// the four quarters.  Needs 16 bytes of ql for quarters 0/2, 16 for 1/3, 16
// bytes of qh, the half's 8 scale bytes and d.
template <> struct GUnit<QT_Q6_K> {
    static constexpr int UE = 64, S = 8;
    uint32_t ra[5], rb[5], rh[5], rs[3], rd, sh;
    int h, l0;
    float D[4];
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int) {
        const uint32_t sb = (uint32_t)u >> 2;
        h = (u >> 1) & 1;
        l0 = 16 * (u & 1);
        const uint32_t o = row_off + sb * 210u;
        sh = o & 3u;
        ld_span<5>(wr, o + 64u * h + l0, ra);
        ld_span<5>(wr, o + 64u * h + 32u + l0, rb);
        ld_span<5>(wr, o + 128u + 32u * h + l0, rh);
        ld_span<3>(wr, o + 192u + 8u * h, rs);
        rd = ld32(wr, (o + 208u) & ~3u);
    }
    __device__ __forceinline__ void prep() {
        const float d = h2f(rd >> (8u * sh));
        const uint32_t sc0 = shr64(rs[0], rs[1], sh), sc1 = shr64(rs[1], rs[2], sh);
        const int add = l0 >> 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int i = 2 * g + add;  // scale byte index within the half
            const uint32_t v = i < 4 ? sc0 : sc1;
            D[g] = d * (float)(int8_t)(v >> (8 * (i & 3)));
        }
    }
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
        const int g = s >> 1, i8 = s & 1;
        const uint32_t L0 = (g & 1) ? rb[2 * i8] : ra[2 * i8];
        const uint32_t L1 = (g & 1) ? rb[2 * i8 + 1] : ra[2 * i8 + 1];
        const uint32_t L2 = (g & 1) ? rb[2 * i8 + 2] : ra[2 * i8 + 2];
        const uint32_t l_a = shr64(L0, L1, sh);
        const uint32_t l_b = shr64(L1, L2, sh);
        const uint32_t h_a = shr64(rh[2 * i8], rh[2 * i8 + 1], sh);
        const uint32_t h_b = shr64(rh[2 * i8 + 1], rh[2 * i8 + 2], sh);
        const int nsh = g >= 2 ? 4 : 0;
        const uint32_t qa = ((l_a >> nsh) & 0x0F0F0F0Fu) | (((h_a >> (2 * g)) & 0x03030303u) << 4);
        const uint32_t qb = ((l_b >> nsh) & 0x0F0F0F0Fu) | (((h_b >> (2 * g)) & 0x03030303u) << 4);
        const float Dg = D[g], D32 = -32.0f * D[g];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            w[b] = __builtin_fmaf(Dg, (float)((qa >> (8 * b)) & 0xFFu), D32);
            w[4 + b] = __builtin_fmaf(Dg, (float)((qb >> (8 * b)) & 0xFFu), D32);
        }
        const int sb = u >> 2;
        e0 = sb * 256 + 128 * h + 32 * g + l0 + 8 * i8;
        e1 = e0 + 4;
    }
};

// NVFP4: one half (32 weights) of a 36-byte group: the group's scale dword
// and 16 bytes of E2M1 nibbles.
template <> struct GUnit<QT_NVFP4> {
    static constexpr int UE = 32, S = 4;
    uint32_t sd;
    u32x4 qs;
    int h;
    float s_lo, s_hi;
    __device__ __forceinline__ void load(rsrc_t wr, uint32_t row_off, int u, int) {
        const uint32_t gi = (uint32_t)u >> 1;
        h = u & 1;
        const uint32_t o = row_off + gi * 36u;
        sd = ld32(wr, o);
        qs = ld128(wr, o + 4u + 16u * (uint32_t)h);
    }
    __device__ __forceinline__ void prep() {
        s_lo = e4m3_to_f32((sd >> (16 * h)) & 0xFFu);
        s_hi = e4m3_to_f32((sd >> (16 * h + 8)) & 0xFFu);
    }
    __device__ __forceinline__ void sub(int s, int u, float (&w)[8], int& e0, int& e1) const {
        const uint32_t q = s == 0 ? qs.x : (s == 1 ? qs.y : (s == 2 ? qs.z : qs.w));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x2 v = e2m1x2_to_f32(q, b);
            w[b] = v.x * s_lo;
            w[4 + b] = v.y * s_hi;
        }
        const int gi = u >> 1;
        e0 = gi * 64 + 32 * h + 4 * s;
        e1 = e0 + 16;
    }
};

// ------------------------------------------------------------------ core

template <int QT>
__device__ __host__ constexpr int UT_elems() { return GUnit<QT>::UE; }

template <int QT, int NT, int R>
__device__ __forceinline__ void gemv_rows(rsrc_t wr, const uint32_t (&roff)[R], rsrc_t xr,
                                          const uint32_t (&xoff)[NT], int k, int gl,
                                          int lpr, float (&acc)[R][NT]) {
    const int n_units = (k + UT_elems<QT>() - 1) / UT_elems<QT>();
    using UT = GUnit<QT>;
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[rr][j] = 0.0f;

    for (int u = gl; u < n_units; u += lpr) {
        UT un[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) un[rr].load(wr, roff[rr], u, k);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) un[rr].prep();
        float part[R][NT];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NT; ++j) part[rr][j] = 0.0f;
#pragma unroll
        for (int s = 0; s < UT::S; ++s) {
            float wv[R][8];
            int e0 = 0, e1 = 0;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) un[rr].sub(s, u, wv[rr], e0, e1);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f32x4 xa = __builtin_bit_cast(f32x4, ld128(xr, xoff[j] + 4u * (uint32_t)e0));
                f32x4 xb = __builtin_bit_cast(f32x4, ld128(xr, xoff[j] + 4u * (uint32_t)e1));
                if constexpr (QT == QT_F32) {  // runs past k belong to the next row
                    if (e0 >= k) xa = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (e1 >= k) xb = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    float p = part[rr][j];
                    p = __builtin_fmaf(wv[rr][0], xa.x, p);
                    p = __builtin_fmaf(wv[rr][1], xa.y, p);
                    p = __builtin_fmaf(wv[rr][2], xa.z, p);
                    p = __builtin_fmaf(wv[rr][3], xa.w, p);
                    p = __builtin_fmaf(wv[rr][4], xb.x, p);
                    p = __builtin_fmaf(wv[rr][5], xb.y, p);
                    p = __builtin_fmaf(wv[rr][6], xb.z, p);
                    p = __builtin_fmaf(wv[rr][7], xb.w, p);
                    part[rr][j] = p;
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[rr][j] += part[rr][j];
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[rr][j] += __shfl_xor(acc[rr][j], off, 64);
    }
}

// grid: x = row blocks of 4 * (64/LPR) * R rows, y = token groups of NT.
template <int QT, int NT, int R>
__global__ __launch_bounds__(256) void gemv_kernel(float* __restrict__ dst,
                                                   const uint8_t* __restrict__ w,
                                                   const float* __restrict__ x, int m, int k,
                                                   int n, int rb, int lpr_log2) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = 1 << lpr_log2;
    const int gl = lane & (lpr - 1), slot = lane >> lpr_log2;
    const int rows_per_wave = (64 >> lpr_log2) * R;
    const int64_t row0 = (int64_t)blockIdx.x * 4 * rows_per_wave;
    int64_t base;
    const rsrc_t wr = row_window(w, row0, 4 * rows_per_wave, m, rb, base);
    const int tok0 = blockIdx.y * NT;
    const int ntok = min(NT, n - tok0);
    const rsrc_t xr = make_rsrc(x + (int64_t)tok0 * k, (uint32_t)ntok * (uint32_t)k * 4u);
    const int64_t myrow0 = row0 + wave * rows_per_wave + slot * R;
    uint32_t roff[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) roff[rr] = (uint32_t)((myrow0 + rr) * rb - base);
    uint32_t xoff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) xoff[j] = (uint32_t)j * (uint32_t)k * 4u;

    float acc[R][NT];
    gemv_rows<QT, NT, R>(wr, roff, xr, xoff, k, gl, lpr, acc);
    if (gl == 0) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int64_t row = myrow0 + rr;
            if (row < m) {
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < ntok) dst[(int64_t)(tok0 + j) * m + row] = acc[rr][j];
            }
        }
    }
}

// ------------------------------------------------------------------ MoE gate/up
// grid: x = row blocks of one expert's n_ff rows, y = pair p, z = plane.
// The work group of the FIRST pair that routes to expert e gathers every pair
// routed to e and applies e's rows to all their tokens, so each selected
// expert's rows are read once per call; work groups of later pairs of the same
// expert exit at once.  The decision uses only expert_ids, so it is the same
// in every work group.
constexpr int MOE_MAXP = 64;  // pairs gathered per chunk (more are looped)

template <int QT, int NT, int R>
__device__ void moe_tokens(float* __restrict__ out, const float* __restrict__ scale, rsrc_t wr,
                           const uint32_t (&roff)[R], rsrc_t xr, const int* plist,
                           const int* tlist, int cnt, int in_f, int n_ff, int gl,
                           int lpr, int64_t myrow0) {
    for (int c0 = 0; c0 < cnt; c0 += NT) {
        uint32_t xoff[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j)
            xoff[j] = (uint32_t)tlist[(c0 + j < cnt) ? c0 + j : c0] * (uint32_t)in_f * 4u;
        float acc[R][NT];
        gemv_rows<QT, NT, R>(wr, roff, xr, xoff, in_f, gl, lpr, acc);
        if (gl == 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (c0 + j < cnt) {
                    const int p = plist[c0 + j];
                    const float f = scale[p];
#pragma unroll
                    for (int rr = 0; rr < R; ++rr) {
                        const int64_t row = myrow0 + rr;
                        if (row < n_ff) out[(int64_t)p * n_ff + row] = f * acc[rr][j];
                    }
                }
            }
        }
    }
}

template <int QT, int R>
__global__ __launch_bounds__(256) void moe_gateup_kernel(
    float* __restrict__ gate_out, float* __restrict__ up_out, const uint8_t* __restrict__ w_gate,
    const uint8_t* __restrict__ w_up, const int* __restrict__ ids, const float* __restrict__ pscale,
    const float* __restrict__ x, int t, int n_used, int n_expert, int in_f, int n_ff, int rb,
    int lpr_log2) {
    __shared__ int plist[MOE_MAXP];
    __shared__ int tlist[MOE_MAXP];
    __shared__ int s_cnt, s_first;
    const int n_pairs = t * n_used;
    const int p = blockIdx.y, plane = blockIdx.z;
    const int e = ids[p];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = 1 << lpr_log2;
    const int gl = lane & (lpr - 1), slot = lane >> lpr_log2;
    const int rows_per_wave = (64 >> lpr_log2) * R;
    const int64_t row0 = (int64_t)blockIdx.x * 4 * rows_per_wave;
    const int64_t myrow0 = row0 + wave * rows_per_wave + slot * R;
    float* out = plane == 0 ? gate_out : up_out;
    const float* scale = pscale + (int64_t)plane * n_pairs;

    if (threadIdx.x == 0) {
        int first = 1;
        for (int q = 0; q < p; ++q)
            if (ids[q] == e) { first = 0; break; }
        s_first = first;
    }
    __syncthreads();
    if (!s_first) return;

    if (e < 0 || e >= n_expert) {  // invalid id: poison every pair that carries it
        for (int q = p; q < n_pairs; ++q) {
            if (ids[q] != e) continue;
            for (int64_t r = myrow0; r < myrow0 + R; ++r)
                if (gl == 0 && r < n_ff && r < row0 + 4 * rows_per_wave)
                    out[(int64_t)q * n_ff + r] = __builtin_nanf("");
        }
        return;
    }

    const uint8_t* wp = (plane == 0 ? w_gate : w_up) + (int64_t)e * n_ff * rb;
    int64_t base;
    const rsrc_t wr = row_window(wp, row0, 4 * rows_per_wave, n_ff, rb, base);
    const rsrc_t xr = make_rsrc(x, (uint32_t)t * (uint32_t)in_f * 4u);
    uint32_t roff[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) roff[rr] = (uint32_t)((myrow0 + rr) * rb - base);
    for (int q0 = p; q0 < n_pairs;) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int cnt = 0, q = q0;
            for (; q < n_pairs && cnt < MOE_MAXP; ++q)
                if (ids[q] == e) { plist[cnt] = q; tlist[cnt] = q / n_used; ++cnt; }
            s_cnt = cnt;
            s_first = q;  // resume point
        }
        __syncthreads();
        const int cnt = s_cnt;
        q0 = s_first;
        if (cnt == 1)
            moe_tokens<QT, 1, R>(out, scale, wr, roff, xr, plist, tlist, cnt, in_f, n_ff, gl, lpr, myrow0);
        else if (cnt == 2)
            moe_tokens<QT, 2, R>(out, scale, wr, roff, xr, plist, tlist, cnt, in_f, n_ff, gl, lpr, myrow0);
        else if (cnt > 0)
            moe_tokens<QT, 4, R>(out, scale, wr, roff, xr, plist, tlist, cnt, in_f, n_ff, gl, lpr, myrow0);
    }
}

// ------------------------------------------------------------------ load-only twin
// Same grid, descriptors and unit loads as gemv_kernel<QT, 1, R>; the decode
// and FMAs are replaced by an XOR of the raw words.
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

template <int QT, int R>
__global__ __launch_bounds__(256) void loadonly_kernel(uint32_t* __restrict__ sink,
                                                       const uint8_t* __restrict__ w, int m, int k,
                                                       int rb, int lpr_log2) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lpr = 1 << lpr_log2;
    const int gl = lane & (lpr - 1), slot = lane >> lpr_log2;
    const int rows_per_wave = (64 >> lpr_log2) * R;
    const int64_t row0 = (int64_t)blockIdx.x * 4 * rows_per_wave;
    int64_t base;
    const rsrc_t wr = row_window(w, row0, 4 * rows_per_wave, m, rb, base);
    const int64_t myrow0 = row0 + wave * rows_per_wave + slot * R;
    uint32_t roff[R], acc[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        roff[rr] = (uint32_t)((myrow0 + rr) * rb - base);
        acc[rr] = 0;
    }
    const int n_units = (k + GUnit<QT>::UE - 1) / GUnit<QT>::UE;
    for (int u = gl; u < n_units; u += lpr) {
        GUnit<QT> un[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) un[rr].load(wr, roff[rr], u, k);
#pragma unroll
        for (int rr = 0; rr < R; ++rr) acc[rr] ^= raw_xor(un[rr]);
    }
    for (int off = lpr >> 1; off > 0; off >>= 1)
#pragma unroll
        for (int rr = 0; rr < R; ++rr) acc[rr] ^= __shfl_xor(acc[rr], off, 64);
    if (gl == 0)
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            if (myrow0 + rr < m) sink[myrow0 + rr] = acc[rr];
}

// ------------------------------------------------------------------ launchers

static int lpr_log2_for(int64_t n_units) {
    int l = 0;
    while (l < 6 && (int64_t(2) << l) <= n_units) ++l;
    return l;  // largest power of two <= min(n_units, 64)
}

int gemv_unit_elems(int qt) {
    switch (qt) {
        case QT_F32: return GUnit<QT_F32>::UE;
        case QT_Q4_0: return GUnit<QT_Q4_0>::UE;
        case QT_Q8_0: return GUnit<QT_Q8_0>::UE;
        case QT_Q4_K: return GUnit<QT_Q4_K>::UE;
        case QT_Q6_K: return GUnit<QT_Q6_K>::UE;
        case QT_NVFP4: return GUnit<QT_NVFP4>::UE;
    }
    return 0;
}

// Rows per work group for a given R (host mirror of the kernels' mapping).
static int64_t rows_per_wg(int lpr_log2, int R) { return 4 * (64 >> lpr_log2) * R; }

static int pick_R(int64_t m, int lpr_log2, int64_t groups_y) {
    for (int R : {4, 2}) {
        const int64_t wgs = (m + rows_per_wg(lpr_log2, R) - 1) / rows_per_wg(lpr_log2, R) * groups_y;
        if (wgs >= 1024) return R;
    }
    return 1;
}

int64_t gemv_max_window_bytes(int qt, int64_t k, int64_t rb) {
    const int l = lpr_log2_for((k + gemv_unit_elems(qt) - 1) / gemv_unit_elems(qt));
    return rows_per_wg(l, 4) * rb + 16;
}

template <int QT, int NT>
static void launch_gemv_nt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k,
                           int64_t n, int64_t rb, hipStream_t st) {
    const int l = lpr_log2_for((k + GUnit<QT>::UE - 1) / GUnit<QT>::UE);
    const int64_t gy = (n + NT - 1) / NT;
    const int R = pick_R(m, l, gy);
    const dim3 grid((unsigned)((m + rows_per_wg(l, R) - 1) / rows_per_wg(l, R)), (unsigned)gy);
    if (R == 4)
        gemv_kernel<QT, NT, 4><<<grid, 256, 0, st>>>(dst, w, x, (int)m, (int)k, (int)n, (int)rb, l);
    else if (R == 2)
        gemv_kernel<QT, NT, 2><<<grid, 256, 0, st>>>(dst, w, x, (int)m, (int)k, (int)n, (int)rb, l);
    else
        gemv_kernel<QT, NT, 1><<<grid, 256, 0, st>>>(dst, w, x, (int)m, (int)k, (int)n, (int)rb, l);
}

template <int QT>
static void launch_gemv_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k,
                           int64_t n, int64_t rb, hipStream_t st) {
    if (n == 1) launch_gemv_nt<QT, 1>(dst, w, x, m, k, n, rb, st);
    else if (n == 2) launch_gemv_nt<QT, 2>(dst, w, x, m, k, n, rb, st);
    else if (n <= 4) launch_gemv_nt<QT, 4>(dst, w, x, m, k, n, rb, st);
    else launch_gemv_nt<QT, 8>(dst, w, x, m, k, n, rb, st);
}

void launch_gemv(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                 int qt, int64_t rb, hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_gemv_qt<QT_F32>(dst, wb, x, m, k, n, rb, st); break;
        case QT_Q4_0: launch_gemv_qt<QT_Q4_0>(dst, wb, x, m, k, n, rb, st); break;
        case QT_Q8_0: launch_gemv_qt<QT_Q8_0>(dst, wb, x, m, k, n, rb, st); break;
        case QT_Q4_K: launch_gemv_qt<QT_Q4_K>(dst, wb, x, m, k, n, rb, st); break;
        case QT_Q6_K: launch_gemv_qt<QT_Q6_K>(dst, wb, x, m, k, n, rb, st); break;
        case QT_NVFP4: launch_gemv_qt<QT_NVFP4>(dst, wb, x, m, k, n, rb, st); break;
    }
}

template <int QT>
static void launch_moe_qt(float* g, float* u, const uint8_t* wg, const uint8_t* wu, const int* ids,
                          const float* sc, const float* x, int64_t t, int64_t n_used,
                          int64_t n_expert, int64_t in_f, int64_t n_ff, int64_t rb,
                          hipStream_t st) {
    const int l = lpr_log2_for(in_f / GUnit<QT>::UE);
    const int64_t n_pairs = t * n_used;
    const int R = pick_R(n_ff, l, n_pairs * 2);
    const dim3 grid((unsigned)((n_ff + rows_per_wg(l, R) - 1) / rows_per_wg(l, R)),
                    (unsigned)n_pairs, 2);
    if (R == 4)
        moe_gateup_kernel<QT, 4><<<grid, 256, 0, st>>>(g, u, wg, wu, ids, sc, x, (int)t, (int)n_used,
                                                       (int)n_expert, (int)in_f, (int)n_ff, (int)rb, l);
    else if (R == 2)
        moe_gateup_kernel<QT, 2><<<grid, 256, 0, st>>>(g, u, wg, wu, ids, sc, x, (int)t, (int)n_used,
                                                       (int)n_expert, (int)in_f, (int)n_ff, (int)rb, l);
    else
        moe_gateup_kernel<QT, 1><<<grid, 256, 0, st>>>(g, u, wg, wu, ids, sc, x, (int)t, (int)n_used,
                                                       (int)n_expert, (int)in_f, (int)n_ff, (int)rb, l);
}

void launch_moe(float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                const float* x, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                int64_t n_ff, int qt, int64_t rb, hipStream_t st) {
    const uint8_t* a = (const uint8_t*)wg;
    const uint8_t* b = (const uint8_t*)wu;
    switch (qt) {
        case QT_F32: launch_moe_qt<QT_F32>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
        case QT_Q4_0: launch_moe_qt<QT_Q4_0>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
        case QT_Q8_0: launch_moe_qt<QT_Q8_0>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
        case QT_Q4_K: launch_moe_qt<QT_Q4_K>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
        case QT_Q6_K: launch_moe_qt<QT_Q6_K>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
        case QT_NVFP4: launch_moe_qt<QT_NVFP4>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb, st); break;
    }
}

template <int QT>
static void launch_lo_qt(uint32_t* sink, const uint8_t* w, int64_t m, int64_t k, int64_t rb,
                         hipStream_t st) {
    const int l = lpr_log2_for((k + GUnit<QT>::UE - 1) / GUnit<QT>::UE);
    const int R = pick_R(m, l, 1);
    const dim3 grid((unsigned)((m + rows_per_wg(l, R) - 1) / rows_per_wg(l, R)));
    if (R == 4) loadonly_kernel<QT, 4><<<grid, 256, 0, st>>>(sink, w, (int)m, (int)k, (int)rb, l);
    else if (R == 2) loadonly_kernel<QT, 2><<<grid, 256, 0, st>>>(sink, w, (int)m, (int)k, (int)rb, l);
    else loadonly_kernel<QT, 1><<<grid, 256, 0, st>>>(sink, w, (int)m, (int)k, (int)rb, l);
}

void launch_loadonly(uint32_t* sink, const void* w, int64_t m, int64_t k, int qt, int64_t rb,
                     hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_lo_qt<QT_F32>(sink, wb, m, k, rb, st); break;
        case QT_Q4_0: launch_lo_qt<QT_Q4_0>(sink, wb, m, k, rb, st); break;
        case QT_Q8_0: launch_lo_qt<QT_Q8_0>(sink, wb, m, k, rb, st); break;
        case QT_Q4_K: launch_lo_qt<QT_Q4_K>(sink, wb, m, k, rb, st); break;
        case QT_Q6_K: launch_lo_qt<QT_Q6_K>(sink, wb, m, k, rb, st); break;
        case QT_NVFP4: launch_lo_qt<QT_NVFP4>(sink, wb, m, k, rb, st); break;
    }
}

}  // namespace qmm
