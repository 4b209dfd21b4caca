// Prefill path with activations rounded to f16 once per call.
//
// x16_perm_kernel rounds x to f16 (round to nearest even, as the tile loads
// of gemm_mfma.hip do) into a caller workspace, with each row laid out in
// the k order of the weight tiles of the format (mfma_tiles.hpp) and padded
// with zeros to a whole number of 64-k steps.  The GEMM then reads its
// activation tiles as plain 16-byte copies: half the bytes of f32
// activations and no conversion in the k loop.
//
// gemm_mfma_x16_kernel<QT, WM>: one work group of 128*WM threads (WM x 2
// waves) computes a (64*WM) x 128 tile of dst (weight rows x tokens).  Each
// wave owns a 64 x 64 sub-tile (v_mfma_f32_16x16x32_f16, f32 accumulators).
// Tall tiles (WM = 4: 256 weight rows) halve the activation bytes each
// weight tile has to read per flop; the weights are decoded exactly as in
// gemm_mfma.hip (two threads per weight row, 32 weights each per step).  The
// k loop, its two-deep register ring, the double-buffered LDS tiles and the
// split of k over work items with a partial-tile workspace are as there.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tiles.hpp"

namespace qmm {

// Activation row p-slot layout: slot 64*kt + 8*s + i of a row holds k =
// g*2H + 4*s' + i (i < 4) or g*2H + H + 4*s' + (i - 4) (i >= 4), with
// U = 8*kt + s, g = U / (H/4), s' = U % (H/4); zero where that k >= k.
template <int H>
__global__ __launch_bounds__(256) void x16_perm_kernel(uint16_t* __restrict__ x16,
                                                       const float* __restrict__ x, int n, int k,
                                                       int kp, int ldx) {
    const int units = kp >> 3;  // 8-slot units per row
    const int64_t total = (int64_t)n * units;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int j = (int)(i / units), su = (int)(i - (int64_t)j * units);
        const int g = su / (H / 4), sp = su % (H / 4);  // U = su: 8 units per 64-slot step
        const int e = g * 2 * H + 4 * sp;
        const float* xr = x + (int64_t)j * ldx;
        const f32x4 a = e < k ? *(const f32x4*)(xr + e) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 b = e + H < k ? *(const f32x4*)(xr + e + H) : f32x4{0.f, 0.f, 0.f, 0.f};
        *(u32x4*)(x16 + (int64_t)j * kp + 8 * (int64_t)su) =
            u32x4{pack_f2h(a.x, a.y), pack_f2h(a.z, a.w), pack_f2h(b.x, b.y), pack_f2h(b.z, b.w)};
    }
}

template <int QT, int WM>
__global__ __launch_bounds__(128 * WM, 1) void gemm_mfma_x16_kernel(
    float* __restrict__ dst, const uint8_t* __restrict__ w, const uint16_t* __restrict__ x16, int m,
    int k, int n, int rb, int kp, int n_mb, int n_nb, int n_split, int sps, float* __restrict__ partial,
    int ldd) {
    constexpr int BMX = 64 * WM, BNX = 128, NT = 128 * WM;
    constexpr int NBC = 1024 / NT;  // 16-byte activation chunks per thread per step
    __shared__ __attribute__((aligned(16))) _Float16 sA[2][BMX * LDK];
    __shared__ __attribute__((aligned(16))) _Float16 sB[2][BNX * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Work items (k split z, tile) dealt to the 8 XCDs in contiguous runs,
    // weight-row tile fastest, as in gemm_mfma.hip.
    const int T = n_mb * n_nb, NI = T * n_split, L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3, per = NI >> 3, rem = NI & 7;
    const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int z = item / T, tile = item - z * T;
    const int nb = tile / n_mb, mb = tile - nb * n_mb;
    const int64_t m0 = (int64_t)mb * BMX, n0 = (int64_t)nb * BNX;

    int64_t base;
    const rsrc_t wr = row_window(w, m0, BMX, m, rb, base);
    const int ntok = (int)imin64(BNX, n - n0);
    const rsrc_t xr = make_rsrc(x16 + n0 * kp, (uint32_t)ntok * (uint32_t)kp * 2u);
    const int arow = tid >> 1, part = tid & 1;
    const uint32_t roff = (uint32_t)((m0 + arow) * rb - base);
    const int nk_all = (k + BK - 1) / BK;
    const int s0 = z * sps;
    const int nk = min(nk_all, s0 + sps);  // steps at or past nk read zeros
    const int kend = min(k, nk * BK);      // so do k positions at or past kend
    const int lds_a = arow * LDK + part * 32;

    // activation chunk c of thread t: token (t + c*NT) / 8, 16-byte piece (t + c*NT) % 8
    struct BLoad {
        u32x4 r[NBC];
        __device__ __forceinline__ void load(rsrc_t xr_, int kp_, int kt, int nk_, int t) {
#pragma unroll
            for (int c = 0; c < NBC; ++c) {
                const int ch = t + c * NT, tok = ch >> 3, pc = ch & 7;
                const uint32_t off = 2u * ((uint32_t)tok * (uint32_t)kp_ + 64u * (uint32_t)kt + 8u * (uint32_t)pc);
                r[c] = ld128(xr_, kt < nk_ ? off : OOB_OFF);
            }
        }
        __device__ __forceinline__ void store(_Float16* sb, int t) const {
#pragma unroll
            for (int c = 0; c < NBC; ++c) {
                const int ch = t + c * NT, tok = ch >> 3, pc = ch & 7;
                *(u32x4*)&sb[tok * LDK + 8 * pc] = r[c];
            }
        }
    };

    ALoad<QT> al0, al1;
    BLoad bl0, bl1;
    uint32_t tmp[16];
    auto stage = [&](const ALoad<QT>& al, const BLoad& bl, int buf) {
        al.decode(tmp);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *(u32x4*)&sA[buf][lds_a + 8 * u] = u32x4{tmp[4 * u], tmp[4 * u + 1], tmp[4 * u + 2], tmp[4 * u + 3]};
        bl.store(sB[buf], tid);
    };

    al0.load(wr, roff, s0, part, kend, nk);
    bl0.load(xr, kp, s0, nk, tid);
    al1.load(wr, roff, s0 + 1, part, kend, nk);
    bl1.load(xr, kp, s0 + 1, nk, tid);
    stage(al0, bl0, 0);
    __syncthreads();

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave % WM, wn = wave / WM;
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

    const int nk2 = s0 + ((nk - s0 + 1) & ~1);
    for (int kt = s0; kt < nk2; kt += 2) {
        al0.load(wr, roff, kt + 2, part, kend, nk);
        bl0.load(xr, kp, kt + 2, nk, tid);
        mfma_step(0);
        stage(al1, bl1, 1);
        interleave_hint();
        __syncthreads();
        al1.load(wr, roff, kt + 3, part, kend, nk);
        bl1.load(xr, kp, kt + 3, nk, tid);
        mfma_step(1);
        stage(al0, bl0, 0);
        interleave_hint();
        __syncthreads();
    }

    float* out = n_split > 1 ? partial + (int64_t)z * splitk_stride(n, m) : dst;
    const int64_t ldo = n_split > 1 ? m : ldd;  // partials are dense
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t mrow = m0 + wm * 64 + i * 16 + (lane >> 4) * 4;
            const int64_t tok = n0 + wn * 64 + j * 16 + (lane & 15);
            if (tok < n) {
                float* p = out + tok * ldo + mrow;
                const f32x4 v = acc[i][j];
                if ((ldo & 3) == 0 && mrow + 4 <= m) {
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

template <int QT>
static void launch_x16_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k,
                          int64_t n, int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd,
                          hipStream_t st) {
    constexpr int H = Perm<QT>::H;
    const int64_t kp = x16_row_halves(k);
    uint16_t* x16 = (uint16_t*)ws;
    float* part = (float*)((uint8_t*)ws + x16_bytes(n, k));
    {
        const int64_t total = n * (kp / 8);
        int64_t blocks = (total + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        x16_perm_kernel<H><<<dim3((unsigned)blocks), 256, 0, st>>>(x16, x, (int)n, (int)k, (int)kp, (int)ldx);
    }
    const int bm = 64 * pl.wm;
    const int n_mb = (int)((m + bm - 1) / bm), n_nb = (int)((n + 127) / 128);
    const dim3 grid((unsigned)(n_mb * n_nb * pl.n_split));
    if (pl.wm == 4)
        gemm_mfma_x16_kernel<QT, 4><<<grid, 512, 0, st>>>(dst, w, x16, (int)m, (int)k, (int)n, (int)rb,
                                                          (int)kp, n_mb, n_nb, pl.n_split, pl.sps, part,
                                                          (int)ldd);
    else
        gemm_mfma_x16_kernel<QT, 2><<<grid, 256, 0, st>>>(dst, w, x16, (int)m, (int)k, (int)n, (int)rb,
                                                          (int)kp, n_mb, n_nb, pl.n_split, pl.sps, part,
                                                          (int)ldd);
    if (pl.n_split > 1) launch_splitk_sum(dst, part, n * m, splitk_stride(n, m), pl.n_split, m, ldd, st);
}

void launch_gemm_mfma_x16(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                          int qt, int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd,
                          hipStream_t st) {
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_x16_qt<QT_F32>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_0: launch_x16_qt<QT_Q4_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q8_0: launch_x16_qt<QT_Q8_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_K: launch_x16_qt<QT_Q4_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q6_K: launch_x16_qt<QT_Q6_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_NVFP4: launch_x16_qt<QT_NVFP4>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
    }
}

}  // namespace qmm
