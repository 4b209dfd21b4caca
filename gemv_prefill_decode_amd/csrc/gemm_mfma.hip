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
// loads, the decode and the matrix-core work overlap.  (This is the kernel
// for calls without a workspace; gemm_lds.hip holds the LDS-ring kernels the
// planner chooses when a workspace is given.)
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_tiles.hpp"

namespace qmm {

constexpr int BM = MFMA_BM, BN = MFMA_BN;

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
// KG k groups (KG = 2: 512 threads): group g of 4 waves takes the steps
// s0 + g, s0 + g + KG, ... of the item with tiles of its own, so a CU holding
// one work group has 2 waves per SIMD whose loads, decode and matrix-core
// work hide each other's latency; at the end group 1 hands its accumulators
// to group 0 through LDS, which adds them (group 0's + group 1's, a fixed
// order) and stores the tile.
template <int QT, int KG>
__global__ __launch_bounds__(256 * KG, 1) void gemm_mfma_kernel(float* __restrict__ dst,
                                                                const uint8_t* __restrict__ w,
                                                                const float* __restrict__ x, int m,
                                                                int k, int n, int rb, int n_mb,
                                                                int n_nb, int n_split, int sps,
                                                                float* __restrict__ partial, int ldx,
                                                                int ldd) {
    constexpr int TILE_H = BM * LDK;  // halves per A or B tile (BM == BN)
    __shared__ __attribute__((aligned(16))) _Float16 lds[KG][2][2][TILE_H];  // [group][buffer][A, B]
    const int tid = threadIdx.x, lane = tid & 63;
    const int g = KG == 1 ? 0 : tid >> 8, lt = tid & 255, wave = lt >> 6;
    // the weight (A) and activation (B) tiles of buffer buf of this thread's group
    auto tileA = [&](int buf) -> _Float16* { return lds[g][buf][0]; };
    auto tileB = [&](int buf) -> _Float16* { return lds[g][buf][1]; };

    // Work groups are dealt round-robin to the 8 XCDs (id % 8); give each XCD
    // a contiguous run of work items, numbered with the weight-row tile mb
    // fastest, so the work groups running together on an XCD share one
    // activation tile (the larger operand per step) in its L2.
    const int T = n_mb * n_nb, NI = T * n_split, L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3, per = NI >> 3, rem = NI & 7;
    const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int z = item / T, tile = item - z * T;
    const int nb = tile / n_mb, mb = tile - nb * n_mb;
    const int64_t m0 = (int64_t)mb * BM, n0 = (int64_t)nb * BN;

    int64_t base;
    const rsrc_t wr = row_window(w, m0, BM, m, rb, base);
    const int ntok = (int)imin64(BN, n - n0);
    // token rows ldx floats apart; the window ends with the last row's k floats
    const rsrc_t xr = make_rsrc(x + n0 * ldx, ((uint32_t)(ntok - 1) * (uint32_t)ldx + (uint32_t)k) * 4u);
    const int arow = lt >> 1, part = lt & 1;
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
        _Float16* a = tileA(buf);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *(u32x4*)&a[lds_a + 8 * u] = u32x4{tmp[4 * u], tmp[4 * u + 1], tmp[4 * u + 2], tmp[4 * u + 3]};
        xl.store(tileB(buf), lt);
    };

    // Every load is unconditional (steps at or past nk read zeros through
    // out-of-range offsets, and their staged tiles are never used), so the
    // loop body is straight-line and the compiler's load counters let the
    // loads of step kt+2 stay in flight while step kt computes.
    const int g0 = s0 + g;  // this group's first step; it takes every KG-th
    al0.load(wr, roff, g0, part, kend, nk);
    xl0.template load<H>(xr, ldx, kend, g0, lt);
    al1.load(wr, roff, g0 + KG, part, kend, nk);
    xl1.template load<H>(xr, ldx, kend, g0 + KG, lt);
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
        const _Float16* A = tileA(buf) + wm * 64 * LDK + frag;
        const _Float16* B = tileB(buf) + wn * 64 * LDK + frag;
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
    // Every group runs the same number of iterations (that of group 0, which
    // has the most steps); steps past nk read zeros.
    const int cnt = (nk - s0 + KG - 1) / KG;
    const int cnt2 = (cnt + 1) & ~1;
    for (int i = 0; i < cnt2; i += 2) {
        const int kt = g0 + KG * i;
        // step kt: buffer 0; set 1 holds step kt+KG, set 0 takes kt+2KG
        al0.load(wr, roff, kt + 2 * KG, part, kend, nk);
        xl0.template load<H>(xr, ldx, kend, kt + 2 * KG, lt);
        mfma_step(0);
        stage(al1, xl1, 1);
        interleave_hint();
        __syncthreads();
        // step kt+KG: buffer 1; set 0 holds step kt+2KG, set 1 takes kt+3KG
        al1.load(wr, roff, kt + 3 * KG, part, kend, nk);
        xl1.template load<H>(xr, ldx, kend, kt + 3 * KG, lt);
        mfma_step(1);
        stage(al0, xl0, 0);
        interleave_hint();
        __syncthreads();
    }

    if constexpr (KG == 2) {
        // group 1's accumulators to group 0 through group 1's tile space
        // (2 x 2 x BM*LDK halves >= 64 KB), value v of thread lt at v*256+lt
        float* red = reinterpret_cast<float*>(&lds[1][0][0][0]);
        if (g == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[((i * 4 + j) * 4 + r) * 256 + lt] = acc[i][j][r];
        }
        __syncthreads();
        if (g == 1) return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] += red[((i * 4 + j) * 4 + r) * 256 + lt];
    }


    // D[row][col] of a 16x16 tile sits in lane (row/4)*16 + col, element row%4:
    // rows are weight rows (contiguous in dst), cols are tokens.
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

// dst[i] = part[0][i] + part[1][i] + ... + part[n_split-1][i], in that
// order, for i < count; part[z] starts at z * splitk_stride (16-byte aligned).
__global__ __launch_bounds__(256) void splitk_sum_kernel(float* __restrict__ dst,
                                                         const float* __restrict__ part,
                                                         int64_t count, int64_t zstride, int n_split,
                                                         int64_t m, int64_t ldd) {
    if (ldd != m) {  // dst rows ldd apart: element i is row i / m, column i % m
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
            float v = part[i];
            for (int z = 1; z < n_split; ++z) v += part[z * zstride + i];
            const int64_t row = i / m;
            dst[row * ldd + (i - row * m)] = v;
        }
        return;
    }
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

void launch_splitk_sum(float* dst, const float* part, int64_t count, int64_t zstride, int n_split,
                       int64_t m, int64_t ldd, hipStream_t st) {
    int64_t blocks = ((ldd == m ? count / 4 : count) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    splitk_sum_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(dst, part, count, zstride, n_split, m, ldd);
}

template <int QT>
static void launch_qt(float* dst, const uint8_t* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd, hipStream_t st) {
    const int n_mb = (int)((m + BM - 1) / BM), n_nb = (int)((n + BN - 1) / BN);
    float* part = (float*)ws;
    const dim3 grid((unsigned)(n_mb * n_nb * pl.n_split));
    if constexpr (QT != QT_F32) {
        if (pl.kg == 2) {
            gemm_mfma_kernel<QT, 2><<<grid, 512, 0, st>>>(dst, w, x, (int)m, (int)k, (int)n, (int)rb, n_mb,
                                                          n_nb, pl.n_split, pl.sps, part, (int)ldx, (int)ldd);
            if (pl.n_split > 1)
                launch_splitk_sum(dst, part, n * m, splitk_stride(n, m), pl.n_split, m, ldd, st);
            return;
        }
    }
    gemm_mfma_kernel<QT, 1><<<grid, 256, 0, st>>>(dst, w, x, (int)m, (int)k, (int)n, (int)rb, n_mb, n_nb,
                                                  pl.n_split, pl.sps, part, (int)ldx, (int)ldd);
    if (pl.n_split > 1) launch_splitk_sum(dst, part, n * m, splitk_stride(n, m), pl.n_split, m, ldd, st);
}

// Cost model of the prefill plans, fitted (least squares on log time, 242
// forced-plan timings) to MI355X measurements of the LFM2 (n = 512) and
// 8B-class (n = 2048) shapes: 7% rms error.  Per kernel family: the time of
// one k step of a work group alone on its CU (latency-bound), the time per
// step per work group when the CU's work groups are throughput-bound, and how
// many work groups fit on a CU (for the LDS-ring kernels the ring decides:
// lds_ring_per_cu).
struct FamCost {
    int x16, wm, kg;  // the plan's kernel family, tile rows / 64 and k groups
    double step_alone_us;
    double step_shared_us;
    int per_cu;
};
constexpr int N_FAM = 18;
constexpr FamCost FAM_COST[N_FAM] = {
    {0, 2, 1, 1.50, 1.04, 2},  // gemm_mfma_kernel, 128 x 128, f32 activations
    {0, 2, 2, 1.06, 1.60, 1},  // gemm_mfma_kernel with 2 k groups (time per step of the item)
    // gemm_lds_kernel; 128 x 256 tiles are priced per step of twice the work.
    // Two work groups per CU where the ring allows (Q4_0, Q4_K, NVFP4 and
    // Q8_0 128 x 128, Q6_K 128 x 128, the 4-bit formats' 128 x 256)
    {2, 2, 1, 1.00, 0.62, 1},  // 128 x 128
    {2, 4, 1, 2.00, 1.40, 1},  // 256 x 128 (slower than two 128-row tiles everywhere measured)
    {3, 2, 1, 1.36, 1.07, 1},  // 128 x 256
    {2, 2, 2, 0.72, 0.80, 1},  // 128 x 128, 2 k groups
    {3, 2, 2, 1.14, 1.10, 1},  // 128 x 256, 2 k groups
    // the same with 128 x 128 tiles on the f32 activations (no pre-pass;
    // each thread rounds its share of the step's activations to f16 once)
    {4, 2, 1, 1.10, 0.80, 1},  // 1 k group
    {4, 2, 2, 0.81, 0.80, 1},  // 2 k groups
    // 64 x 128 tiles (twice the work groups of 128-row tiles for the small
    // products), on f16 and on f32 activations
    {2, 1, 1, 0.53, 0.41, 1},
    {2, 1, 2, 0.43, 0.40, 1},
    {4, 1, 1, 0.65, 0.45, 1},
    {4, 1, 2, 0.51, 0.42, 1},
    // 64 x 64 tiles on f16 activations (four times the work groups of
    // 128 x 128 tiles; the decode work per matrix-core op doubles against
    // 64 x 128, priced by format below)
    {5, 1, 1, 0.273, 0.25, 1},
    {5, 1, 2, 0.212, 0.215, 1},
    // ... and on the f32 activations (no pre-pass; fitted to 55 more timings,
    // 7% rms)
    {6, 1, 1, 0.329, 0.224, 1},
    {6, 1, 2, 0.233, 0.197, 1},
    // 256 x 256 tiles, two token groups of 4 waves (priced per step of four
    // times the 128 x 128 work; one work group per CU; from 8B-class Q4_K
    // and Q6_K timings, 14336 x 4096 x 2048)
    {7, 4, 1, 2.08, 2.08, 1},
};
// f32 weights on the 64 x 64 f32-activation family, on top of lds64_factor
constexpr double LDS64_F32_XF_FACTOR = 1.15;
// 64 x 64 tiles: step time by format against Q4_0 (each decoded weight meets
// 64 tokens instead of 128, so the decode is a larger share of the step);
// fitted with the two families above to 64 forced-plan timings of the LFM2
// shapes (9% rms; Q8_0 raised from 1.26, where its k-split ffn_down plans
// measured slower than the 128-token ones)
constexpr double lds64_factor(int qt) {
    return qt == QT_Q4_0 ? 1.0 : qt == QT_Q8_0 ? 1.33 : qt == QT_Q4_K ? 1.365 : qt == QT_Q6_K ? 1.884 : 1.245;
}
// The LDS-ring kernel's step time by format: Q6_K's two-field 6-bit codes
// take about a quarter longer to decode; with 256-token tiles the decode is
// a smaller share of the step.
constexpr double LDS_Q6K_FACTOR_128 = 1.27, LDS_Q6K_FACTOR_128_KG2 = 1.31, LDS_Q6K_FACTOR_256 = 1.04,
                 LDS_Q6K_FACTOR_TG = 1.24;
// f32 weights on f32 activations: the activation rounding adds to the
// largest weight stages
constexpr double LDS_F32_XF_FACTOR = 1.29;
constexpr double LAUNCH_US = 4.4;      // a launch with its first loads and its stores
constexpr double SPLIT_US = 2.1;       // the split sum's launch
constexpr double X16_US = 2.7;         // the f16 pre-pass launch
constexpr double BYTES_PER_US = 4.0e6; // split partials' traffic
constexpr double X16_BYTES_PER_US = 8.1e6;  // the pre-pass's traffic (a plain stream)
// Kernels on f32 activations read twice the activation bytes of the f16
// ones, once per weight-row tile, from L2: 2nk bytes more per tile row,
// priced at this rate for the quantized formats.  With f32 weights, whose
// own rows dominate the step, the family's step time already holds it.
constexpr double XF_L2_BYTES_PER_US = 20.6e6;

MfmaPlan plan_gemm_mfma(int64_t m, int64_t k, int64_t n, int qt, int num_cu, bool have_ws,
                        const MfmaForce* force) {
    MfmaPlan best;
    const int nk = (int)((k + BK - 1) / BK);
    best.x16 = 0;
    best.wm = 2;
    best.kg = 1;
    best.n_split = 1;
    best.sps = nk + (nk & 1);
    best.ws_bytes = 0;
    if (!have_ws || num_cu < 1) return best;
    const double out_bytes = 4.0 * (double)n * (double)m;
    const double x16_us = X16_US + 6.0 * (double)n * (double)k / X16_BYTES_PER_US;
    double best_cost = 1e30;
    for (int fam = 0; fam < N_FAM; ++fam) {
        const int x16 = FAM_COST[fam].x16, wm = FAM_COST[fam].wm, kg = FAM_COST[fam].kg;
        if (kg == 2 && qt == QT_F32) continue;  // its two register rings of f32 weights exceed 256 VGPRs
        // the LDS ring: whole 64-k steps only, and f32 rows fit it with 128-row tiles only
        const int bn = x16 == 3 || x16 == 7 ? 256 : (x16 == 5 || x16 == 6 ? 64 : 128);
        const bool xf = x16 == 4 || x16 == 6;
        if (x16 >= 2 && (k % 64 != 0 || !lds_ring_fits(qt, 64 * wm, bn, kg, xf))) continue;
        // 64 x 64 tiles for products with fewer 64 x 128 tiles than CUs; with
        // more (two work groups sharing most CUs) the cost model under-prices
        // the two-k-group forms and the Q6_K and f32 rows, so there only the
        // one-group f16-activation form, for the cheaper decodes (measured
        // faster on LFM2 ffn_gate: Q4_0 19.5 -> 17.5 us, Q4_K 22.5 -> 20.6)
        // 256 x 256 tiles: measured faster than the 128-row ones for Q6_K only
        // (8B-class 14336 x 4096 x 2048: 356 against 399 us; Q4_K 291 against 249)
        if (x16 == 7 && !force && qt != QT_Q6_K) continue;
        if ((x16 == 5 || x16 == 6) && !force && ((m + 63) / 64) * ((n + 127) / 128) >= num_cu &&
            (x16 == 6 || kg != 1 || qt == QT_Q6_K || qt == QT_F32))
            continue;
        if (force && (force->x16 != x16 || force->wm != wm || force->kg != kg)) continue;
        const FamCost& fc0 = FAM_COST[fam];
        const double fmul = x16 == 5                   ? lds64_factor(qt)
                            : x16 == 6                 ? lds64_factor(qt) * (qt == QT_F32 ? LDS64_F32_XF_FACTOR : 1.0)
                            : x16 == 4 && qt == QT_F32 ? LDS_F32_XF_FACTOR
                            : x16 == 7                 ? (qt == QT_Q6_K ? LDS_Q6K_FACTOR_TG : 1.0)
                            : x16 < 2 || qt != QT_Q6_K
                                ? 1.0
                                : (x16 == 3 ? LDS_Q6K_FACTOR_256 : (kg == 2 ? LDS_Q6K_FACTOR_128_KG2 : LDS_Q6K_FACTOR_128));
        const int per_cu = x16 >= 2 ? lds_ring_per_cu(qt, 64 * wm, bn, kg, xf) : fc0.per_cu;
        const FamCost fc{x16, wm, kg, fc0.step_alone_us * fmul, fc0.step_shared_us * fmul, per_cu};
        const int64_t T = ((m + 64 * wm - 1) / (64 * wm)) * ((n + bn - 1) / bn);
        for (int S = 1; S <= 16 && (S == 1 || S <= nk / 2); ++S) {
            const int sps = ((nk + S - 1) / S + 1) & ~1;
            const int se = (nk + sps - 1) / sps;
            if (S > 1 && se < 2) continue;
            if (force && force->n_split != se) continue;
            const int64_t items = T * se;
            if (items > (int64_t)1 << 30) continue;
            if (x16 == 2 && wm == 4 && !force) continue;
            // work groups sharing a CU, time per step, and rounds of them
            const int64_t fill = (items + num_cu - 1) / num_cu;
            const int64_t share = fill < fc.per_cu ? fill : fc.per_cu;
            const double step = share > 1 ? share * fc.step_shared_us : fc.step_alone_us;
            const double step_t = step > fc.step_alone_us ? step : fc.step_alone_us;
            double rounds = (double)items / (double)(num_cu * share);
            if (share == 1 || rounds < 1.0) rounds = (double)((items + num_cu * share - 1) / (num_cu * share));
            const double xf_us = xf && qt != QT_F32 ? 2.0 * (double)n * (double)k * (double)((m + 64 * wm - 1) / (64 * wm)) /
                                                 XF_L2_BYTES_PER_US
                                          : 0.0;
            const double cost = (LAUNCH_US + rounds * sps * step_t +
                                 (se > 1 ? SPLIT_US + (2.0 * se + 1.0) * out_bytes / BYTES_PER_US : 0.0) +
                                 (x16 == 2 || x16 == 3 || x16 == 5 || x16 == 7 ? x16_us : 0.0) + xf_us);
            if (cost < best_cost) {
                best_cost = cost;
                best.x16 = x16;
                best.wm = wm;
                best.kg = kg;
                best.n_split = se;
                best.sps = sps;
            }
        }
    }
    best.ws_bytes = (best.x16 == 2 || best.x16 == 3 || best.x16 == 5 || best.x16 == 7 ? x16_bytes(n, k) : 0) +
                    (best.n_split > 1 ? (int64_t)best.n_split * splitk_stride(n, m) * 4 : 0);
    if (best.ws_bytes == 0) best.ws_bytes = 256;  // a plan that uses no workspace still takes one
    return best;
}

void launch_gemm_mfma(float* dst, const void* w, const float* x, int64_t m, int64_t k, int64_t n,
                      int qt, int64_t rb, const MfmaPlan& pl, void* ws, int64_t ldx, int64_t ldd,
                      hipStream_t st) {
    if (pl.x16 >= 2) {
        launch_gemm_lds(dst, w, x, m, k, n, qt, rb, pl, ws, ldx, ldd, st);
        return;
    }
    const uint8_t* wb = (const uint8_t*)w;
    switch (qt) {
        case QT_F32: launch_qt<QT_F32>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_0: launch_qt<QT_Q4_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q8_0: launch_qt<QT_Q8_0>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q4_K: launch_qt<QT_Q4_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_Q6_K: launch_qt<QT_Q6_K>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
        case QT_NVFP4: launch_qt<QT_NVFP4>(dst, wb, x, m, k, n, rb, pl, ws, ldx, ldd, st); break;
    }
}

}  // namespace qmm
