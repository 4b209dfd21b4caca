// MoE projections on the streaming core (stream.hpp): the gate/up rows with
// per-expert de-duplication, on f32 or Q8_1 activations; the down
// projection and its slot sum; the Q8_1 quantization; the NVFP4 V2 repack.
#include "stream.hpp"

namespace qmm {

// ------------------------------------------------------------------ MoE gate/up
// grid: x = work groups per (pair, plane) (their waves stride over the row
// groups of one expert's n_ff rows), y = pair p, z = plane (2: gate and up;
// 1: the down projection's single plane).
// The work groups of the FIRST pair routed to expert e gather every pair
// routed to e and apply e's rows to all their activation rows, so each
// selected expert's rows are read once per call when it has at most MOE_NT
// pairs (in chunks of MOE_NT otherwise), with the chunk's activations staged
// in LDS; the work groups of later pairs of the same expert exit after the
// check.  The decision depends on expert_ids only.  The activation row of
// pair q is its token's row q / n_used (gate/up) or its own row q
// (act_pair: the down projection, whose input is the pair's SwiGLU output).
constexpr int MOE_CHUNK = 256;  // pairs examined (and gathered) per pass
constexpr int MOE_NT = 3;       // token rows staged in LDS at a time
constexpr unsigned MOE_MIN_WG = 32;  // work groups per (pair, plane) at least

template <int QT, int NT, int R, int D, bool XL>
__device__ __forceinline__ void moe_tokens(float* __restrict__ out, const float* __restrict__ scale,
                                           const StreamGeom& g, int n_rg, rsrc_t xr,
                                           const int* plist, const int* tlist, int c0, int cnt,
                                           int in_f, int n_ff) {
    const int wave = wave_id();
    uint32_t xoff[NT];
    int pj[NT];
    float fj[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int c = (c0 + j < cnt) ? c0 + j : c0;  // absent slots repeat a real token
        xoff[j] = (uint32_t)tlist[c] * (uint32_t)in_f * 4u;
        pj[j] = (c0 + j < cnt) ? plist[c] : -1;
        fj[j] = scale[plist[c]];
    }
    auto store = [&](int64_t row, int j, float v) {
        if (row < n_ff && pj[j] >= 0) out[(int64_t)pj[j] * n_ff + row] = fj[j] * v;
    };
    if constexpr (XL) {
        __syncthreads();  // the previous chunk's waves are done with the staged x
        constexpr bool SM = GUnit<QT>::RUNS > 0;
        const XLds<NT, SM> xs{qmm_dyn_lds, xpad_len(in_f), qmm_dyn_lds + NT * xpad_len(in_f), in_f >> 4};
        gemv_stream<QT, NT, R, D>(g, blockIdx.x * 4 + wave, gridDim.x * 4, n_rg, xs, store,
                                  [&]() { stage_x<NT, SM>(qmm_dyn_lds, xr, xoff, in_f); });
    } else {
        XGlobal<NT> xs;
        xs.xr = xr;
#pragma unroll
        for (int j = 0; j < NT; ++j) xs.xoff[j] = xoff[j];
        gemv_stream<QT, NT, R, D>(g, blockIdx.x * 4 + wave, gridDim.x * 4, n_rg, xs, store);
    }
}

// moe_tokens for Q8_1 activations: codes and block scales of the chunk's
// token rows staged in LDS (always: a row is 2.6 bytes per weight there).
template <int QT, int NT, int R, int D>
__device__ __forceinline__ void moe_tokens_q8(float* __restrict__ out, const float* __restrict__ scale,
                                              const StreamGeom& g, int n_rg, rsrc_t qr, rsrc_t dr,
                                              const int* plist, const int* tlist, int c0, int cnt,
                                              int in_f, int n_ff) {
    const int wave = wave_id();
    uint32_t qoff[NT], doff[NT];
    int pj[NT];
    float fj[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int c = (c0 + j < cnt) ? c0 + j : c0;  // absent slots repeat a real token
        qoff[j] = (uint32_t)tlist[c] * (uint32_t)in_f;
        doff[j] = (uint32_t)tlist[c] * (uint32_t)(in_f / 32) * 4u;
        pj[j] = (c0 + j < cnt) ? plist[c] : -1;
        fj[j] = scale[plist[c]];
    }
    auto store = [&](int64_t row, int j, float v) {
        if (row < n_ff && pj[j] >= 0) out[(int64_t)pj[j] * n_ff + row] = fj[j] * v;
    };
    __syncthreads();  // the previous chunk's waves are done with the staged rows
    _Float16* sx = (_Float16*)qmm_dyn_lds;
    const XLdsQ8<NT> xs{sx, q8pad_len(in_f), (const float*)(sx + NT * q8pad_len(in_f)), in_f / 32};
    gemv_stream<QT, NT, R, D>(g, blockIdx.x * 4 + wave, gridDim.x * 4, n_rg, xs, store,
                              [&]() { stage_q8<NT>(sx, qr, dr, qoff, doff, in_f); });
}

template <int QT, int R, int D, bool Q8 = false>
__global__ __launch_bounds__(256) void moe_gateup_kernel(
    float* __restrict__ gate_out, float* __restrict__ up_out, const uint8_t* __restrict__ w_gate,
    const uint8_t* __restrict__ w_up, const int* __restrict__ ids, const float* __restrict__ pscale,
    const float* __restrict__ x, int t, int n_used, int n_expert, int in_f, int n_ff, int rb,
    int lpr_log2, int n_rg, int xl, int act_pair, const int8_t* __restrict__ xq = nullptr,
    const float* __restrict__ xd = nullptr) {
    __shared__ int plist[MOE_CHUNK];
    __shared__ int tlist[MOE_CHUNK];
    __shared__ int wcnt[4];
    __shared__ int s_seen;
    const int n_pairs = t * n_used;
    const int p = blockIdx.y, plane = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int e = uniform_i32(ids[p]);
    float* out = plane == 0 ? gate_out : up_out;
    const float* scale = pscale + (int64_t)plane * n_pairs;

    // Is p the first pair routed to e?
    if (tid == 0) s_seen = 0;
    __syncthreads();
    for (int q0 = 0; q0 < p; q0 += MOE_CHUNK) {
        const int q = q0 + tid;
        if (q < p && ids[q] == e) s_seen = 1;
    }
    __syncthreads();
    if (s_seen) return;

    const int RG = (64 >> lpr_log2) * R;
    if (e < 0 || e >= n_expert) {  // invalid id: poison every pair that carries it
        for (int q = p; q < n_pairs; ++q) {
            if (ids[q] != e) continue;
            for (int rg = blockIdx.x; rg < n_rg; rg += gridDim.x)
                for (int r = tid; r < RG; r += 256) {
                    const int64_t row = (int64_t)rg * RG + r;
                    if (row < n_ff) out[(int64_t)q * n_ff + row] = __builtin_nanf("");
                }
        }
        return;
    }

    const StreamGeom g{(plane == 0 ? w_gate : w_up) + (int64_t)e * n_ff * rb, n_ff, rb, in_f,
                       lpr_log2};
    const rsrc_t xr = make_rsrc(x, (uint32_t)(act_pair ? n_pairs : t) * (uint32_t)in_f * 4u);
    for (int q0 = p; q0 < n_pairs; q0 += MOE_CHUNK) {
        // gather the pairs of this chunk routed to e, in pair order
        const int q = q0 + tid;
        const bool hit = q < n_pairs && ids[q] == e;
        const uint64_t bal = __ballot(hit);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        __syncthreads();
        if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int off = 0;
        for (int wv = 0; wv < wave; ++wv) off += wcnt[wv];
        if (hit) {
            plist[off + before] = q;
            tlist[off + before] = act_pair ? q : q / n_used;  // activation row
        }
        const int cnt = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        __syncthreads();
        for (int c0 = 0; c0 < cnt; c0 += MOE_NT) {
            const int left = cnt - c0;
            if constexpr (Q8) {
                const rsrc_t qr = make_rsrc(xq, (uint32_t)t * (uint32_t)in_f);
                const rsrc_t dr = make_rsrc(xd, (uint32_t)t * (uint32_t)(in_f / 32) * 4u);
                if (left == 1)
                    moe_tokens_q8<QT, 1, R, D>(out, scale, g, n_rg, qr, dr, plist, tlist, c0, cnt, in_f, n_ff);
                else if (left == 2)
                    moe_tokens_q8<QT, 2, R, D>(out, scale, g, n_rg, qr, dr, plist, tlist, c0, cnt, in_f, n_ff);
                else
                    moe_tokens_q8<QT, 3, R, D>(out, scale, g, n_rg, qr, dr, plist, tlist, c0, cnt, in_f, n_ff);
            } else if (xl) {
                if (left == 1)
                    moe_tokens<QT, 1, R, D, true>(out, scale, g, n_rg, xr, plist, tlist, c0, cnt, in_f, n_ff);
                else if (left == 2)
                    moe_tokens<QT, 2, R, D, true>(out, scale, g, n_rg, xr, plist, tlist, c0, cnt, in_f, n_ff);
                else
                    moe_tokens<QT, 3, R, D, true>(out, scale, g, n_rg, xr, plist, tlist, c0, cnt, in_f, n_ff);
            } else {
                moe_tokens<QT, MOE_NT, R, 2, false>(out, scale, g, n_rg, xr, plist, tlist, c0, cnt, in_f, n_ff);
            }
        }
    }
}

// ------------------------------------------------------------------ launchers

template <int QT>
static void launch_moe_qt(float* g, float* u, const uint8_t* wg, const uint8_t* wu, const int* ids,
                          const float* sc, const float* x, int64_t t, int64_t n_used,
                          int64_t n_expert, int64_t in_f, int64_t n_ff, int64_t rb, int planes,
                          int act_pair, const GemvTuning& tune, hipStream_t st) {
    with_rd<1>(tune, [&](auto Rc, auto Dc) {
        constexpr int R = decltype(Rc)::value, D = decltype(Dc)::value;
        const int l = lpr_for(QT, in_f, LPR_CAP_MULTI);
        const int64_t n_pairs = t * n_used;
        const int64_t n_rg = (n_ff + rg_rows(l, R) - 1) / rg_rows(l, R);
        // at most one set of work groups per distinct expert and plane is
        // active; with many pairs the sets are not all distinct, so each set
        // gets at least MOE_MIN_WG work groups
        const int64_t active = planes * (n_pairs < n_expert ? n_pairs : n_expert);
        GemvTuning mt = tune;
        mt.wg_per_cu = tune.moe_wg_per_cu;
        unsigned gx = stream_grid(n_rg, active, mt);
        const unsigned need = (unsigned)((n_rg + 3) / 4);
        if (gx < MOE_MIN_WG) gx = need < MOE_MIN_WG ? need : MOE_MIN_WG;
        const dim3 grid(gx, (unsigned)n_pairs, (unsigned)planes);
        const int64_t lds = (int64_t)xlds_floats(MOE_NT, (int)in_f, GUnit<QT>::RUNS > 0) * 4;
        const int xl = lds <= XLDS_MAX_BYTES;
        moe_gateup_kernel<QT, R, D><<<grid, 256, (size_t)(xl ? lds : 0), st>>>(
            g, u, wg, wu, ids, sc, x, (int)t, (int)n_used, (int)n_expert, (int)in_f, (int)n_ff,
            (int)rb, l, (int)n_rg, xl, act_pair);
    });
}

void launch_moe(float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                const float* x, int64_t t, int64_t n_used, int64_t n_expert, int64_t in_f,
                int64_t n_ff, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const uint8_t* a = (const uint8_t*)wg;
    const uint8_t* b = (const uint8_t*)wu;
    QMM_QT_SWITCH(qt, (launch_moe_qt<Q>(g, u, a, b, ids, sc, x, t, n_used, n_expert, in_f, n_ff, rb,
                                        2, 0, tune, st)))
}

// ------------------------------------------------------------------ Q8_1 gate/up
template <int QT>
static void launch_moe_q8_qt(float* g, float* u, const uint8_t* wg, const uint8_t* wu, const int* ids,
                             const float* sc, const int8_t* xq, const float* xd, int64_t t,
                             int64_t n_used, int64_t n_expert, int64_t in_f, int64_t n_ff, int64_t rb,
                             const GemvTuning& tune, hipStream_t st) {
    with_rd<1>(tune, [&](auto Rc, auto Dc) {
        constexpr int R = decltype(Rc)::value, D = decltype(Dc)::value;
        const int l = lpr_for(QT, in_f, LPR_CAP_MULTI);
        const int64_t n_pairs = t * n_used;
        const int64_t n_rg = (n_ff + rg_rows(l, R) - 1) / rg_rows(l, R);
        const int64_t active = 2 * (n_pairs < n_expert ? n_pairs : n_expert);
        GemvTuning mt = tune;
        mt.wg_per_cu = tune.moe_wg_per_cu;
        unsigned gx = stream_grid(n_rg, active, mt);
        const unsigned need = (unsigned)((n_rg + 3) / 4);
        if (gx < MOE_MIN_WG) gx = need < MOE_MIN_WG ? need : MOE_MIN_WG;
        const dim3 grid(gx, (unsigned)n_pairs, 2);
        moe_gateup_kernel<QT, R, D, true><<<grid, 256, (size_t)q8lds_bytes(MOE_NT, (int)in_f), st>>>(
            g, u, wg, wu, ids, sc, nullptr, (int)t, (int)n_used, (int)n_expert, (int)in_f, (int)n_ff,
            (int)rb, l, (int)n_rg, 1, 0, xq, xd);
    });
}

int64_t moe_q8_lds_bytes(int64_t in_f) { return q8lds_bytes(MOE_NT, (int)in_f); }

void launch_moe_q8(float* g, float* u, const void* wg, const void* wu, const int* ids, const float* sc,
                   const int8_t* xq, const float* xd, int64_t t, int64_t n_used, int64_t n_expert,
                   int64_t in_f, int64_t n_ff, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const uint8_t* a = (const uint8_t*)wg;
    const uint8_t* b = (const uint8_t*)wu;
    if (qt == QT_NVFP4)
        launch_moe_q8_qt<QT_NVFP4>(g, u, a, b, ids, sc, xq, xd, t, n_used, n_expert, in_f, n_ff, rb, tune, st);
    else if (qt == QT_NVFP4_V2)
        launch_moe_q8_qt<QT_NVFP4_V2>(g, u, a, b, ids, sc, xq, xd, t, n_used, n_expert, in_f, n_ff, rb, tune, st);
}

// Q8_1 quantization, one thread per block of 32 activations: d = max|x| /
// 127 and q = round-half-away(x * (1/d)) (0 when d = 0), in f32.
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(int8_t* __restrict__ q, float* __restrict__ d,
                                                            const float* __restrict__ x, int64_t nblk) {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
        const f32x4* xp = (const f32x4*)(x + 32 * b);
        f32x4 v[8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = xp[i];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        }
        const float dd = amax / 127.0f;
        const float id = dd != 0.0f ? 1.0f / dd : 0.0f;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c0 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].x * id);
            const uint32_t c1 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].y * id);
            const uint32_t c2 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].z * id);
            const uint32_t c3 = (uint32_t)(uint8_t)(int8_t)(int)roundf(v[i].w * id);
            w[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        }
        *(u32x4*)(q + 32 * b) = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4*)(q + 32 * b + 16) = u32x4{w[4], w[5], w[6], w[7]};
        d[b] = dd;
    }
}

void launch_quantize_q8_1(int8_t* q, float* d, const float* x, int64_t nblk, hipStream_t st) {
    int64_t blocks = (nblk + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    quantize_q8_1_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(q, d, x, nblk);
}

// ------------------------------------------------------------------ MoE down
// y[tau*d + r] = sum over s < n_used, in order, of pair_out[(tau*n_used + s)*d + r].
// One thread per four consecutive outputs when d is a multiple of 4.
template <int V>
__global__ __launch_bounds__(256) void moe_slot_sum_kernel(float* __restrict__ y,
                                                           const float* __restrict__ pair_out,
                                                           int64_t t, int n_used, int64_t d) {
    const int64_t nv = t * d / V;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
        const int64_t tau = i * V / d, r = i * V - tau * d;
        const float* src = pair_out + tau * n_used * d + r;
        // slots in order 0, 1, ...; the loads of up to 8 slots are issued
        // before their sums, so their latencies overlap
        using T = typename std::conditional<V == 4, f32x4, float>::type;
        T acc = *(const T*)src;
        for (int s0 = 1; s0 < n_used; s0 += 8) {
            T v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n_used) v[u] = *(const T*)(src + (int64_t)(s0 + u) * d);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n_used) acc += v[u];
        }
        *(T*)(y + i * V) = acc;
    }
}

void launch_moe_down(float* y, float* pair_out, const void* wd, const int* ids, const float* sc,
                     const float* act, int64_t t, int64_t n_used, int64_t n_expert, int64_t n_ff,
                     int64_t d_model, int qt, int64_t rb, const GemvTuning& tune, hipStream_t st) {
    const uint8_t* a = (const uint8_t*)wd;
    QMM_QT_SWITCH(qt, (launch_moe_qt<Q>(pair_out, pair_out, a, a, ids, sc, act, t, n_used, n_expert,
                                        n_ff, d_model, rb, 1, 1, tune, st)))
    const bool v4 = (d_model & 3) == 0 && ((uintptr_t)y & 15) == 0 && ((uintptr_t)pair_out & 15) == 0;
    const int64_t nv = t * d_model / (v4 ? 4 : 1);
    int64_t blocks = (nv + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (v4)
        moe_slot_sum_kernel<4><<<dim3((unsigned)blocks), 256, 0, st>>>(y, pair_out, t, (int)n_used, d_model);
    else
        moe_slot_sum_kernel<1><<<dim3((unsigned)blocks), 256, 0, st>>>(y, pair_out, t, (int)n_used, d_model);
}

// ------------------------------------------------------------------ V2 repack
// NVFP4 rows -> NVFP4 V2 rows.  Item (row, G): the 36 bytes of group G are
// its scale word and 32 quant bytes; the quant bytes go to 32G and the scale
// word to k/2 + 4G of the same row (9 dword loads, 9 dword stores).
__global__ __launch_bounds__(256) void nvfp4_repack_v2_kernel(uint32_t* __restrict__ dst,
                                                              const uint32_t* __restrict__ src,
                                                              int64_t rows, int64_t k) {
    const int64_t groups = k / 64, rw = groups * 9;  // dwords per row
    const int64_t items = rows * groups;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < items; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / groups, G = i - r * groups;
        const uint32_t* s = src + r * rw + 9 * G;
        uint32_t* d = dst + r * rw;
        uint32_t v[9];
#pragma unroll
        for (int j = 0; j < 9; ++j) v[j] = s[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) d[8 * G + j] = v[1 + j];
        d[8 * groups + G] = v[0];
    }
}

void launch_nvfp4_repack_v2(void* dst, const void* src, int64_t rows, int64_t k, hipStream_t st) {
    const int64_t items = rows * (k / 64);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    nvfp4_repack_v2_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src,
                                                                   rows, k);
}

}  // namespace qmm
