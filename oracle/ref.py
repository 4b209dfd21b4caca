"""Float64 reference results and the per-element tolerance.  TEST INFRASTRUCTURE.

The projection (cera `wgpu_gemm_bench.rs`, Shape: dst[n, m] = src0[m, k] *
src1[n, k], dst column-major with y_stride = m):

    ref[j, i] = sum_c W[i, c] * x[j, c],    S[j, i] = sum_c |W[i, c] * x[j, c]|

with W decoded exactly (``oracle.formats``) and the sum taken in float64 by a
plain matmul.  A device result g passes when it is finite and
|g - ref| <= tau * S element by element (tau = 2e-3 when activations and
weights are rounded to f16 for the matrix cores, 1e-5 on the f32 path).

The MoE gate/up (memra `moe_rows_ceiling_bench.rs`: gate and up planes over
in_f -> n_ff, n_used experts per token, a per-pair f32 scale indexed
plane*n_pairs + pair, as the pointer table is):

    out_P[p, r] = scale[P*n_pairs + p] * sum_c W_P[e_p][r, c] * x[tau_p, c]

for pair p = tau*n_used + s with expert e_p = ids[tau, s].

The MoE down projection (the same page's down arm: one plane of d_model rows
over n_ff inputs per expert, each pair's own activation row, the down plane's
scale, the result accumulated into a zeroed y over the token's pairs):

    y[tau, r] = sum_s scale[p] * sum_c Wd[e_p][r, c] * act[p, c]

with the slots s taken in order; S_y sums |scale[p] * Wd[e_p][r, c] * act[p, c]|.

Q8_1 activations (the served arithmetic of the same page): x is replaced by
its per-32 quantization d*q (quantize_q8_1 below) and the gate/up (or the
down projection, on each pair's activation row) is the projection of those
dequantized activations.

The activation between gate/up and down (a reading of the same page's
"preclamp" gate/up with argument 7.0 and its "swiglu output"):

    act[p, r] = silu(min(gate[p, r], L)) * clamp(up[p, r], -L, L)

with silu(z) = z / (1 + exp(-z)).
"""

from __future__ import annotations

import numpy as np

from .formats import decode


def gemm_value(name: str, w, x, m: int, k: int, n: int):
    """ref as float64 [n, m] (decode, then one f64 matmul)."""
    W = decode(name, w, m, k)
    X = np.asarray(x, dtype=np.float32).reshape(n, k).astype(np.float64)
    return X @ W.T


def gemm_ref(name: str, w, x, m: int, k: int, n: int):
    """(ref, S) as float64 [n, m]."""
    W = decode(name, w, m, k)
    X = np.asarray(x, dtype=np.float32).reshape(n, k).astype(np.float64)
    return X @ W.T, np.abs(X) @ np.abs(W).T


def gemm_ref_blocks(name: str, w, x, m: int, k: int, n: int, row_bytes: int, rows_per_block: int = 2048):
    """gemm_ref over the weight rows in blocks: yields (i0, i1, ref, S) with
    ref and S float64 [n, i1 - i0] for the rows [i0, i1), so that only one
    block of W is decoded at a time (the whole output of large shapes with
    bounded host memory).  ``row_bytes`` is the packed size of one row."""
    buf = np.asarray(w).reshape(-1).view(np.uint8)
    X = np.asarray(x, dtype=np.float32).reshape(n, k).astype(np.float64)
    aX = np.abs(X)
    for i0 in range(0, m, rows_per_block):
        i1 = min(m, i0 + rows_per_block)
        W = decode(name, buf[i0 * row_bytes:i1 * row_bytes], i1 - i0, k)
        yield i0, i1, X @ W.T, aX @ np.abs(W).T


def gemm_ref_rows(name: str, w, x, m: int, k: int, rows, cols, row_bytes: int):
    """(ref, S) for the sampled outputs dst[cols[t], rows[t]] only.

    Decodes just the sampled weight rows, so full-size shapes stay cheap.
    ``row_bytes`` is the packed size of one row (bytes; 4*k for f32)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    buf = np.asarray(w).reshape(-1).view(np.uint8)
    uniq, inv = np.unique(rows, return_inverse=True)
    sel = np.stack([buf[r * row_bytes:(r + 1) * row_bytes] for r in uniq])
    W = decode(name, sel, len(uniq), k)[inv]                      # [T, k]
    X = np.asarray(x, dtype=np.float32).reshape(-1, k)[cols].astype(np.float64)
    return np.einsum("tk,tk->t", W, X), np.einsum("tk,tk->t", np.abs(W), np.abs(X))


def moe_ref(name: str, w_gate, w_up, ids, scales, x, n_expert: int, in_f: int, n_ff: int,
            exact_x: bool = False):
    """(gate, up, S_gate, S_up) as float64 [n_pairs, n_ff].  x is float32
    (exact_x: float64 values used as they are)."""
    ids = np.asarray(ids, dtype=np.int64)
    t, n_used = ids.shape
    n_pairs = t * n_used
    X = (np.asarray(x, dtype=np.float64) if exact_x else
         np.asarray(x, dtype=np.float32).astype(np.float64)).reshape(t, in_f)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    flat = ids.reshape(-1)
    outs = []
    for plane, wp in enumerate((w_gate, w_up)):
        buf = np.asarray(wp).reshape(-1).view(np.uint8)
        per = buf.size // n_expert
        val = np.empty((n_pairs, n_ff))
        tol = np.empty((n_pairs, n_ff))
        # one expert's rows decoded at a time, applied to every pair that chose it
        for e in np.unique(flat):
            W = decode(name, buf[int(e) * per:(int(e) + 1) * per], n_ff, in_f)
            for p in np.nonzero(flat == e)[0]:
                tau = int(p) // n_used
                f = sc[plane * n_pairs + p]
                val[p] = f * (W @ X[tau])
                tol[p] = abs(f) * (np.abs(W) @ np.abs(X[tau]))
        outs.append((val, tol))
    return outs[0][0], outs[1][0], outs[0][1], outs[1][1]


def moe_ref_pairs_rows(name: str, w_plane, ids, scales, x, plane: int, n_expert: int, in_f: int,
                       n_ff: int, pairs, rows, exact_x: bool = False):
    """(ref, S) of out_P[pairs[t], rows[t]] for one plane P, sampled: only the
    sampled weight rows of the chosen experts are decoded.  x is float32
    (exact_x: float64 values used as they are)."""
    ids = np.asarray(ids, dtype=np.int64)
    t, n_used = ids.shape
    n_pairs = t * n_used
    pairs = np.asarray(pairs, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    buf = np.asarray(w_plane).reshape(-1).view(np.uint8)
    rb = buf.size // (n_expert * n_ff)
    X = (np.asarray(x, dtype=np.float64) if exact_x else
         np.asarray(x, dtype=np.float32).astype(np.float64)).reshape(t, in_f)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    val = np.empty(len(pairs))
    tol = np.empty(len(pairs))
    for i, (p, r) in enumerate(zip(pairs, rows)):
        e = int(ids.reshape(-1)[p])
        row = (e * n_ff + int(r)) * rb
        W = decode(name, buf[row:row + rb], 1, in_f)[0]
        xv = X[p // n_used]
        f = sc[plane * n_pairs + p]
        val[i] = f * float(W @ xv)
        tol[i] = abs(f) * float(np.abs(W) @ np.abs(xv))
    return val, tol


def moe_down_ref(name: str, w_down, ids, scales, act, n_expert: int, n_ff: int, d_model: int,
                 exact_act: bool = False):
    """(y, S_y, pair, S_pair): y and S_y float64 [t, d_model]; the per-pair
    terms scale[p] * Wd[e_p] @ act[p] and their S as float64 [n_pairs, d_model].
    act is float32 (exact_act: float64 values used as they are, e.g. Q8_1
    activations d*q dequantized exactly)."""
    ids = np.asarray(ids, dtype=np.int64)
    t, n_used = ids.shape
    n_pairs = t * n_used
    A = (np.asarray(act, dtype=np.float64) if exact_act else
         np.asarray(act, dtype=np.float32).astype(np.float64)).reshape(n_pairs, n_ff)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    buf = np.asarray(w_down).reshape(-1).view(np.uint8)
    per = buf.size // n_expert
    pair = np.empty((n_pairs, d_model))
    pair_S = np.empty((n_pairs, d_model))
    flat = ids.reshape(-1)
    # one expert's rows decoded at a time, applied to every pair that chose it
    for e in np.unique(flat):
        W = decode(name, buf[int(e) * per:(int(e) + 1) * per], d_model, n_ff)
        for p in np.nonzero(flat == e)[0]:
            pair[p] = sc[p] * (W @ A[p])
            pair_S[p] = abs(sc[p]) * (np.abs(W) @ np.abs(A[p]))
    y = pair.reshape(t, n_used, d_model).sum(axis=1)
    S = pair_S.reshape(t, n_used, d_model).sum(axis=1)
    return y, S, pair, pair_S


def moe_down_ref_rows(name: str, w_down, ids, scales, act, n_expert: int, n_ff: int,
                      d_model: int, toks, rows):
    """(ref, S) of y[toks[i], rows[i]], sampled: only the sampled weight rows
    of the token's experts are decoded."""
    ids = np.asarray(ids, dtype=np.int64)
    t, n_used = ids.shape
    buf = np.asarray(w_down).reshape(-1).view(np.uint8)
    rb = buf.size // (n_expert * d_model)
    A = np.asarray(act, dtype=np.float32).reshape(t * n_used, n_ff).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
    val = np.zeros(len(toks))
    tol = np.zeros(len(toks))
    for i, (tau, r) in enumerate(zip(np.asarray(toks, dtype=np.int64), np.asarray(rows, dtype=np.int64))):
        for s in range(n_used):
            p = int(tau) * n_used + s
            e = int(ids[tau, s])
            row = (e * d_model + int(r)) * rb
            W = decode(name, buf[row:row + rb], 1, n_ff)[0]
            val[i] += sc[p] * float(W @ A[p])
            tol[i] += abs(sc[p]) * float(np.abs(W) @ np.abs(A[p]))
    return val, tol


# |d/dz silu(z)| <= 1.0999 for every real z (its extremes are at z = +-2.3994:
# sigma(z)(1 + z(1 - sigma(z))) = 1.0998 and -0.0998).
SILU_LIPSCHITZ = 1.1


def swiglu_clamp(g, u, limit: float):
    """The activation between the MoE gate/up and down projections, float64.

    The memra page serves its gate/up as `moe_gate_up_preclamp8_q8_rows(...,
    7.0, ...)` and feeds its down arm "a synthetic swiglu output"; the clamp
    it applies before the activation is not spelled out.  Reading: the gate
    is clamped above at `limit`, the up projection to [-limit, limit], then
    SwiGLU: silu(g') * u' with silu(z) = z / (1 + exp(-z)).  limit = inf is
    plain SwiGLU.  NaN inputs stay NaN (np.minimum / np.maximum propagate
    them)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    gc = np.minimum(g, limit)
    uc = np.maximum(np.minimum(u, limit), -limit)
    with np.errstate(over="ignore"):
        return gc / (1.0 + np.exp(-gc)) * uc


def moe_act_ref(name: str, w_gate, w_up, ids, scales, x, n_expert: int, in_f: int, n_ff: int,
                limit: float, tau: float, exact_x: bool = False):
    """(act, S) float64 [n_pairs, n_ff]: swiglu_clamp of the gate and up
    projections of moe_ref, with the tolerance scale carried through it.

    A device result computes the projections within tau*S_g and tau*S_u of
    the exact ones, then the epilogue in f32.  The clamps are 1-Lipschitz and
    silu is SILU_LIPSCHITZ-Lipschitz, so with gc, uc the clamped exact
    projections and s = silu(gc):
        |act' - act| <= tau*(SILU_LIPSCHITZ*|uc|*S_g + |s|*S_u)
                        + SILU_LIPSCHITZ*tau^2*S_g*S_u + (f32 epilogue rounding),
    the last at most 8 f32 ulps of |act| (exp, add, divide, multiply).  S is
    that bound divided by tau, so |act' - act| <= tau*S is the pass test."""
    g, u, Sg, Su = moe_ref(name, w_gate, w_up, ids, scales, x, n_expert, in_f, n_ff, exact_x=exact_x)
    gc = np.minimum(g, limit)
    uc = np.maximum(np.minimum(u, limit), -limit)
    with np.errstate(over="ignore"):
        s = gc / (1.0 + np.exp(-gc))
    act = s * uc
    S = (SILU_LIPSCHITZ * np.abs(uc) * Sg + np.abs(s) * Su + SILU_LIPSCHITZ * tau * Sg * Su
         + 2.0 ** -20 * np.abs(act) / tau)
    return act, S


def quantize_q8_1(x, k: int):
    """Q8_1 activations (memra `moe_rows_ceiling_bench.rs` quantizes x with
    quantize_q8_1 before the served kernel; the pages name the ggml format
    without printing it, so this is a reading): per block of 32 consecutive
    activations of a row, d = max|x| / 127 and q = round-half-away-from-zero
    of x * (1/d) (q = 0 when d = 0), every step in float32 as the device does
    it, since these decide the integer codes.  Returns (q int8 [rows, k],
    d float32 [rows, k/32])."""
    X = np.asarray(x, dtype=np.float32).reshape(-1, k // 32, 32)
    amax = np.max(np.abs(X), axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d != 0, d, np.float32(1.0)).astype(np.float32)
    inv = np.where(d != 0, np.float32(1.0) / safe, np.float32(0.0)).astype(np.float32)
    v = (X * inv[..., None]).astype(np.float32).astype(np.float64)
    q = np.trunc(v + np.copysign(0.5, v))
    assert np.all(np.abs(q) <= 127)
    return q.astype(np.int8).reshape(-1, k), d


def dequantize_q8_1(q, d, k: int):
    """x_hat = d[block] * q (exact in float64)."""
    Q = np.asarray(q, dtype=np.int64).reshape(-1, k // 32, 32).astype(np.float64)
    D = np.asarray(d, dtype=np.float32).reshape(-1, k // 32, 1).astype(np.float64)
    return (Q * D).reshape(-1, k)


def moe_q8_ref(name: str, w_gate, w_up, ids, scales, xq, xd, n_expert: int, in_f: int, n_ff: int):
    """The gate/up projections of Q8_1 activations: moe_ref applied to the
    dequantized activations d*q (what the integer group dot products, scaled
    by the group and block scales, compute).  (gate, up, S_gate, S_up)."""
    xh = dequantize_q8_1(xq, xd, in_f)
    return moe_ref(name, w_gate, w_up, ids, scales, xh, n_expert, in_f, n_ff, exact_x=True)


def moe_down_q8_ref(name: str, w_down, ids, scales, aq, ad, n_expert: int, n_ff: int, d_model: int):
    """The down projection of Q8_1 pair activations (the memra page's down
    arm quantizes each pair's activation row with quantize_q8_1 before
    moe_down8_fma_q8_rows): moe_down_ref on the dequantized rows d*q.
    (y, S_y, pair, S_pair)."""
    ah = dequantize_q8_1(aq, ad, n_ff)
    return moe_down_ref(name, w_down, ids, scales, ah, n_expert, n_ff, d_model, exact_act=True)


def tolerance_check(got, ref, S, tau: float):
    """(ok, worst) where worst = max |got - ref| / (tau * S) over the outputs
    (a ratio <= 1 passes).  Any non-finite value in ``got`` fails outright:
    a max over NaN would otherwise hide every mismatch (cera
    `wgpu_gemm_bench.rs`, the non-finite guard before the relative error)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    s = np.asarray(S, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if not np.all(np.isfinite(g)):
        return False, float("inf")
    err = np.abs(g - r)
    bound = tau * s
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(worst <= 1.0), worst
