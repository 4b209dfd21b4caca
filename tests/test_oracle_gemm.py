"""Pins for the oracle's reference GEMM / MoE and the tolerance check.

- identity activations reduce the GEMM to the decoder: ref[j, i] = W[i, j]
- tiny shapes: brute force with exactly rounded sums (math.fsum) over the
  literal decoder
- invariants: row permutation of x, linearity, S >= |ref|
- MoE: brute force per pair; renaming experts together with their weights
  leaves the outputs unchanged
- MoE down: brute force per token (pair activations, slot sum by fsum); one
  slot per token reduces it to a gate/up plane; expert renaming and slot
  order leave it unchanged
- planted mistakes (in the oracle, on the CPU) are caught by these pins
"""

import numpy as np
import pytest

import encoders as enc
from oracle import formats, ref, scalar
from synth import gen

QTS = ["f32", "q4_0", "q8_0", "q4_k", "q6_k", "nvfp4"]


def _weights(qt, m, k, seed):
    if qt == "f32":
        return gen.unit_f32(m * k, seed)
    if qt == "nvfp4":
        return gen.nvfp4_rows(m, k, seed)
    return gen.quant_bytes(m * formats.row_bytes(qt, k), seed)


@pytest.mark.parametrize("qt", QTS)
def test_identity_activations_return_weights(qt):
    m, k = 5, formats.block_elems(qt) if qt != "f32" else 64
    k = max(k, 64)
    w = _weights(qt, m, k, 3)
    x = np.eye(k, dtype=np.float32)
    r, S = ref.gemm_ref(qt, w, x, m, k, k)
    W = formats.decode(qt, w, m, k)
    assert np.array_equal(r, W.T)
    assert np.array_equal(S, np.abs(W.T))


@pytest.mark.parametrize("qt", QTS)
def test_tiny_shapes_brute_force(qt):
    k = max(formats.block_elems(qt), 32)
    for m in (1, 2, 3):
        for n in (1, 2, 3):
            w = _weights(qt, m, k, 17 + m)
            x = gen.unit_f32(n * k, 23 + n).reshape(n, k)
            r, S = ref.gemm_ref(qt, w, x, m, k, n)
            bf = np.array(scalar.gemm(qt, bytes(np.asarray(w).view(np.uint8)), x.tolist(), m, k, n))
            # f64 matmul vs exactly rounded sum: differ by f64 rounding only
            assert np.all(np.abs(r - bf) <= 1e-12 * S + 1e-300)


def test_invariants_permutation_linearity():
    qt, m, k, n = "q4_k", 16, 512, 6
    w = _weights(qt, m, k, 5)
    x = gen.unit_f32(n * k, 6).reshape(n, k)
    r, S = ref.gemm_ref(qt, w, x, m, k, n)
    perm = np.array([3, 0, 5, 1, 4, 2])
    rp, _ = ref.gemm_ref(qt, w, x[perm], m, k, n)
    assert np.array_equal(rp, r[perm])
    y = gen.unit_f32(n * k, 7).reshape(n, k)
    ry, _ = ref.gemm_ref(qt, w, y, m, k, n)
    rs, _ = ref.gemm_ref(qt, w, (x + y).astype(np.float64).astype(np.float32), m, k, n)
    # x + y is exact in f32 here (both on a 2^-15 grid in [-1, 1))
    assert np.allclose(rs, r + ry, rtol=0, atol=1e-9)
    assert np.all(S >= np.abs(r))


def test_sampled_rows_equal_full():
    qt, m, k, n = "q6_k", 40, 512, 9
    w = _weights(qt, m, k, 8)
    x = gen.unit_f32(n * k, 9).reshape(n, k)
    r, S = ref.gemm_ref(qt, w, x, m, k, n)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, m, 50)
    cols = rng.integers(0, n, 50)
    rr, ss = ref.gemm_ref_rows(qt, w, x, m, k, rows, cols, formats.row_bytes(qt, k))
    assert np.allclose(rr, r[cols, rows], rtol=1e-14, atol=0)
    assert np.allclose(ss, S[cols, rows], rtol=1e-14, atol=0)


def test_moe_ref_brute_force_and_expert_renaming():
    n_expert, in_f, n_ff, t, n_used = 6, 128, 8, 3, 2
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, 5)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, 91)
    g, u, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    per = n_ff * formats.row_bytes("nvfp4", in_f)
    n_pairs = t * n_used
    for tau in range(t):
        for s in range(n_used):
            p = tau * n_used + s
            e = ids[tau, s]
            for plane, wp, out in ((0, wg, g), (1, wu, u)):
                blk = bytes(wp[e * per:(e + 1) * per])
                bf = scalar.gemm("nvfp4", blk, [x[tau * in_f:(tau + 1) * in_f].tolist()], n_ff, in_f, 1)[0]
                assert np.allclose(out[p], np.float64(sc[plane * n_pairs + p]) * np.array(bf),
                                   rtol=1e-13, atol=1e-13)
    # rename experts: permute the weight slabs and map the ids through the same permutation
    perm = np.array([4, 2, 0, 5, 1, 3])          # new slot of old expert e is perm[e]
    inv = np.argsort(perm)
    wg2 = np.concatenate([wg[inv[s] * per:(inv[s] + 1) * per] for s in range(n_expert)])
    wu2 = np.concatenate([wu[inv[s] * per:(inv[s] + 1) * per] for s in range(n_expert)])
    g2, u2, _, _ = ref.moe_ref("nvfp4", wg2, wu2, perm[ids], sc, x, n_expert, in_f, n_ff)
    assert np.array_equal(g2, g) and np.array_equal(u2, u)


def test_moe_sampled_rows_equal_brute_force():
    """The sampled MoE reference against the literal scalar decoder + fsum."""
    n_expert, in_f, n_ff, t, n_used = 5, 128, 6, 4, 3
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, 11)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, 91)
    per = n_ff * formats.row_bytes("nvfp4", in_f)
    n_pairs = t * n_used
    pairs = np.array([0, 5, 11, 7, 3])
    rows = np.array([0, 5, 2, 3, 1])
    for plane in (0, 1):
        val, tol = ref.moe_ref_pairs_rows("nvfp4", wg, ids, sc, x, plane, n_expert, in_f, n_ff,
                                          pairs, rows)
        for i, (p, r) in enumerate(zip(pairs, rows)):
            e = ids.reshape(-1)[p]
            blk = bytes(wg[e * per:(e + 1) * per])
            xt = x[(p // n_used) * in_f:(p // n_used + 1) * in_f].tolist()
            bf = scalar.gemm("nvfp4", blk, [xt], n_ff, in_f, 1)[0][r]
            f = np.float64(sc[plane * n_pairs + p])
            assert abs(val[i] - f * bf) <= 1e-12 * max(1.0, abs(f * bf))
            assert tol[i] >= abs(val[i])


def _down_case(n_expert=5, n_ff=128, d_model=6, t=3, n_used=2, seed=7):
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, 0x4242 + e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, seed)
    sc = gen.pair_scales(t * n_used)
    act = gen.xorshift_f32(t * n_used * n_ff, 1234)
    return wd, ids, sc, act


def test_moe_down_ref_brute_force():
    """y[tau, r] against the literal scalar decoder: each pair's own
    activation row and scale, the token's slots summed exactly (fsum)."""
    import math
    n_expert, n_ff, d_model, t, n_used = 5, 128, 6, 3, 2
    wd, ids, sc, act = _down_case(n_expert, n_ff, d_model, t, n_used)
    y, S, pair, pair_S = ref.moe_down_ref("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model)
    per = d_model * formats.row_bytes("nvfp4", n_ff)
    for tau in range(t):
        terms = [[] for _ in range(d_model)]
        for s in range(n_used):
            p = tau * n_used + s
            e = ids[tau, s]
            blk = bytes(wd[e * per:(e + 1) * per])
            a = act[p * n_ff:(p + 1) * n_ff].tolist()
            bf = scalar.gemm("nvfp4", blk, [a], d_model, n_ff, 1)[0]
            for r in range(d_model):
                terms[r].append(float(np.float64(sc[p])) * bf[r])
                assert abs(pair[p, r] - terms[r][-1]) <= 1e-12 * max(1.0, abs(terms[r][-1]))
        for r in range(d_model):
            want = math.fsum(terms[r])
            assert abs(y[tau, r] - want) <= 1e-12 * max(1.0, sum(abs(v) for v in terms[r]))
            assert S[tau, r] >= abs(y[tau, r])


def test_moe_down_ref_special_cases():
    """One slot per token reduces the down projection to the gate/up plane
    with the pair's activation as the token row; renaming experts with their
    weights and permuting the slots of a token leave y unchanged."""
    n_expert, n_ff, d_model, t = 4, 64, 5, 3
    wd, ids1, sc1, act1 = _down_case(n_expert, n_ff, d_model, t, 1, seed=3)
    y, _, _, _ = ref.moe_down_ref("nvfp4", wd, ids1, sc1, act1, n_expert, n_ff, d_model)
    g, _, _, _ = ref.moe_ref("nvfp4", wd, wd, ids1, np.concatenate([sc1, sc1]), act1, n_expert,
                             n_ff, d_model)
    assert np.allclose(y, g, rtol=1e-13, atol=1e-13)
    n_used = 3
    wd, ids, sc, act = _down_case(n_expert, n_ff, d_model, t, n_used, seed=9)
    y, S, _, _ = ref.moe_down_ref("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model)
    per = d_model * formats.row_bytes("nvfp4", n_ff)
    perm = np.array([2, 0, 3, 1])
    inv = np.argsort(perm)
    wd2 = np.concatenate([wd[inv[e] * per:(inv[e] + 1) * per] for e in range(n_expert)])
    y2, _, _, _ = ref.moe_down_ref("nvfp4", wd2, perm[ids], sc, act, n_expert, n_ff, d_model)
    assert np.array_equal(y2, y)
    # reverse the slots of every token (ids, scales and activation rows move together)
    order = np.concatenate([tau * n_used + np.arange(n_used)[::-1] for tau in range(t)])
    y3, S3, _, _ = ref.moe_down_ref("nvfp4", wd, ids[:, ::-1].copy(), sc[order],
                                    act.reshape(t * n_used, n_ff)[order].reshape(-1), n_expert,
                                    n_ff, d_model)
    assert np.allclose(y3, y, rtol=1e-13, atol=1e-13) and np.allclose(S3, S, rtol=1e-13)


def test_moe_down_sampled_rows_equal_full():
    n_expert, n_ff, d_model, t, n_used = 5, 128, 7, 4, 3
    wd, ids, sc, act = _down_case(n_expert, n_ff, d_model, t, n_used, seed=21)
    y, S, _, _ = ref.moe_down_ref("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model)
    toks = np.array([0, 3, 2, 1, 3])
    rows = np.array([0, 6, 3, 5, 0])
    val, tol = ref.moe_down_ref_rows("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model, toks, rows)
    assert np.allclose(val, y[toks, rows], rtol=1e-12, atol=1e-12)
    assert np.allclose(tol, S[toks, rows], rtol=1e-12, atol=1e-12)


def test_quantize_q8_1_pins():
    """Q8_1 quantization: exactly representable blocks come back exactly;
    halves round away from zero (not to even); a zero block gives d = q = 0;
    the block maximum maps to +-127; |x - d*q| <= d/2 otherwise."""
    k = 96
    # block 0: x = d0 * c with d0 = 2^-6 and max |c| = 127 -> (c, d0) exactly
    c = np.arange(-127, 129, 8)[:32].astype(np.float64)
    c[5] = 127
    blk0 = (c * 2.0 ** -6).astype(np.float32)
    # block 1: amax 127 -> d = 1, id = 1: values +-2.5 and +-0.5 sit on halves
    blk1 = np.zeros(32, np.float32)
    blk1[:6] = [127.0, 2.5, -2.5, 0.5, -0.5, 3.5]
    blk2 = np.zeros(32, np.float32)
    x = np.concatenate([blk0, blk1, blk2])
    q, d = ref.quantize_q8_1(x, k)
    assert d[0, 0] == np.float32(2.0 ** -6) and np.array_equal(q[0, :32], c.astype(np.int8))
    assert d[0, 1] == 1.0 and list(q[0, 32:38]) == [127, 3, -3, 1, -1, 4]
    assert d[0, 2] == 0.0 and not q[0, 64:].any()
    rng = np.random.default_rng(3)
    xr = (rng.standard_normal(4 * 256) * rng.choice([1e-3, 1.0, 50.0], 4 * 256)).astype(np.float32)
    q, d = ref.quantize_q8_1(xr, 256)
    X = xr.reshape(4, 8, 32).astype(np.float64)
    Q = q.reshape(4, 8, 32).astype(np.int64)
    D = d.reshape(4, 8, 1).astype(np.float64)
    am = np.argmax(np.abs(X), axis=2)
    assert np.all(np.abs(np.take_along_axis(Q, am[..., None], 2)) == 127)
    assert np.all(np.abs(X - D * Q) <= D / 2 * (1 + 1e-6))
    assert np.array_equal(ref.dequantize_q8_1(q, d, 256), (D * Q).reshape(4, 256))


def test_moe_q8_ref_brute_force():
    """Gate/up of Q8_1 activations against the literal decoder with the group
    dot products summed as exact integers (2 * E2M1 codes times int8 codes)."""
    from fractions import Fraction
    n_expert, in_f, n_ff, t, n_used = 4, 128, 5, 2, 2
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, 5)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, 91)
    xq, xd = ref.quantize_q8_1(x, in_f)
    g, u, Sg, Su = ref.moe_q8_ref("nvfp4", wg, wu, ids, sc, xq, xd, n_expert, in_f, n_ff)
    per = n_ff * formats.row_bytes("nvfp4", in_f)
    rb = formats.row_bytes("nvfp4", in_f)
    n_pairs = t * n_used
    for tau in range(t):
        for s in range(n_used):
            p = tau * n_used + s
            e = int(ids[tau, s])
            for plane, wp, out in ((0, wg, g), (1, wu, u)):
                for r in range(n_ff):
                    row = bytes(wp[e * per + r * rb:e * per + (r + 1) * rb])
                    tot = Fraction(0)
                    for b in range(in_f // 32):
                        for h in range(2):          # the two 16-element scale groups
                            isum = 0
                            for i in range(16):
                                c = 32 * b + 16 * h + i
                                w2 = scalar.element("nvfp4", row, c) / scalar.fp8_e4m3(row[(c // 64) * 36 + (c % 64) // 16])
                                isum += int(round(2 * w2)) * int(xq[tau, c])
                            gs = row[(32 * b + 16 * h) // 64 * 36 + ((32 * b + 16 * h) % 64) // 16]
                            tot += Fraction(isum) * Fraction(scalar.fp8_e4m3(gs)) / 2 * Fraction(float(xd[tau, b]))
                    want = float(tot * Fraction(float(sc[plane * n_pairs + p])))
                    assert abs(out[p, r] - want) <= 1e-13 * max(1.0, abs(want))


def test_tolerance_check_semantics():
    r = np.array([[1.0, -2.0]])
    S = np.array([[1.0, 2.0]])
    assert ref.tolerance_check(r, r, S, 1e-5) == (True, 0.0)
    ok, worst = ref.tolerance_check(r + np.array([[0.9e-5, 0]]), r, S, 1e-5)
    assert ok and 0.89 < worst < 0.91
    ok, _ = ref.tolerance_check(r + np.array([[2e-5, 0]]), r, S, 1e-5)
    assert not ok
    ok, worst = ref.tolerance_check(np.array([[np.nan, -2.0]]), r, S, 1e-5)
    assert not ok and worst == float("inf")
    # zero tolerance scale: only an exact match passes
    assert ref.tolerance_check(np.array([0.0]), np.array([0.0]), np.array([0.0]), 1e-5)[0]
    assert not ref.tolerance_check(np.array([1e-30]), np.array([0.0]), np.array([0.0]), 1e-5)[0]


# ------------------------------------------------------------ planted mistakes


def _q4k_roundtrip_ok(decode_fn):
    rng = np.random.default_rng(1)
    for _ in range(5):
        d, dmin = 0x3C00, 0x3800
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        blk = np.frombuffer(enc.q4_k(d, dmin, sc, mn, q), np.uint8)
        j = np.arange(256) // 32
        want = 1.0 * sc[j] * q - 0.5 * mn[j]
        if not np.array_equal(decode_fn("q4_k", blk, 1, 256)[0], want):
            return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _q4k_roundtrip_ok(formats.decode)
    orig = formats._q4k_scale_min

    def swapped(sc):                       # min and scale swapped for j >= 4
        s, m = orig(sc)
        s2, m2 = s.copy(), m.copy()
        s2[..., 4:], m2[..., 4:] = m[..., 4:], s[..., 4:]
        return s2, m2
    monkeypatch.setattr(formats, "_q4k_scale_min", swapped)
    assert not _q4k_roundtrip_ok(formats.decode)
    monkeypatch.setattr(formats, "_q4k_scale_min", orig)

    # Q6_K with the qh bit pair of quarter 1 and 2 exchanged
    orig_codes = formats._q6k_codes

    def bad_codes(ql, qh):
        q = orig_codes(ql, qh)
        q2 = q.copy()
        q2[..., 32:64], q2[..., 64:96] = q[..., 64:96], q[..., 32:64]
        return q2
    monkeypatch.setattr(formats, "_q6k_codes", bad_codes)
    rng = np.random.default_rng(3)
    sc = rng.integers(-128, 128, 16)
    q = rng.integers(0, 64, 256)
    got = formats.decode("q6_k", np.frombuffer(enc.q6_k(0x3C00, sc, q), np.uint8), 1, 256)[0]
    assert not np.array_equal(got, sc[np.arange(256) // 16] * (q - 32.0))
    monkeypatch.setattr(formats, "_q6k_codes", orig_codes)

    # f16 decoder that drops the sign: the golden -1.0 code no longer matches
    orig_f16 = formats.f16_bits_to_f64
    monkeypatch.setattr(formats, "f16_bits_to_f64", lambda b: np.abs(orig_f16(b)))
    data = np.frombuffer(enc.q4_0(0xBC00, list(range(16)) * 2), np.uint8)
    got = formats.decode("q4_0", data, 1, 32)[0]
    assert not np.array_equal(got, -1.0 * (np.array(list(range(16)) * 2) - 8.0))


@pytest.mark.parametrize("qt", QTS)
def test_gemm_value_brute_force(qt):
    """gemm_value (the function the CPU baseline times) against the literal
    scalar decoder with exactly rounded sums, on tiny shapes that span
    several blocks; and equal to gemm_ref's value on a larger shape."""
    import math
    k = 2 * max(formats.block_elems(qt), 32)
    for m, n in ((1, 1), (3, 2), (2, 5)):
        w = _weights(qt, m, k, 41 + m)
        x = gen.unit_f32(n * k, 43 + n).reshape(n, k)
        v = ref.gemm_value(qt, w, x, m, k, n)
        data = bytes(np.asarray(w).view(np.uint8))
        W = scalar.decode_matrix(qt, data, m, k)
        bf = np.array(scalar.gemm(qt, data, x.tolist(), m, k, n))
        S = np.array([[math.fsum(abs(W[i][c] * float(x[j][c])) for c in range(k)) for i in range(m)]
                      for j in range(n)])
        assert v.shape == (n, m)
        assert np.all(np.abs(v - bf) <= 1e-12 * S + 1e-300)
    m, k, n = 37, 4 * max(formats.block_elems(qt), 64), 11
    w = _weights(qt, m, k, 47)
    x = gen.unit_f32(n * k, 48).reshape(n, k)
    r, _ = ref.gemm_ref(qt, w, x, m, k, n)
    assert np.array_equal(ref.gemm_value(qt, w, x, m, k, n), r)


@pytest.mark.parametrize("qt", ["q4_k", "q6_k", "nvfp4", "f32"])
def test_gemm_ref_blocks_cover_the_whole_output(qt):
    """The row-blocked reference (whole outputs of large shapes) tiles the
    full one: every row block equals the same rows of gemm_ref, blocks in
    order with a ragged last block."""
    m, k, n = 300, 2 * max(formats.block_elems(qt), 64), 7
    w = _weights(qt, m, k, 51)
    x = gen.unit_f32(n * k, 52).reshape(n, k)
    r, S = ref.gemm_ref(qt, w, x, m, k, n)
    seen = 0
    for i0, i1, rb_, sb in ref.gemm_ref_blocks(qt, w, x, m, k, n, formats.row_bytes(qt, k), 128):
        assert i0 == seen and i1 - i0 == min(128, m - i0)
        assert np.allclose(rb_, r[:, i0:i1], rtol=1e-14, atol=1e-300)
        assert np.allclose(sb, S[:, i0:i1], rtol=1e-14, atol=1e-300)
        seen = i1
    assert seen == m


def test_moe_pairs_rows_exact_x_branch():
    """moe_ref_pairs_rows with exact_x (the reference of the Q8_1 gate/up at
    full size) uses the float64 activations as given: against the full
    moe_q8_ref on the same pairs, and against the literal decoder with
    activations that float32 cannot hold (x = q/3), where the float32 branch
    would differ."""
    n_expert, in_f, n_ff, t, n_used = 5, 128, 6, 3, 2
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, 13)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, 91)
    xq, xd = ref.quantize_q8_1(x, in_f)
    g, u, Sg, Su = ref.moe_q8_ref("nvfp4", wg, wu, ids, sc, xq, xd, n_expert, in_f, n_ff)
    xh = ref.dequantize_q8_1(xq, xd, in_f)
    n_pairs = t * n_used
    pairs = np.repeat(np.arange(n_pairs), n_ff)
    rows = np.tile(np.arange(n_ff), n_pairs)
    for plane, wp, full, Sfull in ((0, wg, g, Sg), (1, wu, u, Su)):
        val, tol = ref.moe_ref_pairs_rows("nvfp4", wp, ids, sc, xh, plane, n_expert, in_f, n_ff,
                                          pairs, rows, exact_x=True)
        assert np.allclose(val, full[pairs, rows], rtol=1e-13, atol=1e-300)
        assert np.allclose(tol, Sfull[pairs, rows], rtol=1e-13, atol=1e-300)
    # activations off the float32 grid: exact_x keeps them, float32 rounds them
    rng = np.random.default_rng(3)
    x3 = rng.integers(-300, 301, (t, in_f)) / 3.0
    per = n_ff * formats.row_bytes("nvfp4", in_f)
    p, r = 3, 4
    e = int(ids.reshape(-1)[p])
    row = bytes(wg[e * per:(e + 1) * per])
    want = float(np.float64(sc[p])) * float(np.dot(scalar.decode_matrix("nvfp4", row, n_ff, in_f)[r],
                                                   x3[p // n_used]))
    v64, _ = ref.moe_ref_pairs_rows("nvfp4", wg, ids, sc, x3, 0, n_expert, in_f, n_ff, [p], [r], exact_x=True)
    v32, _ = ref.moe_ref_pairs_rows("nvfp4", wg, ids, sc, x3, 0, n_expert, in_f, n_ff, [p], [r])
    assert abs(v64[0] - want) <= 1e-12 * max(1.0, abs(want))
    assert abs(v32[0] - want) > 1e-9 * max(1.0, abs(want))


# ------------------------------------------------------------ SwiGLU/clamp epilogue

def test_swiglu_clamp_closed_forms_and_clamp_edges():
    """Values fixed by the definition: silu(0) = 0; the logistic function
    at 1 is 0.7310585786300049 (and 1 - that at -1); the gate clamp is
    flat above L and the up clamp flat outside [-L, L]; NaN stays NaN; a
    very negative gate gives -0, not NaN; limit = inf is plain SwiGLU."""
    L = 7.0
    f = ref.swiglu_clamp
    assert f(0.0, 3.0, L) == 0.0
    assert abs(f(1.0, 1.0, L) - 0.7310585786300049) <= 1e-16
    assert abs(f(-1.0, 1.0, L) - (-1.0) * (1.0 - 0.7310585786300049)) <= 1e-16
    top = f(L, 1.0, L)
    for g in (L, L + 1e-9, 8.0, 50.0, 1e30):
        assert f(g, 1.0, L) == top                       # gate clamped above at L
    assert f(L - 1e-3, 1.0, L) < top
    for u, want in ((L, L), (L + 0.5, L), (1e30, L), (-L, -L), (-L - 0.5, -L), (-1e30, -L), (3.0, 3.0)):
        assert f(2.0, u, L) == f(2.0, 1.0, L) * want     # up clamped to [-L, L]
    assert f(-1e9, 5.0, L) == 0.0 and not np.isnan(f(-1e9, 5.0, L))
    assert np.isnan(f(np.nan, 1.0, L)) and np.isnan(f(1.0, np.nan, L))
    assert f(10.0, 10.0, np.inf) == f(10.0, 1.0, np.inf) * 10.0
    assert f(10.0, 10.0, np.inf) > f(10.0, 10.0, L)


def test_swiglu_silu_matches_library_logistic():
    """silu(z) = z * expit(z) with scipy's logistic function (a library
    routine independent of the oracle's expression), for |z| up to 40."""
    from scipy.special import expit
    rng = np.random.default_rng(4)
    z = np.concatenate([rng.uniform(-40, 40, 5000), np.linspace(-8, 8, 1601)])
    got = ref.swiglu_clamp(z, np.ones_like(z), np.inf)
    want = z * expit(z)
    assert np.all(np.abs(got - want) <= 4e-16 * np.maximum(1.0, np.abs(want)))


def test_silu_lipschitz_bound_is_tight():
    """The derivative sigma(z)(1 + z(1 - sigma(z))) stays within
    +-SILU_LIPSCHITZ, and its extremes come within 0.1% of it."""
    from scipy.special import expit
    z = np.linspace(-60, 60, 1200001)
    s = expit(z)
    d = s * (1 + z * (1 - s))
    assert np.max(np.abs(d)) < ref.SILU_LIPSCHITZ
    assert np.max(np.abs(d)) > 0.999 * 1.0998


def _act_case(t=3, n_used=2, n_expert=5, in_f=128, n_ff=7, seed=5):
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, 0x8181 + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, seed)
    sc = gen.pair_scales(2 * t * n_used) * 20.0        # large enough that the clamps act
    x = gen.xorshift_f32(t * in_f, 91)
    return wg, wu, ids, sc.astype(np.float32), x


def test_moe_act_ref_brute_force():
    """act against the literal scalar decoder, exactly rounded sums and
    math.exp, pair by pair; the scales make some projections exceed L."""
    import math
    n_expert, in_f, n_ff, t, n_used = 5, 128, 7, 3, 2
    wg, wu, ids, sc, x = _act_case(t, n_used, n_expert, in_f, n_ff)
    L = 7.0
    act, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, L, 1e-5)
    per = n_ff * formats.row_bytes("nvfp4", in_f)
    n_pairs = t * n_used
    clamped = 0
    for p in range(n_pairs):
        tau_, e = p // n_used, int(ids.reshape(-1)[p])
        xt = [float(v) for v in x[tau_ * in_f:(tau_ + 1) * in_f]]
        Wg = scalar.decode_matrix("nvfp4", bytes(wg[e * per:(e + 1) * per]), n_ff, in_f)
        Wu = scalar.decode_matrix("nvfp4", bytes(wu[e * per:(e + 1) * per]), n_ff, in_f)
        for r in range(n_ff):
            g = float(sc[p]) * math.fsum(a * b for a, b in zip(Wg[r], xt))
            u = float(sc[n_pairs + p]) * math.fsum(a * b for a, b in zip(Wu[r], xt))
            clamped += (g > L) + (abs(u) > L)
            gc, uc = min(g, L), max(-L, min(u, L))
            want = gc / (1.0 + math.exp(-gc)) * uc
            assert abs(act[p, r] - want) <= 1e-12 * max(1.0, abs(want))
            assert S[p, r] >= 0.0
    assert clamped > 0


def test_moe_act_tolerance_covers_worst_perturbations():
    """The propagated tolerance: projections moved by up to tau*S_g and
    tau*S_u (every sign combination, and random interior points) and the
    epilogue then evaluated in float32 stay within tau*S_act of the exact
    activation.  A planted mistake (the S_u term dropped) is caught."""
    n_expert, in_f, n_ff, t, n_used = 5, 128, 7, 3, 2
    wg, wu, ids, sc, x = _act_case(t, n_used, n_expert, in_f, n_ff)
    tau, L = 1e-5, 7.0
    g, u, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    act, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, L, tau)

    def epi32(gv, uv):
        g32, u32 = gv.astype(np.float32), uv.astype(np.float32)
        L32 = np.float32(L)
        gc = np.minimum(g32, L32)
        uc = np.maximum(np.minimum(u32, L32), -L32)
        with np.errstate(over="ignore"):
            return (gc / (np.float32(1) + np.exp(-gc)) * uc).astype(np.float64)

    rng = np.random.default_rng(8)
    worst = 0.0
    for a in (-1.0, 1.0):
        for b in (-1.0, 1.0):
            for _ in range(3):
                ga = g + a * tau * Sg * rng.uniform(0.5, 1.0, g.shape)
                ub = u + b * tau * Su * rng.uniform(0.5, 1.0, u.shape)
                err = np.abs(epi32(ga, ub) - act)
                assert np.all(err <= tau * S), float(np.max(err / (tau * S)))
                worst = max(worst, float(np.max(err / (tau * S))))
    assert worst > 0.05                              # the bound is not vacuous
    # the bound without the up term does not cover moving u alone
    s = np.minimum(g, L) / (1 + np.exp(-np.minimum(g, L)))
    S_bad = S - np.abs(s) * Su
    err = np.abs(epi32(g, u + tau * Su) - act)
    assert np.any(err > tau * S_bad)


def test_moe_down_q8_ref_brute_force():
    """Down projection of Q8_1 pair activations against the literal decoder
    with exact rational sums: y[tau, r] = sum_s scale[p] * sum_c Wd[r, c] *
    d_p[c/32] * q_p[c]."""
    from fractions import Fraction
    n_expert, n_ff, d_model, t, n_used = 4, 128, 5, 2, 2
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, 0x4242 + e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, 9)
    sc = gen.pair_scales(t * n_used)
    act = gen.xorshift_f32(t * n_used * n_ff, 1234)
    aq, ad = ref.quantize_q8_1(act, n_ff)
    y, S, pair, pS = ref.moe_down_q8_ref("nvfp4", wd, ids, sc, aq, ad, n_expert, n_ff, d_model)
    per = d_model * formats.row_bytes("nvfp4", n_ff)
    for tau_ in range(t):
        for r in range(d_model):
            tot = Fraction(0)
            for s_ in range(n_used):
                p = tau_ * n_used + s_
                e = int(ids[tau_, s_])
                W = scalar.decode_matrix("nvfp4", bytes(wd[e * per:(e + 1) * per]), d_model, n_ff)[r]
                dot = sum(Fraction(W[c]) * Fraction(float(ad[p, c // 32])) * int(aq[p, c]) for c in range(n_ff))
                tot += Fraction(float(sc[p])) * dot
            assert abs(y[tau_, r] - float(tot)) <= 1e-13 * max(1.0, abs(float(tot)))
            assert S[tau_, r] >= abs(y[tau_, r]) * (1 - 1e-12)
