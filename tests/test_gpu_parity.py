"""GPU parity: the HIP path against the CPU oracle, through the C-ABI.

Small shapes that span several tiles and ragged tails are compared element
by element over the whole output; exact-structured inputs must match bit for
bit on both paths; identity activations pin the output layout; repeated runs
must be bit-identical; guard bands around dst must stay untouched.
"""

import numpy as np
import pytest

from gpu_helpers import (TAU_F16, TAU_F32, acts, assert_f16_weights, check_full, exact_weights, gpu_gemm, note,
                         to_dev, weights)
from oracle import formats, ref
from synth import gen

pytestmark = pytest.mark.gpu

QTS = ["f32", "q4_0", "q8_0", "q4_k", "q6_k", "nvfp4"]

# (m, k) per format: ragged m, several units per row, odd unit counts / tails
GEMV_SHAPES = {
    "f32": [(67, 292), (300, 1024)],
    "q4_0": [(67, 1184), (300, 1024)],
    "q8_0": [(67, 1184), (300, 1024)],
    "q4_k": [(67, 1280), (300, 1024)],
    "q6_k": [(67, 1280), (300, 1024)],
    "nvfp4": [(67, 1216), (300, 1024)],
}


@pytest.mark.parametrize("path", ["gemv_fma", "gemv_matrix"])
@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 13, 32])
def test_gemv_parity(qt, n, path):
    """Both streams of the f32 decode path (products on FMAs, or on
    v_mfma_f32_4x4x1f32 with token groups of 4 or 8) at every n; the shapes
    leave the last row group and the last unit iteration of a row ragged."""
    for si, (m, k) in enumerate(GEMV_SHAPES[qt]):
        note(f"gemv {path} {qt} m={m} k={k} n={n}")
        w = weights(qt, m, k, si)
        x = acts(n, k, si)
        got = gpu_gemm(qt, w, x, m, path)
        check_full(qt, w, x, m, k, n, got, TAU_F32, f"{path} {qt} {m}x{k} n={n}")


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("n", [4, 8])
def test_gemv_matrix_long_rows(qt, n):
    """Long rows with few row groups: k = 8192, where four staged rows take
    one work group per CU and eight do not fit (n = 8 runs as two token
    groups of four), k = 4608 and k = 2048; with so few row groups 8 (4 for
    the 4 unit iterations of k = 2048 at 32 weights per unit) waves share each
    row group and add their partial sums in LDS."""
    import gemv_prefill_decode_amd as qmm
    for si, (m, k) in enumerate(((37, 8192), (1030, 8192), (600, 4608), (300, 2048))):
        note(f"gemv_matrix long rows {qt} m={m} k={k} n={n}")
        if k == 8192:
            assert qmm.gemm_plan(m, k, n, qt, "gemv_matrix")["tokens_per_pass"] == 4
        w = weights(qt, m, k, 60 + si)
        x = acts(n, k, 60 + si)
        got = gpu_gemm(qt, w, x, m, "gemv_matrix")
        check_full(qt, w, x, m, k, n, got, TAU_F32, f"gemv_matrix {qt} {m}x{k} n={n}")


@pytest.mark.parametrize("mfma_min", ["0", "1", "4"])
def test_moe_stream_choice(mfma_min):
    """The MoE projections with each choice of the chunks that run on the
    matrix-core stream (none; every chunk, also of one pair; chunks of four
    pairs only), in a process of its own since the choice is read once per
    process; every output against the oracle."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, QMM_MOE_MFMA_MIN=mfma_min)
    note(f"moe stream choice QMM_MOE_MFMA_MIN={mfma_min}")
    r = subprocess.run([sys.executable, os.path.join(here, "moe_env_check.py")], env=env, capture_output=True,
                       text=True, timeout=600)
    sys.stderr.write(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.count("OK ") == 4


MFMA_SHAPES = {
    "f32": [(300, 292, 33), (128, 1024, 200)],
    "q4_0": [(300, 1184, 33), (129, 1024, 257)],
    "q8_0": [(300, 1184, 33), (129, 1024, 257)],
    "q4_k": [(300, 1280, 33), (129, 1024, 257)],
    "q6_k": [(300, 1280, 33), (129, 1024, 257)],
    "nvfp4": [(300, 1216, 33), (129, 1024, 257)],
}


@pytest.mark.parametrize("qt", QTS)
def test_mfma_parity(qt):
    for si, (m, k, n) in enumerate(MFMA_SHAPES[qt]):
        note(f"mfma {qt} m={m} k={k} n={n}")
        w = weights(qt, m, k, 10 + si)
        x = acts(n, k, 10 + si)
        got = gpu_gemm(qt, w, x, m, "mfma")
        check_full(qt, w, x, m, k, n, got, TAU_F16, f"mfma {qt} {m}x{k} n={n}")


@pytest.mark.parametrize("qt", QTS)
def test_mfma_parity_no_workspace(qt):
    """The prefill kernel that converts f32 activations in its k loop (calls
    without a workspace)."""
    for si, (m, k, n) in enumerate(MFMA_SHAPES[qt]):
        note(f"mfma no-workspace {qt} m={m} k={k} n={n}")
        w = weights(qt, m, k, 10 + si)
        x = acts(n, k, 10 + si)
        got = gpu_gemm(qt, w, x, m, "mfma", workspace=None)
        check_full(qt, w, x, m, k, n, got, TAU_F16, f"mfma no-ws {qt} {m}x{k} n={n}")


@pytest.mark.parametrize("qt", QTS)
def test_mfma_paths_agree_bit_for_bit_unsplit(qt):
    """The LDS-ring kernel on the pre-pass's f16 activations and on the f32
    activations themselves (rounded as the operands are read) round x to f16
    the same way and order their k slots alike; unsplit and with the same k
    groups, their sums run in the same order, so the outputs are equal.  The
    kernel without a workspace orders the slots inside each matrix-core op
    differently: within tolerance only."""
    import os
    import gemv_prefill_decode_amd as qmm
    m, k, n = 512, 1024, 300
    note(f"mfma kernels agree {qt}")
    w = weights(qt, m, k, 50)
    x = acts(n, k, 50)
    a = gpu_gemm(qt, w, x, m, "mfma", workspace=None)
    check_full(qt, w, x, m, k, n, a, TAU_F16, f"agree {qt}")
    outs = []
    # 128- and 64-row tiles: each output's k sum runs in the same order
    for plan in ("2,2,1,1", "4,2,1,1", "2,1,1,1", "4,1,1,1"):
        os.environ["QMM_MFMA_PLAN"] = plan
        try:
            p = qmm.gemm_plan(m, k, n, qt, "mfma")
            assert p["x16"] == int(plan[0]) and p["n_split"] == 1, p
            outs.append(gpu_gemm(qt, w, x, m, "mfma"))
        finally:
            del os.environ["QMM_MFMA_PLAN"]
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)
    check_full(qt, w, x, m, k, n, outs[0], TAU_F16, f"agree lds ring {qt}")
    c = gpu_gemm(qt, w, x, m, "mfma")
    check_full(qt, w, x, m, k, n, c, TAU_F16, f"agree planned {qt}")


@pytest.mark.parametrize("qt", QTS)
def test_auto_dispatch_threshold(qt):
    """AUTO: the GEMV for every n <= 32 (the f32 path), the matrix-core path
    above; the result equals the forced path's bit for bit."""
    m, k = 130, 512
    w = weights(qt, m, k, 3)
    for n in (32, 33):
        note(f"auto {qt} {m}x{k} n={n}")
        x = acts(n, k, 3)
        got = gpu_gemm(qt, w, x, m, "auto")
        gv = gpu_gemm(qt, w, x, m, "gemv" if n <= 32 else "mfma")
        assert np.array_equal(got, gv)


@pytest.mark.parametrize("qt", ["q4_0", "q4_k", "q6_k", "f32"])
def test_qmm_gemm_entry_points_through_ctypes(qt):
    """qmm_gemm and qmm_gemm_path called through the C-ABI themselves (no
    binding wrapper) at n on both sides of the dispatch threshold, each
    result against the oracle at the tolerance of the path it takes (n <= 32:
    the f32 GEMV, 1e-5; above: the f16 matrix cores, 2e-3)."""
    import ctypes
    import torch
    import gemv_prefill_decode_amd as qmm
    lib = qmm.load()
    m, k = 300, 1024
    w = weights(qt, m, k, 31)
    dw = to_dev(w)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    qi = qmm.QTYPES[qt]
    for n in (8, 9, 16, 17, 32, 33):
        note(f"ctypes qmm_gemm {qt} n={n}")
        x = acts(n, k, 31 + n)
        dx = to_dev(x)
        tau = TAU_F32 if n <= 32 else TAU_F16
        out = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
        st = lib.qmm_gemm(out.data_ptr(), dw.data_ptr(), dx.data_ptr(), m, k, n, qi, s)
        torch.cuda.synchronize()
        assert st == 0, qmm.status_str(st)
        check_full(qt, w, x, m, k, n, out.cpu().numpy(), tau, f"qmm_gemm {qt} n={n}")
        for path, ptau in ((1, TAU_F32), (2, TAU_F16), (0, tau)):
            out2 = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
            st = lib.qmm_gemm_path(out2.data_ptr(), dw.data_ptr(), dx.data_ptr(), m, k, n, qi, path, s)
            torch.cuda.synchronize()
            assert st == 0, qmm.status_str(st)
            check_full(qt, w, x, m, k, n, out2.cpu().numpy(), ptau, f"qmm_gemm_path {qt} n={n} path={path}")
            if path == 0:
                assert torch.equal(out, out2)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_exact_structured_inputs(qt, path):
    """Power-of-two scales, small integer codes, x on a 1/16 grid: every
    product and partial sum is exact, so the GPU must equal the oracle bit
    for bit on both paths (f16 rounding included)."""
    m, k = 150, 512
    n = 8 if path == "gemv" else 70
    note(f"exact {qt} {path}")
    w = exact_weights(qt, m, k, 7)
    x = gen.structured_exact(n * k, 11).reshape(n, k)
    got = gpu_gemm(qt, w, x, m, path)
    r, _ = ref.gemm_ref(qt, w, x, m, k, n)
    assert np.array_equal(got.astype(np.float64), r)


@pytest.mark.parametrize("qt", QTS)
def test_identity_activations_mfma(qt):
    """x = I_k (n = k): dst[j, i] = f16(W[i, j]) exactly (each weight reaches
    the matrix cores rounded once, to nearest even, from its exact decoded
    value).  Pins the tile mapping of every weight row and k index into dst."""
    m, k = 130, 256
    note(f"identity mfma {qt}")
    w = weights(qt, m, k, 21)
    x = np.eye(k, dtype=np.float32)
    got = gpu_gemm(qt, w, x, m, "mfma")
    W = formats.decode(qt, w, m, k)
    assert_f16_weights(got, W)


# The LDS-ring kernel assigns k to operand slots per format and lays the f16
# activations out in the same order; identity activations and exact inputs
# pin that mapping bit for bit for both tile heights.
@pytest.mark.parametrize("plan", ["2,2,1", "2,4,1", "2,4,2", "3,2,1", "3,2,2", "2,2,1,2", "2,2,2,2", "3,2,1,2",
                                  "4,2,1", "4,2,2", "4,2,1,2", "2,1,1", "2,1,1,2", "4,1,1", "4,1,2,2"])
@pytest.mark.parametrize("qt", QTS)
def test_lds_ring_identity_and_exact(qt, plan, monkeypatch):
    import gemv_prefill_decode_amd as qmm
    if qt == "f32" and (plan.startswith("2,4") or plan.count(",") == 3):
        pytest.skip("not a plan the library runs for f32 weights")
    if plan == "3,2,1,2" and qt in ("q6_k", "q8_0"):
        pytest.skip("its LDS ring does not fit 160 KB")
    monkeypatch.setenv("QMM_MFMA_PLAN", plan)
    m, k = 300, 512
    assert qmm.gemm_plan(m, k, k, qt, "mfma")["x16"] == int(plan[0])
    note(f"lds ring identity {qt} {plan}")
    w = weights(qt, m, k, 23)
    x = np.eye(k, dtype=np.float32)
    got = gpu_gemm(qt, w, x, m, "mfma")
    W = formats.decode(qt, w, m, k)
    assert_f16_weights(got, W)
    note(f"lds ring exact {qt} {plan}")
    we = exact_weights(qt, m, k, 8)
    xe = gen.structured_exact(150 * k, 12).reshape(150, k)
    got = gpu_gemm(qt, we, xe, m, "mfma")
    r, _ = ref.gemm_ref(qt, we, xe, m, k, 150)
    assert np.array_equal(got.astype(np.float64), r)


@pytest.mark.parametrize("path", ["gemv_fma", "gemv_matrix"])
@pytest.mark.parametrize("qt", QTS)
def test_identity_windows_gemv(qt, path):
    """Sliding one-hot windows (n = 32 tokens, token j selects k index
    c0 + j): dst[j, i] = f32(W[i, c0 + j]) exactly on both f32 streams."""
    m, k = 70, 512
    note(f"identity {path} {qt}")
    w = weights(qt, m, k, 22)
    W = formats.decode(qt, w, m, k)
    for c0 in range(0, k, 32):
        x = np.zeros((32, k), dtype=np.float32)
        x[np.arange(32), c0 + np.arange(32)] = 1.0
        got = gpu_gemm(qt, w, x, m, path)
        want = W[:, c0:c0 + 32].T.astype(np.float32)
        assert np.array_equal(got, want), c0


@pytest.mark.parametrize("qt", ["q4_0", "q4_k", "q6_k"])
def test_gemv_single_row_equals_row_of_two(qt):
    """One activation row takes the packed-half products (q as an f16
    subnormal scaled by a power of two, one v_fma_mix_f32 each), two rows the
    widened-float ones; the scaling is exact for activations of normal size,
    so each output equals, bit for bit, the same row computed beside another."""
    for si, (m, k) in enumerate([(67, 1280), (300, 1024), (1030, 4096)]):
        note(f"gemv n=1 vs n=2 {qt} m={m} k={k}")
        w = weights(qt, m, k, 40 + si)
        x2 = acts(2, k, 40 + si)
        got1 = gpu_gemm(qt, w, x2[:1].copy(), m, "gemv")
        got1b = gpu_gemm(qt, w, x2[1:].copy(), m, "gemv")
        got2 = gpu_gemm(qt, w, x2, m, "gemv")
        assert np.array_equal(got1[0], got2[0]) and np.array_equal(got1b[0], got2[1]), (m, k)


@pytest.mark.parametrize("qt", QTS)
@pytest.mark.parametrize("n", [1, 2])
def test_gemv_long_rows(qt, n):
    """Rows of k = 14336: the staged activations leave room for one or two
    work groups per CU, which then run 8 waves each; fewer row groups than
    resident waves, and a ragged last work group at m = 301."""
    k = 14336
    for si, m in enumerate((301, 1030)):
        note(f"gemv long rows {qt} m={m} k={k} n={n}")
        w = weights(qt, m, k, 50 + si)
        x = acts(n, k, 50 + si)
        got = gpu_gemm(qt, w, x, m, "gemv")
        check_full(qt, w, x, m, k, n, got, TAU_F32, f"gemv {qt} {m}x{k} n={n}")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_deterministic_and_guard_bands(path):
    import torch
    import gemv_prefill_decode_amd as qmm
    qt, m, k = "q6_k", 260, 1024
    n = 5 if path == "gemv" else 90
    note(f"determinism {path}")
    w, x = to_dev(weights(qt, m, k, 4)), to_dev(acts(n, k, 4))
    pad = 1024
    buf = torch.full((2 * pad + n * m,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n * m].view(n, m)
    qmm.gemm(w, x, m, qt, out=out, path=path)
    first = out.clone()
    qmm.gemm(w, x, m, qt, out=out, path=path)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:pad] == 12345.0).all()) and bool((buf[pad + n * m:] == 12345.0).all())


def test_gemv_and_mfma_agree_within_tolerance():
    m, k, n = 200, 1024, 16
    for qt in QTS:
        note(f"cross-path {qt}")
        w = weights(qt, m, k, 30)
        x = acts(n, k, 30)
        a = gpu_gemm(qt, w, x, m, "gemv")
        b = gpu_gemm(qt, w, x, m, "mfma")
        _, S = ref.gemm_ref(qt, w, x, m, k, n)
        assert np.all(np.abs(a - b) <= (TAU_F16 + TAU_F32) * S)


# ------------------------------------------------------------------ MoE


def _moe_inputs(n_expert, in_f, n_ff, t, n_used, seed=0):
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + 0) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + seed)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, gen.SEED_MOE_X + seed).reshape(t, in_f)
    return wg, wu, ids, sc, x


def _gpu_moe(wg, wu, ids, sc, x, n_expert, n_ff):
    import torch
    import gemv_prefill_decode_amd as qmm
    g, u = qmm.moe_gateup(to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc),
                          to_dev(x), n_expert, n_ff, "nvfp4")
    torch.cuda.synchronize()
    return g.cpu().numpy(), u.cpu().numpy()


@pytest.mark.parametrize("t,n_used", [(1, 4), (3, 2), (5, 4), (16, 3)])
def test_moe_parity_small(t, n_used):
    n_expert, in_f, n_ff = 6, 256, 80
    note(f"moe small t={t} n_used={n_used}")
    wg, wu, ids, sc, x = _moe_inputs(n_expert, in_f, n_ff, t, n_used, seed=t)
    g, u = _gpu_moe(wg, wu, ids, sc, x, n_expert, n_ff)
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    for got, r, S in ((g, rg, Sg), (u, ru, Su)):
        ok, worst = ref.tolerance_check(got, r, S, TAU_F32)
        assert ok, worst


def test_moe_repeated_expert_many_tokens():
    """One expert chosen by 70 tokens (more than one gather chunk)."""
    n_expert, in_f, n_ff, t, n_used = 4, 128, 40, 70, 2
    note("moe repeated expert")
    wg, wu, _, sc, x = _moe_inputs(n_expert, in_f, n_ff, t, n_used)
    ids = np.zeros((t, n_used), dtype=np.int32)
    ids[:, 0] = 2
    ids[:, 1] = np.arange(t) % 2 * 3  # experts 0 and 3 alternate
    g, u = _gpu_moe(wg, wu, ids, sc, x, n_expert, n_ff)
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    assert ref.tolerance_check(g, rg, Sg, TAU_F32)[0]
    assert ref.tolerance_check(u, ru, Su, TAU_F32)[0]


def test_moe_invalid_expert_id_gives_nan():
    n_expert, in_f, n_ff, t, n_used = 4, 128, 40, 2, 2
    note("moe invalid id")
    wg, wu, ids, sc, x = _moe_inputs(n_expert, in_f, n_ff, t, n_used)
    ids = np.array([[1, 7], [2, -1]], dtype=np.int32)
    g, u = _gpu_moe(wg, wu, ids, sc, x, n_expert, n_ff)
    for out in (g, u):
        assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[3]))
        assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(out[2]))
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, np.array([[1, 0], [2, 0]]), sc, x, n_expert, in_f, n_ff)
    assert ref.tolerance_check(g[[0, 2]], rg[[0, 2]], Sg[[0, 2]], TAU_F32)[0]


def _down_inputs(n_expert, n_ff, d_model, t, n_used, seed=0):
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + seed)
    sc = gen.pair_scales(t * n_used)
    act = gen.xorshift_f32(t * n_used * n_ff, gen.SEED_MOE_ACT + seed).reshape(t * n_used, n_ff)
    return wd, ids, sc, act


def _gpu_down(wd, ids, sc, act, n_expert, d_model, qt="nvfp4"):
    import torch
    import gemv_prefill_decode_amd as qmm
    y, pair = qmm.moe_down(to_dev(wd), to_dev(ids.astype(np.int32)), to_dev(sc), to_dev(act),
                           n_expert, d_model, qt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), pair.cpu().numpy()


# d_model 80 takes the 4-wide slot sum, 78 the scalar one; n_used 10 and 12
# take the slot sum's second batch of 8 loads
@pytest.mark.parametrize("t,n_used,d_model", [(1, 8, 80), (3, 2, 78), (5, 4, 80), (16, 3, 78), (2, 10, 80),
                                              (3, 12, 78)])
def test_moe_down_parity_small(t, n_used, d_model):
    n_expert, n_ff = max(9, n_used), 256
    note(f"moe down small t={t} n_used={n_used} d_model={d_model}")
    wd, ids, sc, act = _down_inputs(n_expert, n_ff, d_model, t, n_used, seed=t)
    y, pair = _gpu_down(wd, ids, sc, act, n_expert, d_model)
    ry, Sy, rp, Sp = ref.moe_down_ref("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model)
    ok, worst = ref.tolerance_check(pair, rp, Sp, TAU_F32)
    assert ok, f"pair terms: {worst}"
    ok, worst = ref.tolerance_check(y, ry, Sy, TAU_F32)
    assert ok, f"y: {worst}"
    # the slot sum is the plain f32 sum of the returned pair terms in slot order
    want = pair.reshape(t, n_used, d_model)[:, 0].copy()
    for s in range(1, n_used):
        want += pair.reshape(t, n_used, d_model)[:, s]
    assert np.array_equal(y, want)


@pytest.mark.parametrize("qt", ["q4_k", "q8_0"])
def test_moe_down_other_formats_and_repeats(qt):
    """Other weight formats; one expert shared by many tokens (several gather
    chunks); two identical calls are bit-identical."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, n_ff, d_model, t, n_used = 3, 512, 96, 40, 2
    note(f"moe down {qt} repeats")
    wd = weights(qt, n_expert * d_model, n_ff, 31)
    _, _, sc, act = _down_inputs(n_expert, n_ff, d_model, t, n_used, seed=2)
    ids = np.stack([np.full(t, 1), np.arange(t) % 2 * 2], axis=1).astype(np.int32)
    y, pair = _gpu_down(wd, ids, sc, act, n_expert, d_model, qt)
    ry, Sy, _, _ = ref.moe_down_ref(qt, wd, ids, sc, act, n_expert, n_ff, d_model)
    ok, worst = ref.tolerance_check(y, ry, Sy, TAU_F32)
    assert ok, worst
    y2, pair2 = _gpu_down(wd, ids, sc, act, n_expert, d_model, qt)
    assert np.array_equal(y, y2) and np.array_equal(pair, pair2)


def test_moe_down_invalid_expert_id_gives_nan():
    n_expert, n_ff, d_model, t, n_used = 4, 128, 40, 3, 2
    note("moe down invalid id")
    wd, _, sc, act = _down_inputs(n_expert, n_ff, d_model, t, n_used)
    ids = np.array([[1, 3], [2, 9], [0, 1]], dtype=np.int32)
    y, pair = _gpu_down(wd, ids, sc, act, n_expert, d_model)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(pair[3]))
    assert np.all(np.isfinite(y[[0, 2]])) and np.all(np.isfinite(pair[[0, 1, 2, 4, 5]]))
    ok_ids = np.array([[1, 3], [2, 0], [0, 1]])
    ry, Sy, _, _ = ref.moe_down_ref("nvfp4", wd, ok_ids, sc, act, n_expert, n_ff, d_model)
    assert ref.tolerance_check(y[[0, 2]], ry[[0, 2]], Sy[[0, 2]], TAU_F32)[0]


def test_loadonly_twin_runs_and_is_deterministic():
    import torch
    import gemv_prefill_decode_amd as qmm
    for qt in QTS:
        m, k = 300, 1024
        note(f"loadonly {qt}")
        w = to_dev(weights(qt, m, k, 5))
        a = qmm.stream_loadonly(w, m, k, qt).clone()
        b = qmm.stream_loadonly(w, m, k, qt)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_split_k_workspace_contract():
    """The k-split MFMA path (few output tiles): parity with and without a
    workspace, bit-identical repeats, size and alignment checks."""
    import torch
    import gemv_prefill_decode_amd as qmm
    qt, m, k, n = "q4_k", 1024, 4608, 200
    note(f"split-k {qt} {m}x{k} n={n}")
    nbytes = qmm.workspace_bytes(m, k, n, qt, "mfma")
    assert nbytes > 0
    w = weights(qt, m, k, 21)
    x = acts(n, k, 21)
    wd, xd = to_dev(w), to_dev(x)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")   # contents must not matter
    a = qmm.gemm(wd, xd, m, qt, path="mfma", workspace=ws).clone()
    b = qmm.gemm(wd, xd, m, qt, path="mfma", workspace=ws).clone()
    c = qmm.gemm(wd, xd, m, qt, path="mfma", workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "split-k result not reproducible"
    for got in (a, c):
        check_full(qt, w, x, m, k, n, got.cpu().numpy(), TAU_F16, "split-k")
    with pytest.raises(qmm.QmmError) as e:
        qmm.gemm(wd, xd, m, qt, path="mfma", workspace=ws[:nbytes - 256])
    assert e.value.status == 9
    with pytest.raises(qmm.QmmError) as e:
        qmm.gemm(wd, xd, m, qt, path="mfma", workspace=ws[16:])
    assert e.value.status == 5


def test_split_k_shared_workspace_growing_tile_count():
    """Calls with different shapes share one workspace, each leaving its
    partials behind for the next."""
    import torch
    import gemv_prefill_decode_amd as qmm
    qt = "q8_0"
    shapes = [(256, 2048, 130), (640, 1024, 300), (384, 1536, 200)]   # 6, 15, 6 tiles
    need = max(qmm.workspace_bytes(m, k, n, qt, "mfma") for m, k, n in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for si, (m, k, n) in enumerate(shapes):
        note(f"shared workspace {qt} {m}x{k} n={n}")
        assert qmm.workspace_bytes(m, k, n, qt, "mfma") > 0
        w = weights(qt, m, k, 40 + si)
        x = acts(n, k, 40 + si)
        got = qmm.gemm(to_dev(w), to_dev(x), m, qt, path="mfma", workspace=ws)
        torch.cuda.synchronize()
        check_full(qt, w, x, m, k, n, got.cpu().numpy(), TAU_F16, f"shared ws {m}x{k}x{n}")


def test_split_k_graph_replays(monkeypatch):
    """A k-split call (the GEMM kernel, then the sum of its partials)
    captured in a HIP graph: every replay equals the eager result bit for
    bit, with eager calls of another shape on the same workspace between the
    replays, and the eager result matches the oracle."""
    import torch
    import gemv_prefill_decode_amd as qmm
    qt, m, k, n = "q4_0", 1024, 1024, 512
    monkeypatch.setenv("QMM_MFMA_PLAN", "2,1,4,2")   # the LDS ring, k split 4, 2 k groups
    p = qmm.gemm_plan(m, k, n, qt, "mfma")
    assert p["n_split"] > 1, p
    m2, k2, n2 = 640, 2048, 300
    assert qmm.gemm_plan(m2, k2, n2, qt, "mfma")["n_split"] > 1   # 2048 / 64 / 4 steps per split
    note(f"split-k graph {qt} {m}x{k} n={n} {p}")
    w, x = weights(qt, m, k, 81), acts(n, k, 81)
    w2, x2 = weights(qt, m2, k2, 82), acts(n2, k2, 82)
    wd, xd, wd2, xd2 = to_dev(w), to_dev(x), to_dev(w2), to_dev(x2)
    nbytes = max(qmm.workspace_bytes(m, k, n, qt, "mfma"), qmm.workspace_bytes(m2, k2, n2, qt, "mfma"))
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    eager = qmm.gemm(wd, xd, m, qt, path="mfma", workspace=ws).clone()
    eager2 = qmm.gemm(wd2, xd2, m2, qt, path="mfma", workspace=ws).clone()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qmm.gemm(wd, xd, m, qt, path="mfma", out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmm.gemm(wd, xd, m, qt, path="mfma", out=out, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        other = qmm.gemm(wd2, xd2, m2, qt, path="mfma", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager2), f"eager call after replay {r} differs"
    del g
    check_full(qt, w, x, m, k, n, eager.cpu().numpy(), TAU_F16, "split-k graph")
    check_full(qt, w2, x2, m2, k2, n2, eager2.cpu().numpy(), TAU_F16, "split-k graph, other shape")


# Every prefill kernel family, forced through QMM_MFMA_PLAN on a ragged shape
# (m, n not multiples of any tile; k with a partial split): x16 (5, 6: 64-token
# tiles; 7: 256 x 256 tiles in two token groups), tile rows (wm*64), k splits,
# k groups.
FORCED_PLANS = ["0,2,1,1", "0,2,3,1", "0,2,1,2", "0,2,3,2",
                "2,2,1", "2,2,3", "2,4,1", "2,4,3", "3,2,1", "3,2,3", "2,2,1,2", "2,2,3,2", "3,2,1,2", "3,2,3,2",
                "4,2,1", "4,2,3", "4,2,1,2", "4,2,3,2", "2,1,1", "2,1,3", "2,1,1,2", "4,1,1", "4,1,3,2",
                "5,1,1", "5,1,3", "5,1,1,2", "5,1,3,2", "6,1,1", "6,1,3", "6,1,1,2", "6,1,3,2", "7,4,1", "7,4,3"]


@pytest.mark.parametrize("plan", FORCED_PLANS)
@pytest.mark.parametrize("qt", ["q4_k", "q6_k", "q8_0", "nvfp4", "q4_0", "f32"])
def test_forced_prefill_plans(plan, qt, monkeypatch):
    import gemv_prefill_decode_amd as qmm
    x16, wm = int(plan.split(",")[0]), int(plan.split(",")[1])
    kg = int(plan.split(",")[3]) if plan.count(",") == 3 else 1
    m, k, n = 300, 1536 if qt != "q6_k" else 1792, 270
    if qt == "f32" and (kg == 2 or (x16, wm) == (2, 4)):
        pytest.skip("not a plan the library runs for f32 weights")
    if (x16 == 3 and kg == 2 and qt in ("q6_k", "q8_0", "f32")) or (x16 == 7 and qt == "f32"):
        pytest.skip("its LDS ring does not fit 160 KB")
    monkeypatch.setenv("QMM_MFMA_PLAN", plan)
    p = qmm.gemm_plan(m, k, n, qt, "mfma")
    assert (p["x16"], p["tile_rows"], p["k_groups"]) == (x16, 64 * wm, kg), p
    note(f"forced plan {plan} {qt} {p}")
    w = weights(qt, m, k, 60)
    x = acts(n, k, 60)
    got = gpu_gemm(qt, w, x, m, "mfma")
    check_full(qt, w, x, m, k, n, got, TAU_F16, f"plan {plan} {qt}")


# ------------------------------------------------------------------ NVFP4 V2

def _nvfp4_every_scale_code(m, k, seed):
    """NVFP4 rows (36-byte groups: 4 E4M3 scale bytes, 32 bytes of E2M1
    nibbles) whose scale bytes run through every finite E4M3 code (all but
    0x7F and 0xFF) in turn, random nibbles."""
    w = gen.nvfp4_rows(m, k, gen.SEED_MOE_W + seed).copy()
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    groups = w.reshape(-1, 36)
    groups[:, :4] = np.resize(codes, groups.shape[0] * 4).reshape(-1, 4)
    return w


def test_nvfp4_every_scale_code():
    """The device's E4M3 scale decode (v_cvt_f32_fp8) on all 254 finite codes,
    subnormals and both signs included: the GEMV against the oracle at the f32
    tolerance, and the matrix-core paths on identity activations giving
    f16(W) exactly (every NVFP4 weight is exact in f16)."""
    import os
    import gemv_prefill_decode_amd as qmm
    m, k = 96, 768   # 96 * 12 groups * 4 = 4608 scale slots: every code 18 times
    w = _nvfp4_every_scale_code(m, k, 71)
    W = formats.decode("nvfp4", w, m, k)
    assert np.all(np.isfinite(W))
    note("nvfp4 every scale code: gemv")
    x = acts(3, k, 71)
    check_full("nvfp4", w, x, m, k, 3, gpu_gemm("nvfp4", w, x, m, "gemv"), TAU_F32, "e4m3 codes gemv")
    eye = np.eye(k, dtype=np.float32)
    for plan in (None, "0,2,1,1", "2,2,1", "4,1,1,2"):
        note(f"nvfp4 every scale code: mfma plan {plan}")
        if plan:
            os.environ["QMM_MFMA_PLAN"] = plan
        try:
            got = gpu_gemm("nvfp4", w, eye, m, "mfma")
        finally:
            os.environ.pop("QMM_MFMA_PLAN", None)
        assert_f16_weights(got, W)


def test_nvfp4_v2_repack_bit_exact():
    """The device repack equals the oracle's byte permutation, on a ragged
    row count and on an expert tensor (experts x rows flattened)."""
    import torch
    import gemv_prefill_decode_amd as qmm
    for rows, k in ((37, 192), (8 * 96, 1024)):
        note(f"nvfp4 v2 repack rows={rows} k={k}")
        v1 = gen.nvfp4_rows(rows, k, gen.SEED_MOE_W + rows)
        got = qmm.repack_nvfp4_v2(to_dev(v1), rows, k)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), formats.repack_nvfp4_v2(v1, rows, k))


@pytest.mark.parametrize("n", [1, 3, 8, 32])
def test_gemv_nvfp4_v2_parity_and_identity(n):
    """GEMV on V2 rows: oracle parity, and bit-identical to the same values
    in V1 rows (the unit arithmetic is the same)."""
    m, k = 300, 1536
    note(f"gemv nvfp4_v2 n={n}")
    v1 = gen.nvfp4_rows(m, k, gen.SEED_MOE_W + 77)
    v2 = formats.repack_nvfp4_v2(v1, m, k)
    x = acts(n, k, 5)
    got = gpu_gemm("nvfp4_v2", v2, x, m, "gemv")
    check_full("nvfp4_v2", v2, x, m, k, n, got, TAU_F32, f"gemv nvfp4_v2 n={n}")
    assert np.array_equal(got, gpu_gemm("nvfp4", v1, x, m, "gemv"))


def test_nvfp4_v2_rejected_on_matrix_cores():
    import gemv_prefill_decode_amd as qmm
    m, k, n = 64, 256, 64
    v2 = formats.repack_nvfp4_v2(gen.nvfp4_rows(m, k, 3), m, k)
    with pytest.raises(qmm.QmmError) as ei:
        gpu_gemm("nvfp4_v2", v2, acts(n, k), m, "mfma", workspace=None)
    assert ei.value.status == 4


@pytest.mark.parametrize("t,n_used", [(1, 8), (16, 3)])
def test_moe_nvfp4_v2_bit_identical_to_v1(t, n_used):
    """Gate/up and down on V2 expert rows (repacked on the device) equal the
    V1 results bit for bit, as the pages assert before timing their V2 arms;
    and the V1 results pass the oracle."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff = 9, 512, 96
    note(f"moe nvfp4_v2 t={t}")
    wg, wu, ids, sc, x = _moe_inputs(n_expert, in_f, n_ff, t, n_used, seed=t)
    rows = n_expert * n_ff
    dg, du, di, ds, dx = to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc), to_dev(x)
    g1, u1 = qmm.moe_gateup(dg, du, di, ds, dx, n_expert, n_ff, "nvfp4")
    g2, u2 = qmm.moe_gateup(qmm.repack_nvfp4_v2(dg, rows, in_f), qmm.repack_nvfp4_v2(du, rows, in_f),
                            di, ds, dx, n_expert, n_ff, "nvfp4_v2")
    torch.cuda.synchronize()
    assert torch.equal(g1, g2) and torch.equal(u1, u2)
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    assert ref.tolerance_check(g1.cpu().numpy(), rg, Sg, TAU_F32)[0]
    assert ref.tolerance_check(u1.cpu().numpy(), ru, Su, TAU_F32)[0]
    # down projection: d_model rows over n_ff inputs
    d_model = 80
    wd, _, scd, act = _down_inputs(n_expert, 128, d_model, t, n_used, seed=t)
    dwd = to_dev(wd)
    y1, p1 = qmm.moe_down(dwd, di, to_dev(scd), to_dev(act), n_expert, d_model, "nvfp4")
    y2, p2 = qmm.moe_down(qmm.repack_nvfp4_v2(dwd, n_expert * d_model, 128), di, to_dev(scd),
                          to_dev(act), n_expert, d_model, "nvfp4_v2")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(p1, p2)


# ------------------------------------------------------------------ Q8_1 activations

def test_quantize_q8_1_bit_exact():
    """Device quantization equals the oracle's float32 steps bit for bit:
    random magnitudes, zero blocks, halves that round away from zero."""
    import torch
    import gemv_prefill_decode_amd as qmm
    rng = np.random.default_rng(11)
    rows, k = 7, 1024
    x = (rng.standard_normal(rows * k) * rng.choice([1e-4, 1.0, 300.0], rows * k)).astype(np.float32)
    x[:32] = 0.0                                   # a zero block
    x[32:64] = 0.0
    x[32:38] = [127.0, 2.5, -2.5, 0.5, -0.5, 3.5]  # d = 1: halves
    x = x.reshape(rows, k)
    note("quantize q8_1")
    q, d = qmm.quantize_q8_1(to_dev(x))
    torch.cuda.synchronize()
    rq, rd = ref.quantize_q8_1(x, k)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), rd.reshape(rows, k // 32).view(np.uint32))


@pytest.mark.parametrize("t,n_used", [(1, 8), (3, 2), (16, 3)])
def test_moe_q8_parity_and_v2_identity(t, n_used):
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff = 9, 512, 96
    note(f"moe q8 t={t} n_used={n_used}")
    wg, wu, ids, sc, x = _moe_inputs(n_expert, in_f, n_ff, t, n_used, seed=t + 40)
    dg, du, di, ds = to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc)
    xq, xd = qmm.quantize_q8_1(to_dev(x))
    g, u = qmm.moe_gateup_q8(dg, du, di, ds, xq, xd, n_expert, n_ff, "nvfp4")
    rows = n_expert * n_ff
    g2, u2 = qmm.moe_gateup_q8(qmm.repack_nvfp4_v2(dg, rows, in_f), qmm.repack_nvfp4_v2(du, rows, in_f),
                               di, ds, xq, xd, n_expert, n_ff, "nvfp4_v2")
    torch.cuda.synchronize()
    assert torch.equal(g, g2) and torch.equal(u, u2)
    rq, rd = ref.quantize_q8_1(x, in_f)
    assert np.array_equal(xq.cpu().numpy(), rq)
    rg, ru, Sg, Su = ref.moe_q8_ref("nvfp4", wg, wu, ids, sc, rq, rd, n_expert, in_f, n_ff)
    for got, r, S in ((g, rg, Sg), (u, ru, Su)):
        ok, worst = ref.tolerance_check(got.cpu().numpy(), r, S, TAU_F32)
        assert ok, worst


def test_moe_q8_exact_activations_match_f32_path():
    """Activations that Q8_1 represents exactly (x = d0 * code, d0 a power of
    two, one code +-127 per block): the Q8_1 path and the f32 path compute
    the same exact products; both pass the same oracle."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, t, n_used = 5, 256, 40, 2, 2
    note("moe q8 exact activations")
    wg, wu, ids, sc, _ = _moe_inputs(n_expert, in_f, n_ff, t, n_used, seed=3)
    rng = np.random.default_rng(5)
    codes = rng.integers(-126, 127, (t, in_f))
    codes[:, ::32] = 127
    x = (codes * 2.0 ** -7).astype(np.float32)
    xq, xd = qmm.quantize_q8_1(to_dev(x))
    dg, du, di, ds = to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc)
    g, u = qmm.moe_gateup_q8(dg, du, di, ds, xq, xd, n_expert, n_ff)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), codes.astype(np.int8))
    assert np.all(xd.cpu().numpy() == np.float32(2.0 ** -7))
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
    assert ref.tolerance_check(g.cpu().numpy(), rg, Sg, TAU_F32)[0]
    assert ref.tolerance_check(u.cpu().numpy(), ru, Su, TAU_F32)[0]


# ------------------------------------------------------------------ strided x and dst

@pytest.mark.parametrize("plan", [None, "0,2,1,1", "0,2,3,2", "2,2,1", "2,4,3", "3,2,2",
                                  "4,2,1", "4,2,2,2"])
@pytest.mark.parametrize("qt", ["q4_k", "f32"])
def test_strided_rows_bit_identical(qt, plan, monkeypatch):
    """Row-strided x and dst (qmm_gemm_ex) give bit-identical results to the
    contiguous call on every path and prefill kernel family, and leave the
    padding between dst rows untouched."""
    import torch
    import gemv_prefill_decode_amd as qmm
    if plan is not None:
        if qt == "f32" and ((plan.count(",") == 3 and plan.endswith(",2")) or plan.startswith("2,4")):
            pytest.skip("not a plan the library runs for f32 weights")
        monkeypatch.setenv("QMM_MFMA_PLAN", plan)
    m, k = 300, 1024
    w = to_dev(weights(qt, m, k, 41))
    for n, path in ((5, "gemv"), (13, "gemv"), (200, "mfma")):
        if plan is not None and path == "gemv":
            continue
        note(f"strided {qt} plan={plan} n={n} {path}")
        x = acts(n, k, 41)
        ref_out = qmm.gemm(w, to_dev(x), m, qt, path=path)
        for padx, padd in ((12, 7), (4, 4)):
            xb = torch.zeros((n, k + padx), dtype=torch.float32, device="cuda")
            xb[:, :k] = to_dev(x)
            ob = torch.full((n, m + padd), -7.0, dtype=torch.float32, device="cuda")
            got = qmm.gemm(w, xb[:, :k], m, qt, out=ob[:, :m], path=path)
            torch.cuda.synchronize()
            assert got.data_ptr() == ob.data_ptr()
            assert torch.equal(ob[:, :m], ref_out), f"padx={padx} padd={padd}"
            assert torch.all(ob[:, m:] == -7.0)
