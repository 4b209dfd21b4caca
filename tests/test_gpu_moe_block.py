"""GPU parity of the MoE block around the gate/up projection: the fused
SwiGLU/clamp activation (f32 and Q8_1 activations), the down projection on
Q8_1 pair activations, the whole block gate/up + activation + down, and the
measurement twins of the gate/up kernel.  Every output is compared with the
oracle on the same seeded inputs."""

import numpy as np
import pytest

from gpu_helpers import TAU_F32, note, to_dev
from oracle import formats, ref
from synth import gen

pytestmark = pytest.mark.gpu


def _inputs(n_expert, in_f, n_ff, t, n_used, seed=0, scale=1.0):
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + seed)
    sc = (gen.pair_scales(2 * t * n_used) * np.float32(scale)).astype(np.float32)
    x = gen.xorshift_f32(t * in_f, gen.SEED_MOE_X + seed).reshape(t, in_f)
    return wg, wu, ids, sc, x


def _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff, qt="nvfp4", limit=7.0, q8=False):
    import torch
    import gemv_prefill_decode_amd as qmm
    in_f = x.shape[1]
    rows = n_expert * n_ff
    dg, du = to_dev(wg), to_dev(wu)
    if qt == "nvfp4_v2":
        dg, du = qmm.repack_nvfp4_v2(dg, rows, in_f), qmm.repack_nvfp4_v2(du, rows, in_f)
    di, ds = to_dev(ids.astype(np.int32)), to_dev(sc)
    if q8:
        xq, xd = qmm.quantize_q8_1(to_dev(x))
        act = qmm.moe_gateup_act_q8(dg, du, di, ds, xq, xd, n_expert, n_ff, qt, limit)
    else:
        act = qmm.moe_gateup_act(dg, du, di, ds, to_dev(x), n_expert, n_ff, qt, limit)
    torch.cuda.synchronize()
    return act.cpu().numpy()


# scale 20: many projections exceed the clamp limit on both sides
@pytest.mark.parametrize("t,n_used,scale", [(1, 8, 1.0), (1, 8, 20.0), (3, 2, 20.0), (5, 4, 20.0), (16, 3, 20.0)])
def test_moe_act_parity_and_v2_identity(t, n_used, scale):
    n_expert, in_f, n_ff = 9, 512, 96
    L = 7.0
    note(f"moe act t={t} n_used={n_used} scale={scale}")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=t, scale=scale)
    got = _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff)
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, L, TAU_F32)
    ok, worst = ref.tolerance_check(got, r, S, TAU_F32)
    assert ok, worst
    if scale > 1:
        g, u, _, _ = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
        assert np.any(g > L) and np.any(np.abs(u) > L)      # the clamps were exercised
    assert np.array_equal(got, _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff, "nvfp4_v2"))


def test_moe_act_without_clamp_is_plain_swiglu():
    n_expert, in_f, n_ff, t, n_used = 7, 256, 64, 4, 3
    note("moe act limit=inf")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=2, scale=20.0)
    got = _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff, limit=np.inf)
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, np.inf, TAU_F32)
    ok, worst = ref.tolerance_check(got, r, S, TAU_F32)
    assert ok, worst


@pytest.mark.parametrize("t,n_used", [(1, 8), (3, 2), (16, 3)])
def test_moe_act_q8_parity_and_v2_identity(t, n_used):
    n_expert, in_f, n_ff = 9, 512, 96
    note(f"moe act q8 t={t} n_used={n_used}")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=t + 30, scale=20.0)
    got = _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff, q8=True)
    xq, xd = ref.quantize_q8_1(x, in_f)
    xh = ref.dequantize_q8_1(xq, xd, in_f)
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, xh, n_expert, in_f, n_ff, 7.0, TAU_F32, exact_x=True)
    ok, worst = ref.tolerance_check(got, r, S, TAU_F32)
    assert ok, worst
    assert np.array_equal(got, _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff, "nvfp4_v2", q8=True))


def test_moe_act_invalid_expert_id_gives_nan_rows():
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, t, n_used = 6, 256, 64, 3, 2
    note("moe act invalid id")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=4)
    bad = ids.copy()
    bad[1, 0] = n_expert + 3
    act = qmm.moe_gateup_act(to_dev(wg), to_dev(wu), to_dev(bad.astype(np.int32)), to_dev(sc), to_dev(x),
                             n_expert, n_ff)
    torch.cuda.synchronize()
    act = act.cpu().numpy()
    p_bad = 1 * n_used + 0
    assert np.all(np.isnan(act[p_bad]))
    keep = [p for p in range(t * n_used) if p != p_bad]
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, 7.0, TAU_F32)
    ok, worst = ref.tolerance_check(act[keep], r[keep], S[keep], TAU_F32)
    assert ok, worst


def _down_gpu(wd, ids, sc, aq, ad, n_expert, d_model, qt="nvfp4"):
    import torch
    import gemv_prefill_decode_amd as qmm
    dwd = to_dev(wd)
    n_ff = aq.shape[1]
    if qt == "nvfp4_v2":
        dwd = qmm.repack_nvfp4_v2(dwd, n_expert * d_model, n_ff)
    y, pair = qmm.moe_down_q8(dwd, to_dev(ids.astype(np.int32)), to_dev(sc), to_dev(aq), to_dev(ad), n_expert,
                              d_model, qt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), pair.cpu().numpy()


@pytest.mark.parametrize("t,n_used,d_model", [(1, 8, 80), (3, 2, 78), (16, 3, 80), (2, 10, 78)])
def test_moe_down_q8_parity_and_v2_identity(t, n_used, d_model):
    n_expert, n_ff = max(9, n_used), 256
    note(f"moe down q8 t={t} n_used={n_used} d_model={d_model}")
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + t)
    sc = gen.pair_scales(t * n_used)
    act = gen.xorshift_f32(t * n_used * n_ff, gen.SEED_MOE_ACT + t).reshape(t * n_used, n_ff)
    aq, ad = ref.quantize_q8_1(act, n_ff)
    y, pair = _down_gpu(wd, ids, sc, aq, ad, n_expert, d_model)
    ry, Sy, rp, Sp = ref.moe_down_q8_ref("nvfp4", wd, ids, sc, aq, ad, n_expert, n_ff, d_model)
    assert ref.tolerance_check(y, ry, Sy, TAU_F32)[0]
    assert ref.tolerance_check(pair, rp, Sp, TAU_F32)[0]
    y2, pair2 = _down_gpu(wd, ids, sc, aq, ad, n_expert, d_model, "nvfp4_v2")
    assert np.array_equal(y, y2) and np.array_equal(pair, pair2)


def test_moe_block_gateup_act_down():
    """The whole block on the device: x -> gate/up + activation -> down; the
    down projection checked against the oracle on the device's activation,
    the activation against the oracle on x."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, d_model, t, n_used = 9, 512, 128, 96, 4, 3
    note("moe block")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=9, scale=5.0)
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
    scd = gen.pair_scales(3 * t * n_used)[2 * t * n_used:]
    di = to_dev(ids.astype(np.int32))
    act = qmm.moe_gateup_act(to_dev(wg), to_dev(wu), di, to_dev(sc), to_dev(x), n_expert, n_ff)
    y, pair = qmm.moe_down(to_dev(wd), di, to_dev(scd), act, n_expert, d_model)
    torch.cuda.synchronize()
    a = act.cpu().numpy()
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, 7.0, TAU_F32)
    assert ref.tolerance_check(a, r, S, TAU_F32)[0]
    ry, Sy, _, _ = ref.moe_down_ref("nvfp4", wd, ids, scd, a, n_expert, n_ff, d_model)
    ok, worst = ref.tolerance_check(y.cpu().numpy(), ry, Sy, TAU_F32)
    assert ok, worst


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [1, 16])
def test_moe_act_and_down_q8_full_size(t):
    """The page's shape: gate/up 64 experts of 2048 rows over 4096 inputs,
    8 per token, limit 7.0; the down projection of the same draw on Q8_1
    activations, 4096 rows over 2048.  Every output element."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, n_used, d_model = 64, 4096, 2048, 8, 4096
    note(f"moe act full size t={t}")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used)
    got = _act_gpu(wg, wu, ids, sc, x, n_expert, n_ff)
    r, S = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, 7.0, TAU_F32)
    ok, worst = ref.tolerance_check(got, r, S, TAU_F32)
    assert ok, f"act t={t}: {worst:.3g}"
    del wg, wu
    note(f"moe down q8 full size t={t}")
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
    n_pairs = t * n_used
    scd = gen.pair_scales(3 * n_pairs)[2 * n_pairs:]
    act = gen.xorshift_f32(n_pairs * n_ff, gen.SEED_MOE_ACT).reshape(n_pairs, n_ff)
    aq, ad = ref.quantize_q8_1(act, n_ff)
    y, pair = _down_gpu(wd, ids, scd, aq, ad, n_expert, d_model)
    ry, Sy, rp, Sp = ref.moe_down_q8_ref("nvfp4", wd, ids, scd, aq, ad, n_expert, n_ff, d_model)
    ok, worst = ref.tolerance_check(y, ry, Sy, TAU_F32)
    assert ok, f"down q8 t={t}: {worst:.3g}"
    assert ref.tolerance_check(pair, rp, Sp, TAU_F32)[0]
    torch.cuda.synchronize()


@pytest.mark.parametrize("arm", ["loadonly", "mathonly"])
def test_moe_probe_arms_run_and_are_deterministic(arm):
    """The twins are measurement kernels (their outputs are not
    projections): they run on the served grid and give the same bits on
    two calls; their rows of an invalid id are NaN like the served kernel's."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, t, n_used = 9, 512, 96, 16, 3
    note(f"moe probe {arm}")
    wg, wu, ids, sc, x = _inputs(n_expert, in_f, n_ff, t, n_used, seed=5)
    args = [to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc), to_dev(x), n_expert, n_ff]
    g1, u1 = qmm.moe_gateup_probe(arm, *args)
    g1, u1 = g1.clone(), u1.clone()
    g2, u2 = qmm.moe_gateup_probe(arm, *args)
    torch.cuda.synchronize()
    assert torch.equal(g1.view(torch.int32), g2.view(torch.int32))
    assert torch.equal(u1.view(torch.int32), u2.view(torch.int32))
    with pytest.raises(qmm.QmmError):
        qmm.moe_gateup_probe(arm, *args[:-2], n_expert, n_ff, "q4_k")
