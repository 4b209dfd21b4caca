"""GPU parity at the benchmarked sizes, in the launch configurations bench.py
times: every output element is compared with the oracle on the same seeded
inputs (the reference is built one block of weight rows, or one expert, at
a time, so host memory stays bounded).

  - Q4_0 GEMM m=1024 k=1024 n=64 (auto dispatch, the matrix-core path)
  - LFM2.5-350M-shaped prefill n=512: 4 shapes x f32/q4_0/q8_0/q4_k/q6_k
  - decode sweep n in {1,4,8,16,32}: q4_k/q6_k at 4608x1024 and 14336x4096
  - NVFP4 MoE gate/up: 64 experts, 8 used, in_f 4096, n_ff 2048, t in {1,16}
  - NVFP4 MoE down: 64 experts of 4096 rows over 2048 inputs, t in {1,16}
  - NVFP4 MoE gate/up on Q8_1 activations at the gate/up shape, t in {1,16}
  - 8B-class prefill n=2048: q4_k/q6_k at 14336x4096 and 4096x14336
"""

import numpy as np
import pytest

from gpu_helpers import TAU_F16, TAU_F32, check_full, check_full_blocked, gpu_gemm, note, to_dev, weights
from oracle import ref
from synth import gen

pytestmark = pytest.mark.gpu

LFM2 = [("ffn_gate", 4608, 1024), ("ffn_down", 1024, 4608), ("conv_in", 3072, 1024),
        ("attn_out", 1024, 1024)]
PREFILL_QTS = ["f32", "q4_0", "q8_0", "q4_k", "q6_k"]


def bench_acts(n, k):
    """The prefill activations bench.py uses (one seed per k)."""
    return gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k)


def _moe_planes(n_expert, in_f, n_ff):
    return [np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + p)
                            for e in range(n_expert)]) for p in range(2)]


def test_q4_0_gemm_1024_n64_whole_output():
    m = k = 1024
    n = 64
    note("q4_0 1024x1024 n=64 auto")
    w = weights("q4_0", m, k, 0)
    x = gen.unit_f32(n * k, gen.SEED_X).reshape(n, k)
    got = gpu_gemm("q4_0", w, x, m, "auto")
    check_full("q4_0", w, x, m, k, n, got, TAU_F16, "q4_0 1024^2 n=64")


@pytest.mark.parametrize("qt", PREFILL_QTS)
def test_lfm2_prefill_n512(qt):
    qi = PREFILL_QTS.index(qt)
    n = 512
    for si, (label, m, k) in enumerate(LFM2):
        note(f"prefill {qt} {label} {m}x{k} n={n}")
        w = weights(qt, m, k, 16 * qi + si)       # the bench's buffers
        x = bench_acts(n, k)
        got = gpu_gemm(qt, w, x, m, "mfma")
        check_full_blocked(qt, w, x, m, k, n, got, TAU_F16, f"prefill {qt} {label}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("qt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("m,k", [(4608, 1024), (14336, 4096)])
def test_decode_sweep(qt, m, k):
    w = weights(qt, m, k, 99)
    for n in (1, 4, 8, 16, 32):
        note(f"decode {qt} {m}x{k} n={n}")
        x = gen.unit_f32(n * k, gen.SEED_X).reshape(n, k)
        got = gpu_gemm(qt, w, x, m, "gemv")
        check_full_blocked(qt, w, x, m, k, n, got, TAU_F32, f"decode {qt} {m}x{k} n={n}", 4096)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [1, 16])
def test_moe_gateup_full_size(t):
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, n_used = 64, 4096, 2048, 8
    note(f"moe full size t={t}")
    planes = _moe_planes(n_expert, in_f, n_ff)
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS)
    n_pairs = t * n_used
    sc = gen.pair_scales(2 * n_pairs)
    x = gen.xorshift_f32(t * in_f, gen.SEED_MOE_X).reshape(t, in_f)
    g, u = qmm.moe_gateup(to_dev(planes[0]), to_dev(planes[1]), to_dev(ids), to_dev(sc), to_dev(x),
                          n_expert, n_ff, "nvfp4")
    torch.cuda.synchronize()
    rg, ru, Sg, Su = ref.moe_ref("nvfp4", planes[0], planes[1], ids, sc, x, n_expert, in_f, n_ff)
    for plane, got, r, S in ((0, g, rg, Sg), (1, u, ru, Su)):
        ok, worst = ref.tolerance_check(got.cpu().numpy(), r, S, TAU_F32)
        assert ok, f"moe t={t} plane {plane}: worst {worst:.3g}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [1, 16])
def test_moe_gateup_q8_full_size(t):
    """Gate/up on Q8_1 activations at the full shape against the oracle on
    the dequantized activations (every output)."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, in_f, n_ff, n_used = 64, 4096, 2048, 8
    note(f"moe q8 full size t={t}")
    planes = _moe_planes(n_expert, in_f, n_ff)
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS)
    n_pairs = t * n_used
    sc = gen.pair_scales(2 * n_pairs)
    x = gen.xorshift_f32(t * in_f, gen.SEED_MOE_X).reshape(t, in_f)
    xq, xd = qmm.quantize_q8_1(to_dev(x))
    g, u = qmm.moe_gateup_q8(to_dev(planes[0]), to_dev(planes[1]), to_dev(ids), to_dev(sc), xq, xd,
                             n_expert, n_ff, "nvfp4")
    torch.cuda.synchronize()
    rq, rd = ref.quantize_q8_1(x, in_f)
    assert np.array_equal(xq.cpu().numpy(), rq)
    rg, ru, Sg, Su = ref.moe_q8_ref("nvfp4", planes[0], planes[1], ids, sc, rq, rd, n_expert, in_f, n_ff)
    for plane, got, r, S in ((0, g, rg, Sg), (1, u, ru, Su)):
        ok, worst = ref.tolerance_check(got.cpu().numpy(), r, S, TAU_F32)
        assert ok, f"moe q8 t={t} plane {plane}: worst {worst:.3g}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [1, 16])
def test_moe_down_full_size(t):
    """The down projection at its full shape: 64 experts of 4096 rows over
    2048 inputs, 8 per token, the same expert draw as the gate/up; y and the
    per-pair terms, every element."""
    import torch
    import gemv_prefill_decode_amd as qmm
    n_expert, n_ff, d_model, n_used = 64, 2048, 4096, 8
    note(f"moe down full size t={t}")
    wd = np.concatenate([gen.nvfp4_rows(d_model, n_ff, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS)
    n_pairs = t * n_used
    sc = gen.pair_scales(3 * n_pairs)[2 * n_pairs:]          # the down plane's block
    act = gen.xorshift_f32(n_pairs * n_ff, gen.SEED_MOE_ACT).reshape(n_pairs, n_ff)
    y, po = qmm.moe_down(to_dev(wd), to_dev(ids), to_dev(sc), to_dev(act), n_expert, d_model, "nvfp4")
    torch.cuda.synchronize()
    ry, Sy, rp, Sp = ref.moe_down_ref("nvfp4", wd, ids, sc, act, n_expert, n_ff, d_model)
    ok, worst = ref.tolerance_check(y.cpu().numpy(), ry, Sy, TAU_F32)
    assert ok, f"moe down t={t}: worst {worst:.3g}"
    ok, worst = ref.tolerance_check(po.cpu().numpy(), rp, Sp, TAU_F32)
    assert ok, f"moe down pair terms t={t}: worst {worst:.3g}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("qt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("m,k", [(14336, 4096), (4096, 14336)])
def test_8b_prefill_n2048(qt, m, k):
    n = 2048
    note(f"8b prefill {qt} {m}x{k} n={n}")
    w = weights(qt, m, k, 7)
    x = gen.unit_f32(n * k, gen.SEED_X + k).reshape(n, k)
    got = gpu_gemm(qt, w, x, m, "mfma")
    check_full_blocked(qt, w, x, m, k, n, got, TAU_F16, f"8b {qt} {m}x{k}", 2048)
