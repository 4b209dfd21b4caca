"""MoE projections against the oracle in a process of its own, for the GPU
tests that set a once-per-process tuning variable (QMM_MOE_MFMA_MIN: the
smallest chunk of pairs the matrix-core stream takes; 0 = none).  Checks the
gate/up, the fused SwiGLU/clamp and the down projection on shapes whose
experts carry 1 to 70 pairs; prints one OK line per case and exits non-zero
at the first failure."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from gpu_helpers import TAU_F32, to_dev  # noqa: E402
from oracle import ref  # noqa: E402
from synth import gen  # noqa: E402


def inputs(n_expert, in_f, n_ff, t, n_used, seed):
    wg = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e) for e in range(n_expert)])
    wu = np.concatenate([gen.nvfp4_rows(n_ff, in_f, gen.SEED_MOE_W + 2 * e + 1) for e in range(n_expert)])
    ids = gen.expert_ids(t, n_used, n_expert, gen.SEED_EXPERTS + seed)
    sc = gen.pair_scales(2 * t * n_used)
    x = gen.xorshift_f32(t * in_f, gen.SEED_MOE_X + seed).reshape(t, in_f)
    return wg, wu, ids, sc, x


def main():
    import torch
    import gemv_prefill_decode_amd as qmm
    cases = [(6, 256, 80, 5, 4, 0), (9, 512, 96, 16, 3, 1), (4, 128, 40, 70, 2, 2), (64, 1024, 72, 16, 8, 3)]
    for n_expert, in_f, n_ff, t, n_used, seed in cases:
        what = f"env={os.environ.get('QMM_MOE_MFMA_MIN')} E={n_expert} in_f={in_f} n_ff={n_ff} t={t} n_used={n_used}"
        print("case", what, flush=True)
        wg, wu, ids, sc, x = inputs(n_expert, in_f, n_ff, t, n_used, seed)
        if seed == 2:  # one expert chosen by every token, the others alternating
            ids = np.zeros((t, n_used), dtype=np.int32)
            ids[:, 0] = 2
            ids[:, 1] = np.arange(t) % 2 * 3
        dg, du, di, ds, dx = to_dev(wg), to_dev(wu), to_dev(ids.astype(np.int32)), to_dev(sc), to_dev(x)
        g, u = qmm.moe_gateup(dg, du, di, ds, dx, n_expert, n_ff, "nvfp4")
        act = qmm.moe_gateup_act(dg, du, di, ds, dx, n_expert, n_ff, "nvfp4", 7.0)
        torch.cuda.synchronize()
        rg, ru, Sg, Su = ref.moe_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff)
        for got, r, S, nm in ((g, rg, Sg, "gate"), (u, ru, Su, "up")):
            ok, worst = ref.tolerance_check(got.cpu().numpy(), r, S, TAU_F32)
            if not ok:
                sys.exit(f"FAIL {nm} {what}: {worst}")
        ra, Sa = ref.moe_act_ref("nvfp4", wg, wu, ids, sc, x, n_expert, in_f, n_ff, 7.0, TAU_F32)
        ok, worst = ref.tolerance_check(act.cpu().numpy(), ra, Sa, TAU_F32)
        if not ok:
            sys.exit(f"FAIL act {what}: {worst}")
        # down projection: d_model rows over n_ff inputs, each pair's own activation row
        d_model = 48
        wd = np.concatenate([gen.nvfp4_rows(d_model, in_f, gen.SEED_MOE_DOWN_W + e) for e in range(n_expert)])
        a = gen.xorshift_f32(t * n_used * in_f, gen.SEED_MOE_ACT + seed).reshape(t * n_used, in_f)
        scd = gen.pair_scales(t * n_used)
        y, pair = qmm.moe_down(to_dev(wd), di, to_dev(scd), to_dev(a), n_expert, d_model, "nvfp4")
        torch.cuda.synchronize()
        ry, Sy, rp, Sp = ref.moe_down_ref("nvfp4", wd, ids, scd, a, n_expert, in_f, d_model)
        for got, r, S, nm in ((pair, rp, Sp, "down pairs"), (y, ry, Sy, "down y")):
            ok, worst = ref.tolerance_check(got.cpu().numpy(), r, S, TAU_F32)
            if not ok:
                sys.exit(f"FAIL {nm} {what}: {worst}")
        print("OK", what, flush=True)


if __name__ == "__main__":
    main()
