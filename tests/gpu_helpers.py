"""Shared helpers for the GPU parity tests: seeded inputs, device transfer,
oracle comparison.  Inputs come from ``synth`` (shared with nothing else);
expected values come only from ``oracle``."""

from __future__ import annotations

import sys

import numpy as np

import encoders as enc
from oracle import formats, ref
from synth import gen

TAU_F16 = 2e-3     # MFMA path: W and x rounded to f16, f32 accumulation
TAU_F32 = 1e-5     # GEMV and MoE: f32 arithmetic


def note(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def weights(qt: str, m: int, k: int, buf_id: int = 0) -> np.ndarray:
    """Seeded weights: f32 values, NVFP4 rows, or the page's packed byte stream."""
    if qt == "f32":
        return gen.dense_weights(m * k, True, buf_id)
    if qt == "nvfp4":
        return gen.nvfp4_rows(m, k, gen.SEED_MOE_W + buf_id)
    return gen.dense_weights(m * formats.row_bytes(qt, k), False, buf_id)


def acts(n: int, k: int, seed_off: int = 0) -> np.ndarray:
    return gen.unit_f32(n * k, gen.SEED_X + 0x9E37 * seed_off).reshape(n, k)


def exact_weights(qt: str, m: int, k: int, seed: int) -> np.ndarray:
    """Blocks whose every weight and every product with a grid_f32 activation
    is exact in f16 and f32 (power-of-two scales, small integers)."""
    rng = np.random.default_rng(seed)
    if qt == "f32":
        return (rng.integers(-64, 65, m * k) / 16.0).astype(np.float32)
    qk = formats.block_elems(qt)
    nb = m * k // qk
    # largest d exponent per format so that every weight is a multiple of 1/16
    # below 128 in magnitude (11 significant bits: exact in f16)
    e_hi = {"q4_0": 16, "q8_0": 16, "q4_k": 15, "q6_k": 14, "nvfp4": 0}[qt]
    out = []
    for _ in range(nb):
        e = int(rng.integers(11, e_hi + 1)) if e_hi else 0   # d = 2^(e-15) >= 1/16
        d = (int(rng.integers(0, 2)) << 15) | (e << 10)
        if qt == "q4_0":
            out.append(enc.q4_0(d, rng.integers(0, 16, 32)))
        elif qt == "q8_0":
            out.append(enc.q8_0(d, rng.integers(-16, 17, 32)))
        elif qt == "q4_k":
            dmin = (int(rng.integers(0, 2)) << 15) | (int(rng.integers(11, 15)) << 10)
            out.append(enc.q4_k(d, dmin, rng.integers(0, 8, 8), rng.integers(0, 8, 8),
                                rng.integers(0, 16, 256)))
        elif qt == "q6_k":
            out.append(enc.q6_k(d, rng.integers(-4, 5, 16), rng.integers(0, 64, 256)))
        elif qt == "nvfp4":
            out.append(enc.nvfp4(rng.integers(0, 8, 4) | 0x38, rng.integers(0, 16, 64)))
        else:
            raise ValueError(qt)
    return np.frombuffer(b"".join(out), dtype=np.uint8).copy()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def gpu_gemm(qt: str, w: np.ndarray, x: np.ndarray, m: int, path: str, workspace="auto") -> np.ndarray:
    """qmm.gemm on the device; workspace "auto" takes the f16-activation
    prefill kernel (and k splits), None the no-workspace kernel."""
    import torch
    import gemv_prefill_decode_amd as qmm
    out = qmm.gemm(to_dev(w), to_dev(x), m, qt, path=path, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_f16_weights(got, W):
    """Identity activations on the matrix-core path: got[j, i] is weight
    W[i, j] as the matrix cores received it.  Each weight is rounded to f16
    from its exact decoded value, once, to nearest even (numpy's f64 -> f16
    conversion), where the compiler fuses the K-quant decode's multiply-add
    with its f16 conversion (v_fma_mix*_f16); a decode that first rounds to
    f32 may give the f16 of that f32 value instead, which differs only when
    the f32 value lands exactly halfway between two f16 values.  Every
    element must be one of the two, and the second form is counted."""
    once = W.T.astype(np.float16).astype(np.float64)
    via32 = W.T.astype(np.float32).astype(np.float16).astype(np.float64)
    g = got.astype(np.float64)
    ok = (g == once) | (g == via32)
    assert np.all(ok), f"{int((~ok).sum())} weights neither f16(W) nor f16(f32(W))"
    return int(np.sum((g != once) & ok))


def check_full(qt, w, x, m, k, n, got, tau, what=""):
    r, S = ref.gemm_ref(qt, w, x, m, k, n)
    ok, worst = ref.tolerance_check(got, r, S, tau)
    assert ok, f"{what}: worst |gpu-ref|/(tau*S) = {worst:.3g}"
    return worst


def check_full_blocked(qt, w, x, m, k, n, got, tau, what="", rows_per_block=2048):
    """check_full over the whole output of a large shape, the oracle's
    reference computed one block of weight rows at a time."""
    assert got.shape == (n, m), f"{what}: shape {got.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    worst = 0.0
    for i0, i1, r, S in ref.gemm_ref_blocks(qt, w, x, m, k, n, formats.row_bytes(qt, k), rows_per_block):
        ok, wst = ref.tolerance_check(got[:, i0:i1], r, S, tau)
        assert ok, f"{what}: rows {i0}..{i1}: worst |gpu-ref|/(tau*S) = {wst:.3g}"
        worst = max(worst, wst)
    return worst
