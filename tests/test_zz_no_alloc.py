"""qmm_gemm_noalloc, the entry point for callers that cannot allocate: its
workspace is the library's static device array.  Through the C-ABI, its
output equals qmm_gemm_ws's with caller memory (the same plan and kernels)
bit for bit, and passes the oracle on the whole output, on consecutive calls
of decreasing size that reuse the array; products whose plan needs more than
the array are rejected before any launch."""

import ctypes

import numpy as np
import pytest

from gpu_helpers import TAU_F16, TAU_F32, acts, check_full, note, weights

QI = {"f32": 0, "q4_0": 1, "q8_0": 2, "q4_k": 3, "q6_k": 4, "nvfp4": 5}


def _lib():
    import gemv_prefill_decode_amd as qmm
    return qmm.load()


def test_noalloc_rejects_products_beyond_the_scratch():
    """No GPU needed: the size check comes before any runtime call."""
    lib = _lib()
    cap = lib.qmm_gemm_noalloc_max_bytes()
    assert cap == 64 << 20
    m, k, n, qt = 4096, 14336, 8192, 3
    need = lib.qmm_gemm_workspace_bytes(m, k, n, qt, 2)
    assert need > cap
    A = ctypes.c_void_p(1 << 20)
    assert lib.qmm_gemm_noalloc(A, A, A, m, k, n, qt, 2, ctypes.c_void_p(0)) == 11
    assert lib.qmm_gemm_noalloc(None, A, A, m, k, n, qt, 2, ctypes.c_void_p(0)) == 1
    assert lib.qmm_gemm_noalloc(A, A, A, m, k, n, 9, 2, ctypes.c_void_p(0)) == 4
    assert lib.qmm_status_str(11).decode() != "unknown status"


@pytest.mark.gpu
def test_noalloc_equals_gemm_ws_on_consecutive_calls():
    import torch
    lib = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [
        ("q4_k", 1024, 4608, 512, 2),   # LFM2 ffn_down: k split, partials in the scratch
        ("q6_k", 4608, 1024, 512, 2),   # LFM2 ffn_gate: f16 activations in the scratch
        ("q4_0", 300, 1536, 270, 2),    # smaller, ragged
        ("q8_0", 130, 512, 8, 0),       # AUTO -> the GEMV: no scratch
    ]
    for qt, m, k, n, path in cases:
        note(f"noalloc {qt} {m}x{k} n={n} path={path}")
        qi = QI[qt]
        need = lib.qmm_gemm_workspace_bytes(m, k, n, qi, path)
        assert 0 <= need <= lib.qmm_gemm_noalloc_max_bytes()
        w = weights(qt, m, k, 70 + m)
        x = acts(n, k, 70 + n)
        dw = torch.from_numpy(w).cuda()
        dx = torch.from_numpy(x).cuda()
        a = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
        b = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        st = lib.qmm_gemm_ws(a.data_ptr(), dw.data_ptr(), dx.data_ptr(), m, k, n, qi, path,
                             ws.data_ptr() if need else None, need, s)
        assert st == 0, st
        st = lib.qmm_gemm_noalloc(b.data_ptr(), dw.data_ptr(), dx.data_ptr(), m, k, n, qi, path, s)
        assert st == 0, st
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        tau = TAU_F32 if (path == 1 or (path == 0 and n <= 32)) else TAU_F16
        check_full(qt, w, x, m, k, n, b.cpu().numpy(), tau, f"noalloc {qt} {m}x{k} n={n}")
