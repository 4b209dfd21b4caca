"""The C-ABI boundary, on the CPU: the library loads, exports every function
include/qmm.h declares, reports the pages' packed sizes, and rejects bad
arguments with a status before anything is launched (no GPU needed)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def _lib():
    from gemv_prefill_decode_amd import load, lib_path
    if not os.path.exists(lib_path()):
        pytest.skip("libqmm.so not built")
    return load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_entry_points():
    names = _declared()
    for want in ("qmm_gemm", "qmm_gemm_path", "qmm_moe_gateup", "qmm_moe_down", "qmm_row_bytes",
                 "qmm_block_elems", "qmm_status_str", "qmm_stream_loadonly"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (qmm_\w+)", out.stdout))
        assert set(_declared()) <= exported


def test_row_bytes_match_pages_and_oracle():
    from gemv_prefill_decode_amd import row_bytes, block_elems, QTYPES
    from oracle import formats
    _lib()
    for name in QTYPES:
        qk = formats.block_elems(name)
        assert block_elems(name) == qk
        for k in (qk * 4, qk * 32, 4096 if 4096 % qk == 0 else qk):
            assert row_bytes(name, k) == formats.row_bytes(name, k)
    lib = _lib()
    assert lib.qmm_row_bytes(3, 1000) == -3        # Q4_K, k % 256 != 0 -> -QMM_ERR_K_ALIGN
    assert lib.qmm_row_bytes(9, 256) == -4         # unknown qtype
    assert lib.qmm_row_bytes(1, 0) == -2           # k < 1
    assert lib.qmm_block_elems(7) == -4


def test_status_strings():
    lib = _lib()
    for s in range(9):
        assert lib.qmm_status_str(s).decode() not in ("", "unknown status")
    assert lib.qmm_status_str(99).decode() == "unknown status"
    assert lib.qmm_abi_version() == 1


def test_validation_rejects_before_launch():
    """Every call here fails validation on the host; none reaches a launch, so
    this runs without a GPU."""
    lib = _lib()
    A = ctypes.c_void_p(1 << 20)        # 16-byte aligned fake device pointers
    B = ctypes.c_void_p((1 << 20) + 4)  # misaligned
    z = ctypes.c_void_p(0)
    s0 = ctypes.c_void_p(0)
    g = lib.qmm_gemm_path
    assert g(z, A, A, 64, 256, 4, 3, 0, s0) == 1          # null dst
    assert g(A, z, A, 64, 256, 4, 3, 0, s0) == 1          # null w
    assert g(A, A, z, 64, 256, 4, 3, 0, s0) == 1          # null x
    assert g(A, A, A, 0, 256, 4, 3, 0, s0) == 2           # m < 1
    assert g(A, A, A, 64, 256, 0, 3, 0, s0) == 2          # n < 1
    assert g(A, A, A, 64, 0, 4, 3, 0, s0) == 2            # k < 1
    assert g(A, A, A, 64, 128, 4, 3, 0, s0) == 3          # Q4_K needs k % 256
    assert g(A, A, A, 64, 48, 4, 1, 0, s0) == 3           # Q4_0 needs k % 32
    assert g(A, A, A, 64, 6, 4, 0, 0, s0) == 3            # f32 needs k % 4
    assert g(A, A, A, 64, 256, 4, 7, 0, s0) == 4          # unknown qtype
    assert g(A, B, A, 64, 256, 4, 3, 0, s0) == 5          # misaligned w
    assert g(A, A, B, 64, 256, 4, 3, 0, s0) == 5          # misaligned x
    assert g(B, A, A, 64, 256, 4, 3, 0, s0) == 5          # misaligned dst
    assert g(A, A, A, 64, 256, 4, 3, 9, s0) == 7          # unknown path
    assert g(A, A, A, 1 << 40, 256, 4, 3, 0, s0) == 8     # m beyond int range
    m = lib.qmm_moe_gateup
    assert m(A, A, A, A, z, A, A, 1, 8, 64, 4096, 2048, 5, s0) == 1   # null ids
    assert m(A, A, A, A, A, A, A, 1, 9, 8, 4096, 2048, 5, s0) == 2    # n_used > n_expert
    assert m(A, A, A, A, A, A, A, 1, 8, 64, 4000, 2048, 5, s0) == 3   # in_f % 64
    assert m(A, A, A, A, A, A, A, 1, 8, 64, 4096, 2048, 8, s0) == 4   # qtype
    d = lib.qmm_moe_down
    assert d(A, z, A, A, A, A, 1, 8, 64, 2048, 4096, 5, s0) == 1     # null pair_out
    assert d(A, A, A, A, A, A, 1, 9, 8, 2048, 4096, 5, s0) == 2      # n_used > n_expert
    assert d(A, A, A, A, A, A, 0, 8, 64, 2048, 4096, 5, s0) == 2     # t = 0
    assert d(A, A, A, A, A, A, 1, 8, 64, 2000, 4096, 5, s0) == 3     # n_ff % 64
    assert d(A, A, A, A, A, A, 1, 8, 64, 2048, 4096, 8, s0) == 4     # qtype
    assert d(A, A, A, A, A, A, 70000, 1, 64, 64, 4096, 5, s0) == 8   # more pairs than the grid
    ex = lib.qmm_gemm_ex
    assert ex(A, 64, A, A, 255, 64, 256, 4, 3, 0, z, 0, s0) == 2      # ldx < k
    assert ex(A, 63, A, A, 256, 64, 256, 4, 3, 0, z, 0, s0) == 2      # ldd < m
    assert ex(A, 64, A, A, 258, 64, 256, 4, 3, 0, z, 0, s0) == 5      # ldx % 4
    assert ex(z, 64, A, A, 256, 64, 256, 4, 3, 0, z, 0, s0) == 1      # null dst
    assert ex(A, 64, A, A, 1 << 28, 64, 256, 4, 3, 1, z, 0, s0) == 8  # GEMV x window >= 2^31
    assert ex(A, 64, A, A, 1 << 23, 64, 256, 200, 3, 2, z, 0, s0) == 8  # tile x window >= 2^31
    # an output overlapping an input is rejected (checked last, before any launch)
    C = ctypes.c_void_p((1 << 20) + 64)
    D = ctypes.c_void_p(1 << 24)
    E = ctypes.c_void_p(1 << 26)
    assert ex(A, 64, D, C, 256, 64, 256, 4, 3, 1, z, 0, s0) == 10     # dst over x
    assert ex(A, 64, C, E, 256, 64, 256, 4, 3, 1, z, 0, s0) == 10     # dst over w
    assert d(A, C, D, E, ctypes.c_void_p(1 << 27), ctypes.c_void_p(1 << 28), 1, 8, 64, 2048, 4096, 5,
             s0) == 10                                                  # y over pair_out
    qz = lib.qmm_quantize_q8_1
    assert qz(A, C, D, 4, 256, s0) == 10                              # q over d
    assert qz(A, z, A, 4, 256, s0) == 1                               # null d
    assert qz(A, A, A, 0, 256, s0) == 2                               # rows < 1
    assert qz(A, A, A, 4, 48, s0) == 3                                # k % 32
    assert qz(B, A, A, 4, 256, s0) == 5                               # misaligned q
    mq = lib.qmm_moe_gateup_q8
    assert mq(A, A, A, A, A, A, z, A, 1, 8, 64, 4096, 2048, 5, s0) == 1   # null xq
    assert mq(A, A, A, A, A, A, A, A, 1, 8, 64, 4096, 2048, 3, s0) == 4   # Q4_K weights
    assert mq(A, A, A, A, A, A, A, A, 1, 9, 8, 4096, 2048, 5, s0) == 2    # n_used > n_expert
    assert mq(A, A, A, A, A, A, A, A, 1, 8, 64, 4000, 2048, 5, s0) == 3   # in_f % 64
    assert mq(A, A, A, A, A, A, A, A, 1, 8, 64, 8448, 2048, 5, s0) == 8   # rows exceed LDS
    r = lib.qmm_nvfp4_repack_v2
    assert r(z, A, 4, 128, s0) == 1                                  # null dst
    assert r(A, A, 0, 128, s0) == 2                                  # rows < 1
    assert r(A, ctypes.c_void_p((1 << 21)), 4, 96, s0) == 3          # k % 64
    assert r(ctypes.c_void_p((1 << 20) + 2), ctypes.c_void_p(1 << 21), 4, 128, s0) == 5
    assert r(A, ctypes.c_void_p((1 << 20) + 64), 4, 128, s0) == 10   # overlapping
    # NVFP4 V2 is a streaming-path format: the matrix-core path rejects it
    assert g(A, A, A, 64, 256, 64, 6, 2, s0) == 4
    assert lib.qmm_gemm_workspace_bytes(64, 256, 64, 6, 2) == -4
    assert lib.qmm_gemm_workspace_bytes(64, 256, 8, 6, 0) == 0        # auto -> GEMV
    lo = lib.qmm_stream_loadonly
    assert lo(z, A, 64, 256, 3, s0) == 1
    assert lo(A, A, 64, 255, 3, s0) == 3


@pytest.mark.parametrize("value,expect", [("16", 16), ("1", 1), ("abc", -8), ("0", -8), ("-3", -8)])
def test_gemv_max_n_env_is_strict(value, expect):
    _lib()
    code = ("import sys; sys.path.insert(0, %r); from gemv_prefill_decode_amd import load; "
            "print(load().qmm_gemv_max_n())" % ROOT)
    env = dict(os.environ, QMM_GEMV_MAX_N=value)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env)
    assert out.returncode == 0, out.stderr
    assert int(out.stdout.strip()) == expect
    if expect < 0:
        # an AUTO call with a bad knob fails loudly (before any launch)
        code2 = ("import sys, ctypes; sys.path.insert(0, %r); from gemv_prefill_decode_amd import load; "
                 "A = ctypes.c_void_p(1 << 20); "
                 "print(load().qmm_gemm(A, A, A, 64, 256, 4, 3, ctypes.c_void_p(0)))" % ROOT)
        out = subprocess.run([sys.executable, "-c", code2], capture_output=True, text=True, env=env)
        assert int(out.stdout.strip()) == 8


@pytest.mark.parametrize("var,value", [(v, x) for v in ("QMM_GEMV_WG_PER_CU", "QMM_MOE_WG_PER_CU", "QMM_GEMV_ROWS",
                                                         "QMM_GEMV_DEPTH", "QMM_MOE_LPR_LOG2", "QMM_GEMV_MFMA_TT")
                                       for x in ("0", "abc", "65", "3x")] +
                         [(v, x) for v in ("QMM_MOE_MFMA_MIN", "QMM_GEMV_MFMA_MIN") for x in ("-1", "abc", "65", "3x")])
def test_streaming_tuning_env_is_strict(var, value):
    """A malformed or out-of-range launch-shape knob makes the streaming
    entry points fail with QMM_ERR_RANGE before any launch."""
    _lib()
    code = ("import sys, ctypes; sys.path.insert(0, %r); from gemv_prefill_decode_amd import load; "
            "A = ctypes.c_void_p(1 << 20); lib = load(); "
            "print(lib.qmm_moe_gateup(A, A, A, A, A, A, A, 1, 8, 64, 4096, 2048, 5, ctypes.c_void_p(0)), "
            "lib.qmm_moe_down(A, A, A, A, A, A, 1, 8, 64, 2048, 4096, 5, ctypes.c_void_p(0)), "
            "lib.qmm_stream_loadonly(A, A, 64, 256, 3, ctypes.c_void_p(0)))" % ROOT)
    env = dict(os.environ, **{var: value})
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["8", "8", "8"]


def test_default_gemv_max_n():
    lib = _lib()
    if "QMM_GEMV_MAX_N" in os.environ:
        pytest.skip("QMM_GEMV_MAX_N set in the environment")
    assert lib.qmm_gemv_max_n() == 32


def test_workspace_bytes_plan_and_errors():
    """Workspace sizes: the matrix-core path takes one (f16 activations, and
    split-k partials for few-tile products), at least n*k*2 bytes; the GEMV
    path none; bad arguments give -status."""
    lib = _lib()
    f = lib.qmm_gemm_workspace_bytes
    assert f(1024, 4608, 512, 3, 2) >= 512 * 4608 * 2
    assert f(14336, 4096, 2048, 3, 2) >= 2048 * 4096 * 2
    assert f(4096, 4096, 8, 3, 1) == 0           # GEMV path
    assert f(4096, 4096, 8, 3, 0) == 0           # AUTO -> GEMV at n = 8
    assert f(10, 256, 40, 9, 2) == -4
    assert f(0, 256, 40, 3, 2) == -2
    assert f(10, 256, 40, 3, 7) == -7
    ws = f(1024, 4608, 512, 3, 2)
    assert ws % 256 == 0


def test_gemm_ws_validates_before_launch():
    lib = _lib()
    import ctypes
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    # null dst / x
    assert lib.qmm_gemm_ws(None, p, p, 10, 256, 40, 3, 2, None, 0, None) == 1
    # unknown path
    assert lib.qmm_gemm_ws(p, p, p, 10, 256, 40, 3, 9, None, 0, None) in (5, 7)


def test_gemm_ws_rejects_a_workspace_overlapping_an_operand():
    """The matrix-core kernels write the workspace (f16 activations, k-split
    partials) while they read x and w and write dst: a workspace that
    overlaps any of them is QMM_ERR_ALIAS (fake pointers, no launch)."""
    lib = _lib()
    m, k, n, qt = 1024, 4608, 512, 3
    need = lib.qmm_gemm_workspace_bytes(m, k, n, qt, 2)
    assert need > 0
    dst, x, w = 1 << 30, 1 << 31, 1 << 32          # dst 2 MB, x 9.4 MB, w 2.7 MB: disjoint
    V = ctypes.c_void_p
    s0 = V(0)
    for ws in (dst + 4096, x + (1 << 20), w + 256, dst - (1 << 12) * 256):
        st = lib.qmm_gemm_ws(V(dst), V(w), V(x), m, k, n, qt, 2, V(ws), need, s0)
        assert st == 10, (hex(ws), st)
    # the workspace's own size decides: one ending right before dst is fine up
    # to the launch, which never happens here (too small: QMM_ERR_WORKSPACE first)
    assert lib.qmm_gemm_ws(V(dst), V(w), V(x), m, k, n, qt, 2, V(dst - 256), 256, s0) == 9


def test_gemm_plan_reports_kernels():
    """qmm_gemm_plan: GEMV below the crossover (its FMA stream at n < 3, the
    matrix-core stream from n = 8 and, below, where the rows or row groups are
    many, with 8 activation rows per pass where they fit the LDS, which at
    k = 1024 they do on any device), MFMA above; without a
    workspace never a pre-pass or a k split; bad arguments give a status."""
    import gemv_prefill_decode_amd as qmm
    _lib()
    assert qmm.gemm_plan(4096, 1024, 8, "q4_k") == {"path": "gemv", "stream": "matrix", "tokens_per_pass": 8}
    # below n = 8 the matrix-core stream only with many row groups or long rows
    # (the CPU build sees the default 256 CUs)
    assert qmm.gemm_plan(4096, 1024, 4, "q4_k") == {"path": "gemv", "stream": "fma", "tokens_per_pass": 0}
    assert qmm.gemm_plan(16384, 1024, 4, "q4_k")["stream"] == "matrix"
    assert qmm.gemm_plan(1024, 2048, 4, "q4_k")["stream"] == "matrix"
    assert qmm.gemm_plan(4096, 1024, 2, "q4_k") == {"path": "gemv", "stream": "fma", "tokens_per_pass": 0}
    assert qmm.gemm_plan(4096, 1024, 8, "q4_k", "gemv_fma")["stream"] == "fma"
    assert qmm.gemm_plan(4096, 1024, 1, "q4_k", "gemv_matrix")["tokens_per_pass"] == 4
    assert qmm.gemm_plan(4096, 4096, 8, "q4_k")["path"] == "gemv"
    p = qmm.gemm_plan(4096, 4096, 512, "q4_k", workspace=False)
    assert p["path"] == "mfma" and p["x16"] == 0 and p["n_split"] == 1 and p["k_groups"] == 1
    p = qmm.gemm_plan(1024, 4608, 512, "q4_k", "mfma")
    assert p["n_split"] > 1 and p["steps_per_split"] % 2 == 0
    assert p["n_split"] * p["steps_per_split"] >= 4608 // 64
    import ctypes
    lib = _lib()
    out = (ctypes.c_int32 * 6)()
    assert lib.qmm_gemm_plan(10, 256, 40, 9, 2, 1, out) == 4
    assert lib.qmm_gemm_plan(10, 256, 40, 3, 2, 1, None) == 1


def test_moe_block_entry_points_validate_before_launch():
    """The SwiGLU/clamp gate/up, its Q8_1 form, the Q8_1 down projection
    and the gate/up measurement twins reject bad arguments on the host."""
    lib = _lib()
    A = ctypes.c_void_p(1 << 20)
    z = ctypes.c_void_p(0)
    s0 = ctypes.c_void_p(0)
    F = ctypes.c_float
    act = lib.qmm_moe_gateup_act
    act.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 5 + [ctypes.c_int, F, ctypes.c_void_p]
    ok_args = (1, 8, 64, 4096, 2048, 5)
    assert act(z, A, A, A, A, A, *ok_args, F(7.0), s0) == 1                 # null act
    assert act(A, A, A, A, A, A, 1, 9, 8, 4096, 2048, 5, F(7.0), s0) == 2   # n_used > n_expert
    assert act(A, A, A, A, A, A, 1, 8, 64, 4096, 2048, 8, F(7.0), s0) == 4  # qtype
    assert act(A, A, A, A, A, A, *ok_args, F(0.0), s0) == 8                 # limit <= 0
    assert act(A, A, A, A, A, A, *ok_args, F(float("nan")), s0) == 8       # limit NaN
    X = ctypes.c_void_p(1 << 24)
    assert act(ctypes.c_void_p((1 << 24) + 64), ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31),
               ctypes.c_void_p(1 << 26), ctypes.c_void_p(1 << 27), X, *ok_args, F(7.0), s0) == 10  # act over x
    aq8 = lib.qmm_moe_gateup_act_q8
    aq8.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + [ctypes.c_int, F, ctypes.c_void_p]
    assert aq8(A, A, A, A, A, A, A, *ok_args[:5], 3, F(7.0), s0) == 4         # Q4_K weights
    assert aq8(A, A, A, A, A, A, z, *ok_args, F(7.0), s0) == 1                # null xd
    assert aq8(A, A, A, A, A, A, A, 1, 8, 64, 8448, 2048, 5, F(7.0), s0) == 8  # rows exceed LDS
    dq = lib.qmm_moe_down_q8
    dq.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_void_p]
    assert dq(A, A, A, A, A, z, A, 1, 8, 64, 2048, 4096, 5, s0) == 1        # null aq
    assert dq(A, A, A, A, A, A, A, 1, 8, 64, 2048, 4096, 2, s0) == 4        # Q8_0 weights
    assert dq(A, A, A, A, A, A, A, 1, 8, 64, 2000, 4096, 5, s0) == 3        # n_ff % 64
    assert dq(A, A, A, A, A, A, A, 1, 9, 8, 2048, 4096, 5, s0) == 2         # n_used > n_expert
    pr = lib.qmm_moe_gateup_probe
    pr.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_void_p]
    assert pr(0, A, A, A, A, A, A, A, *ok_args, s0) == 7                    # unknown arm
    assert pr(3, A, A, A, A, A, A, A, *ok_args, s0) == 7
    assert pr(1, A, A, A, A, A, A, A, 1, 8, 64, 4096, 2048, 3, s0) == 4     # Q4_K weights
    assert pr(2, z, A, A, A, A, A, A, *ok_args, s0) == 1
