"""gemv_prefill_decode_amd - dequant-fused projection matmul for MI355X (gfx950).

A thin ctypes binding over ``libqmm.so`` (the C-ABI declared in
``include/qmm.h``).  Every step of the computation runs in the library's HIP
kernels; this module only checks tensor dtypes/devices and passes data
pointers and the current HIP stream.  PyTorch is used for device memory and
streams.

    out = gemm(w, x, m, "q4_k")            # dst[n, m] = x[n, k] @ deq(w)[m, k]^T
    g, u = moe_gateup(wg, wu, ids, scales, x, n_expert, n_ff, "nvfp4")

If the library has not been built, every call raises RuntimeError: there is
no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "QTYPES", "PATHS", "QmmError", "lib_path", "load", "gemm", "workspace_bytes", "gemm_plan",
    "plan_kernel_name", "moe_gateup", "moe_down", "moe_gateup_act", "moe_gateup_act_q8", "moe_gateup_probe",
    "moe_down_q8",
    "stream_loadonly", "repack_nvfp4_v2", "quantize_q8_1", "moe_gateup_q8",
    "row_bytes", "block_elems", "gemv_max_n", "status_str", "abi_version",
]

QTYPES = {"f32": 0, "q4_0": 1, "q8_0": 2, "q4_k": 3, "q6_k": 4, "nvfp4": 5, "nvfp4_v2": 6}
PATHS = {"auto": 0, "gemv": 1, "mfma": 2, "gemv_fma": 3, "gemv_matrix": 4}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()


class QmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: qmm status {status} ({status_str(status)})")


def lib_path() -> str:
    """The in-tree libqmm.so, or the library QMM_LIBRARY names (the host-only
    sanitized build that the boundary tests also run against)."""
    return os.environ.get("QMM_LIBRARY") or os.path.join(_HERE, "libqmm.so")


def load() -> ctypes.CDLL:
    """Load libqmm.so (built in-tree by ``__graft_entry__.build()``)."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built: run `python -m gemv_prefill_decode_amd.build` "
                "(or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.qmm_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp]
        lib.qmm_gemm.restype = i32
        lib.qmm_gemm_path.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp]
        lib.qmm_gemm_path.restype = i32
        lib.qmm_gemm_ws.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp, i64, vp]
        lib.qmm_gemm_ex.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, i32, i32, vp, i64, vp]
        lib.qmm_gemm_ex.restype = i32
        lib.qmm_gemm_ws.restype = i32
        lib.qmm_gemm_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, vp]
        lib.qmm_gemm_noalloc.restype = i32
        lib.qmm_gemm_noalloc_max_bytes.argtypes = []
        lib.qmm_gemm_noalloc_max_bytes.restype = i64
        lib.qmm_gemm_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        lib.qmm_gemm_workspace_bytes.restype = i64
        lib.qmm_gemm_plan.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(ctypes.c_int32)]
        lib.qmm_gemm_plan.restype = i32
        lib.qmm_moe_gateup.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.qmm_moe_gateup.restype = i32
        lib.qmm_moe_down.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.qmm_moe_down.restype = i32
        f32 = ctypes.c_float
        lib.qmm_moe_gateup_act.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, vp]
        lib.qmm_moe_gateup_act.restype = i32
        lib.qmm_moe_gateup_act_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, f32, vp]
        lib.qmm_moe_gateup_act_q8.restype = i32
        lib.qmm_moe_gateup_probe.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.qmm_moe_gateup_probe.restype = i32
        lib.qmm_moe_down_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.qmm_moe_down_q8.restype = i32
        lib.qmm_quantize_q8_1.argtypes = [vp, vp, vp, i64, i64, vp]
        lib.qmm_quantize_q8_1.restype = i32
        lib.qmm_moe_gateup_q8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.qmm_moe_gateup_q8.restype = i32
        lib.qmm_nvfp4_repack_v2.argtypes = [vp, vp, i64, i64, vp]
        lib.qmm_nvfp4_repack_v2.restype = i32
        lib.qmm_stream_loadonly.argtypes = [vp, vp, i64, i64, i32, vp]
        lib.qmm_stream_loadonly.restype = i32
        lib.qmm_row_bytes.argtypes = [i32, i64]
        lib.qmm_row_bytes.restype = i64
        lib.qmm_block_elems.argtypes = [i32]
        lib.qmm_block_elems.restype = i32
        lib.qmm_gemv_max_n.argtypes = []
        lib.qmm_gemv_max_n.restype = i32
        lib.qmm_status_str.argtypes = [i32]
        lib.qmm_status_str.restype = ctypes.c_char_p
        lib.qmm_abi_version.argtypes = []
        lib.qmm_abi_version.restype = i32
        _LIB = lib
        return lib


def _qt(qtype) -> int:
    if isinstance(qtype, str):
        if qtype not in QTYPES:
            raise ValueError(f"unknown qtype {qtype!r}")
        return QTYPES[qtype]
    return int(qtype)


def status_str(status: int) -> str:
    return load().qmm_status_str(int(status)).decode()


def abi_version() -> int:
    return load().qmm_abi_version()


def row_bytes(qtype, k: int) -> int:
    r = load().qmm_row_bytes(_qt(qtype), int(k))
    if r < 0:
        raise QmmError(-r, "qmm_row_bytes")
    return r


def block_elems(qtype) -> int:
    r = load().qmm_block_elems(_qt(qtype))
    if r < 0:
        raise QmmError(-r, "qmm_block_elems")
    return r


def gemv_max_n() -> int:
    return load().qmm_gemv_max_n()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, what, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def workspace_bytes(m: int, k: int, n: int, qtype, path: str = "auto") -> int:
    """Bytes of workspace qmm_gemm_ws uses for this product (0: none)."""
    v = load().qmm_gemm_workspace_bytes(m, k, n, _qt(qtype), PATHS[path])
    if v < 0:
        raise QmmError(-v, "qmm_gemm_workspace_bytes")
    return v


def gemm_plan(m: int, k: int, n: int, qtype, path: str = "auto", workspace: bool = True) -> dict:
    """The kernels qmm_gemm_ws (workspace=True) or qmm_gemm would run."""
    out = (ctypes.c_int32 * 6)()
    st = load().qmm_gemm_plan(m, k, n, _qt(qtype), PATHS[path], int(workspace), out)
    if st != 0:
        raise QmmError(st, "qmm_gemm_plan")
    if out[0] == PATHS["gemv"]:
        return {"path": "gemv", "stream": "matrix" if out[1] else "fma", "tokens_per_pass": out[2]}
    return {"path": "mfma", "x16": out[1], "tile_rows": out[2], "k_groups": out[3], "n_split": out[4],
            "steps_per_split": out[5]}


def plan_kernel_name(plan: dict, qtype) -> str:
    """Kernel symbol (as the profiler names it) of a gemm_plan() result."""
    qt = _qt(qtype)
    if plan["path"] == "gemv":
        return "gemv_mfma_kernel" if plan["stream"] == "matrix" else "gemv_kernel"
    if plan["x16"] == 7:
        return f"gemm_lds_tg_kernel<{qt}, 64, 256>"
    if plan["x16"] >= 2:
        cols = 256 if plan["x16"] == 3 else 64 if plan["x16"] in (5, 6) else 128
        return (f"gemm_lds_kernel<{qt}, {plan['tile_rows'] // 4}, {cols}, "
                f"{plan['k_groups']}, {'true' if plan['x16'] in (4, 6) else 'false'}>")
    return f"gemm_mfma_kernel<{qt}, {plan['k_groups']}>"


# Workspaces handed to qmm_gemm_ws by gemm(workspace="auto"): one buffer per
# (device, stream), grown when a product needs more.  Buffers are never
# freed, so a call captured in a graph keeps a valid workspace.
_WS = {}
_WS_ALL = []


def _auto_workspace(device, stream_handle: int, nbytes: int):
    import torch
    key = (device.index, stream_handle)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WS[key] = buf
        _WS_ALL.append(buf)
    return buf


def gemm(w, x, m: int, qtype, out=None, path: str = "auto", stream=None, workspace="auto"):
    """dst[n, m] with dst[j, i] = sum_c deq(w)[i, c] * x[j, c].

    w: packed weights (uint8, m*row_bytes(qtype, k) bytes; float32 [m, k] for
    "f32"); x: float32 [n, k]; out: optional float32 [n, m].  x and out may
    be row-strided views (unit stride along a row, rows any stride apart:
    qmm_gemm_ex); otherwise they must be contiguous.
    workspace: "auto" (a buffer kept per device and stream), None (no k split
    on the matrix-core path), or a device tensor of at least
    workspace_bytes() bytes."""
    import torch
    lib = load()
    qt = _qt(qtype)
    if x.dim() != 2:
        raise ValueError("x must be [n, k]")
    n, k = x.shape
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (n, m):
        raise ValueError(f"out must be [{n}, {m}]")
    need = m * row_bytes(qt, k)
    if w.numel() * w.element_size() != need:
        raise ValueError(f"w holds {w.numel() * w.element_size()} bytes, expected {need}")
    sh = _stream(stream)
    ws_ptr, ws_len = None, 0
    if workspace is not None:
        nbytes = workspace_bytes(m, k, n, qt, path)
        if nbytes > 0:
            if isinstance(workspace, str):
                if workspace != "auto":
                    raise ValueError("workspace must be 'auto', None or a tensor")
                workspace = _auto_workspace(x.device, sh.value or 0, nbytes)
            ws_ptr = _dev(workspace, "workspace")
            ws_len = workspace.numel() * workspace.element_size()
    st = lib.qmm_gemm_ex(*_rows(out, "out"), _dev(w, "w"), *_rows(x, "x"), m, k, n, qt, PATHS[path],
                         ws_ptr, ws_len, sh)
    if st != 0:
        raise QmmError(st, "qmm_gemm_ex")
    return out


def _rows(t, what):
    """(pointer, row stride in elements) of a float32 [rows, cols] device
    tensor with unit stride along its rows."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device (cuda/hip) tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{what} must be torch.float32, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{what} must be 2-D with unit stride along its rows")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    if ld < t.shape[1]:
        raise ValueError(f"{what} rows overlap (row stride {ld} < {t.shape[1]})")
    return ctypes.c_void_p(t.data_ptr()), ld


def moe_gateup(w_gate, w_up, expert_ids, pair_scale, x, n_expert: int, n_ff: int,
               qtype="nvfp4", gate_out=None, up_out=None, stream=None):
    """Gate and up projections over routed experts; returns (gate, up), each
    float32 [t*n_used, n_ff].  expert_ids: int32 [t, n_used]; pair_scale:
    float32 [2*t*n_used] (gate plane then up plane); x: float32 [t, in_f]."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    t2, in_f = x.shape
    if t2 != t:
        raise ValueError("x and expert_ids disagree on t")
    n_pairs = t * n_used
    if pair_scale.numel() != 2 * n_pairs:
        raise ValueError("pair_scale must hold 2*t*n_used floats")
    if gate_out is None:
        gate_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=x.device)
    if up_out is None:
        up_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=x.device)
    st = lib.qmm_moe_gateup(_dev(gate_out, "gate_out", torch.float32),
                            _dev(up_out, "up_out", torch.float32), _dev(w_gate, "w_gate"),
                            _dev(w_up, "w_up"), _dev(expert_ids, "expert_ids", torch.int32),
                            _dev(pair_scale, "pair_scale", torch.float32),
                            _dev(x, "x", torch.float32), t, n_used, n_expert, in_f, n_ff, qt,
                            _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_gateup")
    return gate_out, up_out


def moe_down(w_down, expert_ids, pair_scale, act, n_expert: int, d_model: int, qtype="nvfp4",
             y=None, pair_out=None, stream=None):
    """MoE down projection; returns (y, pair_out): y float32 [t, d_model] (the
    token's slots summed in order), pair_out float32 [t*n_used, d_model] (each
    pair's scaled projection).  expert_ids: int32 [t, n_used]; pair_scale:
    float32 [t*n_used] (the down plane's); act: float32 [t*n_used, n_ff]."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    n_pairs = t * n_used
    n_p2, n_ff = act.shape
    if n_p2 != n_pairs:
        raise ValueError("act must hold one row per pair (t*n_used rows)")
    if pair_scale.numel() != n_pairs:
        raise ValueError("pair_scale must hold t*n_used floats")
    if y is None:
        y = torch.empty((t, d_model), dtype=torch.float32, device=act.device)
    if pair_out is None:
        pair_out = torch.empty((n_pairs, d_model), dtype=torch.float32, device=act.device)
    st = lib.qmm_moe_down(_dev(y, "y", torch.float32), _dev(pair_out, "pair_out", torch.float32),
                          _dev(w_down, "w_down"), _dev(expert_ids, "expert_ids", torch.int32),
                          _dev(pair_scale, "pair_scale", torch.float32),
                          _dev(act, "act", torch.float32), t, n_used, n_expert, n_ff, d_model, qt,
                          _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_down")
    return y, pair_out


def quantize_q8_1(x, q=None, d=None, stream=None):
    """Q8_1 activations of x (float32 [rows, k], k % 32 == 0): returns
    (q int8 [rows, k], d float32 [rows, k/32])."""
    import torch
    lib = load()
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((rows, k // 32), dtype=torch.float32, device=x.device)
    st = lib.qmm_quantize_q8_1(_dev(q, "q", torch.int8), _dev(d, "d", torch.float32),
                               _dev(x, "x", torch.float32), rows, k, _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_quantize_q8_1")
    return q, d


def moe_gateup_q8(w_gate, w_up, expert_ids, pair_scale, xq, xd, n_expert: int, n_ff: int,
                  qtype="nvfp4", gate_out=None, up_out=None, stream=None):
    """moe_gateup on Q8_1 activations (xq int8 [t, in_f], xd float32
    [t, in_f/32] from quantize_q8_1); returns (gate, up)."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    t2, in_f = xq.shape
    if t2 != t or xd.numel() != t * (in_f // 32):
        raise ValueError("xq / xd do not match expert_ids")
    n_pairs = t * n_used
    if pair_scale.numel() != 2 * n_pairs:
        raise ValueError("pair_scale must hold 2*t*n_used floats")
    if gate_out is None:
        gate_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=xq.device)
    if up_out is None:
        up_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=xq.device)
    st = lib.qmm_moe_gateup_q8(_dev(gate_out, "gate_out", torch.float32),
                               _dev(up_out, "up_out", torch.float32), _dev(w_gate, "w_gate"),
                               _dev(w_up, "w_up"), _dev(expert_ids, "expert_ids", torch.int32),
                               _dev(pair_scale, "pair_scale", torch.float32),
                               _dev(xq, "xq", torch.int8), _dev(xd, "xd", torch.float32), t, n_used,
                               n_expert, in_f, n_ff, qt, _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_gateup_q8")
    return gate_out, up_out


def moe_gateup_act(w_gate, w_up, expert_ids, pair_scale, x, n_expert: int, n_ff: int, qtype="nvfp4",
                   limit: float = 7.0, act=None, stream=None):
    """Gate and up projections fused with the SwiGLU/clamp activation:
    returns act float32 [t*n_used, n_ff] = silu(min(gate, limit)) *
    clamp(up, -limit, limit) (the down projection's input).  Arguments as
    moe_gateup; limit > 0 or inf."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    t2, in_f = x.shape
    if t2 != t:
        raise ValueError("x and expert_ids disagree on t")
    n_pairs = t * n_used
    if pair_scale.numel() != 2 * n_pairs:
        raise ValueError("pair_scale must hold 2*t*n_used floats")
    if act is None:
        act = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=x.device)
    st = lib.qmm_moe_gateup_act(_dev(act, "act", torch.float32), _dev(w_gate, "w_gate"), _dev(w_up, "w_up"),
                                _dev(expert_ids, "expert_ids", torch.int32),
                                _dev(pair_scale, "pair_scale", torch.float32), _dev(x, "x", torch.float32),
                                t, n_used, n_expert, in_f, n_ff, qt, float(limit), _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_gateup_act")
    return act


def moe_gateup_act_q8(w_gate, w_up, expert_ids, pair_scale, xq, xd, n_expert: int, n_ff: int,
                      qtype="nvfp4", limit: float = 7.0, act=None, stream=None):
    """moe_gateup_act on Q8_1 activations (xq, xd from quantize_q8_1)."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    t2, in_f = xq.shape
    if t2 != t or xd.numel() != t * (in_f // 32):
        raise ValueError("xq / xd do not match expert_ids")
    n_pairs = t * n_used
    if pair_scale.numel() != 2 * n_pairs:
        raise ValueError("pair_scale must hold 2*t*n_used floats")
    if act is None:
        act = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=xq.device)
    st = lib.qmm_moe_gateup_act_q8(_dev(act, "act", torch.float32), _dev(w_gate, "w_gate"), _dev(w_up, "w_up"),
                                   _dev(expert_ids, "expert_ids", torch.int32),
                                   _dev(pair_scale, "pair_scale", torch.float32), _dev(xq, "xq", torch.int8),
                                   _dev(xd, "xd", torch.float32), t, n_used, n_expert, in_f, n_ff, qt,
                                   float(limit), _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_gateup_act_q8")
    return act


def moe_gateup_probe(arm: str, w_gate, w_up, expert_ids, pair_scale, x, n_expert: int, n_ff: int,
                     qtype="nvfp4", gate_out=None, up_out=None, stream=None):
    """A measurement twin of moe_gateup: arm "loadonly" (the same loads, no
    arithmetic) or "mathonly" (the arithmetic on one cached unit per row
    group).  The outputs are not projections."""
    import torch
    lib = load()
    arms = {"loadonly": 1, "mathonly": 2}
    if arm not in arms:
        raise ValueError(f"unknown arm {arm!r}")
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    in_f = x.shape[1]
    n_pairs = t * n_used
    if gate_out is None:
        gate_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=x.device)
    if up_out is None:
        up_out = torch.empty((n_pairs, n_ff), dtype=torch.float32, device=x.device)
    st = lib.qmm_moe_gateup_probe(arms[arm], _dev(gate_out, "gate_out", torch.float32),
                                  _dev(up_out, "up_out", torch.float32), _dev(w_gate, "w_gate"),
                                  _dev(w_up, "w_up"), _dev(expert_ids, "expert_ids", torch.int32),
                                  _dev(pair_scale, "pair_scale", torch.float32), _dev(x, "x", torch.float32),
                                  t, n_used, n_expert, in_f, n_ff, qt, _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_gateup_probe")
    return gate_out, up_out


def moe_down_q8(w_down, expert_ids, pair_scale, aq, ad, n_expert: int, d_model: int, qtype="nvfp4",
                y=None, pair_out=None, stream=None):
    """moe_down on Q8_1 pair activations (aq int8 [t*n_used, n_ff], ad
    float32 [t*n_used, n_ff/32] from quantize_q8_1); returns (y, pair_out)."""
    import torch
    lib = load()
    qt = _qt(qtype)
    t, n_used = expert_ids.shape
    n_pairs = t * n_used
    n_p2, n_ff = aq.shape
    if n_p2 != n_pairs or ad.numel() != n_pairs * (n_ff // 32):
        raise ValueError("aq / ad must hold one row per pair (t*n_used rows)")
    if pair_scale.numel() != n_pairs:
        raise ValueError("pair_scale must hold t*n_used floats")
    if y is None:
        y = torch.empty((t, d_model), dtype=torch.float32, device=aq.device)
    if pair_out is None:
        pair_out = torch.empty((n_pairs, d_model), dtype=torch.float32, device=aq.device)
    st = lib.qmm_moe_down_q8(_dev(y, "y", torch.float32), _dev(pair_out, "pair_out", torch.float32),
                             _dev(w_down, "w_down"), _dev(expert_ids, "expert_ids", torch.int32),
                             _dev(pair_scale, "pair_scale", torch.float32), _dev(aq, "aq", torch.int8),
                             _dev(ad, "ad", torch.float32), t, n_used, n_expert, n_ff, d_model, qt,
                             _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_moe_down_q8")
    return y, pair_out


def repack_nvfp4_v2(w, rows: int, k: int, out=None, stream=None):
    """NVFP4 rows (uint8, rows*k/64*36 bytes) -> the same values in the
    NVFP4_V2 layout (a new uint8 tensor, or ``out``)."""
    import torch
    lib = load()
    nbytes = rows * (k // 64) * 36
    if w.numel() * w.element_size() < nbytes:
        raise ValueError("w holds fewer than rows*k/64*36 bytes")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = lib.qmm_nvfp4_repack_v2(_dev(out, "out"), _dev(w, "w"), rows, k, _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_nvfp4_repack_v2")
    return out


def stream_loadonly(w, m: int, k: int, qtype, sink=None, stream=None):
    """Load-only twin of the GEMV: reads all of w, writes one checksum per row."""
    import torch
    lib = load()
    if sink is None:
        sink = torch.empty(m, dtype=torch.int32, device=w.device)
    st = lib.qmm_stream_loadonly(_dev(sink, "sink"), _dev(w, "w"), m, k, _qt(qtype), _stream(stream))
    if st != 0:
        raise QmmError(st, "qmm_stream_loadonly")
    return sink
