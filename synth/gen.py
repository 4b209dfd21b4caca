"""Seeded synthetic inputs for the dequant-fused projection matmul.

Every generator here restates an input recipe from the pages (cited per
function) or is a plain seeded draw.  None of them decodes or multiplies
anything: the bytes they emit are opaque until a decoder (the oracle's or the
HIP kernels') interprets them.

All generators are deterministic functions of their arguments.  The linear
congruential streams are evaluated with a jump-ahead so that tens of megabytes
of packed weights take well under a second.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "LCG_A",
    "LCG_C",
    "lcg_states",
    "quant_bytes",
    "unit_f32",
    "grid_f32",
    "nvfp4_rows",
    "xorshift_f32",
    "expert_ids",
    "pair_scales",
    "dense_weights",
    "structured_exact",
    "SEED_QUANT",
    "SEED_W_F32",
    "SEED_X",
    "SEED_MOE_W",
    "SEED_MOE_X",
    "SEED_EXPERTS",
    "SEED_MOE_DOWN_W",
    "SEED_MOE_ACT",
]

# Numerical Recipes LCG constants used by every byte/float stream on the pages
# (cera `wgpu_gemm_bench.rs`, fill_quant_bytes / fill_f32; memra
# `moe_rows_ceiling_bench.rs`, Lcg::byte).
LCG_A = 1664525
LCG_C = 1013904223
_M32 = 0xFFFFFFFF

# Seeds.  The dense-weight seed is the page's; distinct buffers get distinct
# seeds by adding 0x9E37 * buffer_id.  The f32-weight seed differs from the
# activation seed on purpose: the page reuses one seed for both, which makes
# the first rows of W equal the rows of x.
SEED_QUANT = 0x12345678
SEED_W_F32 = 0x2545F491
SEED_X = 0x9E3779B9
SEED_MOE_W = 0x8181
SEED_MOE_X = 91
SEED_EXPERTS = 0xE4E4
# MoE down projection (memra `moe_rows_ceiling_bench.rs`, the down arm): the
# page's rows seed, plus the expert index for distinct experts, and the seed of
# its synthetic per-pair activations (a stand-in for the SwiGLU output).
SEED_MOE_DOWN_W = 0x4242
SEED_MOE_ACT = 1234
BUFFER_STRIDE = 0x9E37

_BLOCK = 1 << 16


def _jump_tables(count: int):
    """(A[j], C[j]) with s_{j+1} = A[j]*s_0 + C[j] (mod 2^32), j < count."""
    a = np.empty(count, dtype=np.uint64)
    c = np.empty(count, dtype=np.uint64)
    a[0] = LCG_A
    c[0] = LCG_C
    filled = 1
    while filled < count:
        take = min(filled, count - filled)
        a_l = a[filled - 1]
        c_l = c[filled - 1]
        a[filled:filled + take] = (a_l * a[:take]) & _M32
        c[filled:filled + take] = (a_l * c[:take] + c_l) & _M32
        filled += take
    return a, c


_TABLES = None


def lcg_states(seed: int, n: int) -> np.ndarray:
    """States s_1..s_n of s <- s*1664525 + 1013904223 (mod 2^32), s_0 = seed.

    Returned as uint32.  Equivalent to the sequential loop on the pages
    (`wrapping_mul(1664525).wrapping_add(1013904223)` before each draw).
    """
    global _TABLES
    if n <= 0:
        return np.zeros(0, dtype=np.uint32)
    if _TABLES is None:
        _TABLES = _jump_tables(_BLOCK)
    a, c = _TABLES
    nblk = (n + _BLOCK - 1) // _BLOCK
    starts = np.empty(nblk, dtype=np.uint64)
    s = seed & _M32
    a_b, c_b = int(a[_BLOCK - 1]), int(c[_BLOCK - 1])
    for b in range(nblk):
        starts[b] = s
        s = (a_b * s + c_b) & _M32
    out = np.empty(nblk * _BLOCK, dtype=np.uint32)
    # chunk the 2-D broadcast to bound temporary memory (8 B per state)
    rows_per = max(1, (1 << 24) // _BLOCK)
    for r0 in range(0, nblk, rows_per):
        r1 = min(nblk, r0 + rows_per)
        st = (a[None, :] * starts[r0:r1, None] + c[None, :]) & _M32
        out[r0 * _BLOCK:r1 * _BLOCK] = st.reshape(-1).astype(np.uint32)
    return out[:n]


def quant_bytes(nbytes: int, seed: int = SEED_QUANT, mask_odd: bool = True) -> np.ndarray:
    """Packed-weight byte stream (cera `wgpu_gemm_bench.rs`, fill_quant_bytes).

    byte_i = (s_{i+1} >> 16) & 0xFF; every byte at an odd offset has bit 6
    cleared so that every f16 scale stored at an even offset keeps a finite
    exponent, while its sign bit is kept.  ``mask_odd=False`` gives the raw
    stream (used to check the page's claim about non-finite scales).
    """
    st = lcg_states(seed, nbytes)
    b = ((st >> np.uint32(16)) & np.uint32(0xFF)).astype(np.uint8)
    if mask_odd:
        b[1::2] &= np.uint8(0xBF)
    return b


def unit_f32(n: int, seed: int = SEED_X) -> np.ndarray:
    """Uniform [-1, 1) floats in steps of 2^-15 (cera `wgpu_gemm_bench.rs`, fill_f32)."""
    st = lcg_states(seed, n)
    hi = (st >> np.uint32(16)).astype(np.float32)
    return (hi / np.float32(32768.0) - np.float32(1.0)).astype(np.float32)


def grid_f32(n: int, seed: int, lo: int = -8, hi: int = 8, denom: int = 16) -> np.ndarray:
    """Seeded values (integer in [lo, hi]) / denom.  With a power-of-two denom
    every value and every short sum of products with small integers is exact
    in f16 and f32, which the zero-slack tests rely on."""
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, size=n).astype(np.float64) / denom
    return v.astype(np.float32)


def nvfp4_rows(out_f: int, in_f: int, seed: int) -> np.ndarray:
    """NVFP4 interleaved rows (memra `moe_rows_ceiling_bench.rs`, synth_rows).

    Each 36-byte group (64 weights) gets 4 scale bytes ``(b & 7) | 0x38`` then
    32 payload bytes, all from one LCG byte stream with byte = s >> 24.
    Returns a uint8 array of out_f * (in_f/64*36) bytes (rows contiguous).
    """
    if in_f % 64:
        raise ValueError("in_f must be a multiple of 64")
    nbytes = out_f * (in_f // 64) * 36
    st = lcg_states(seed, nbytes)
    b = (st >> np.uint32(24)).astype(np.uint8)
    g = b.reshape(-1, 36)
    g[:, :4] = (g[:, :4] & np.uint8(0x07)) | np.uint8(0x38)
    return b


def xorshift_f32(n: int, seed: int) -> np.ndarray:
    """Uniform [-1, 1) floats in steps of 2^-23 from xorshift64
    (memra `moe_rows_ceiling_bench.rs`, vecf)."""
    m64 = (1 << 64) - 1
    s = ((seed * 0x9E3779B97F4A7C15) & m64) | 1
    out = np.empty(n, dtype=np.float32)
    for i in range(n):
        s ^= (s << 13) & m64
        s ^= s >> 7
        s ^= (s << 17) & m64
        out[i] = (np.float32(s >> 40) / np.float32(1 << 24) - np.float32(0.5)) * np.float32(2.0)
    return out


def expert_ids(t: int, n_used: int, n_expert: int, seed: int = SEED_EXPERTS) -> np.ndarray:
    """Top-k style routing draw: for each token, ``n_used`` distinct experts
    chosen uniformly from ``n_expert``.  int32 [t, n_used], row-major."""
    if n_used > n_expert:
        raise ValueError("n_used > n_expert")
    rng = np.random.default_rng(seed)
    ids = np.empty((t, n_used), dtype=np.int32)
    for tau in range(t):
        ids[tau] = rng.permutation(n_expert)[:n_used]
    return ids


def pair_scales(count: int) -> np.ndarray:
    """Per-pair f32 scales 0.5 + 0.01*i, evaluated in f32
    (memra `moe_rows_ceiling_bench.rs`, the `scl` vector)."""
    i = np.arange(count, dtype=np.float32)
    return (np.float32(0.01) * i + np.float32(0.5)).astype(np.float32)


def dense_weights(nbytes_or_elems: int, is_f32: bool, buffer_id: int = 0) -> np.ndarray:
    """Weights for one dense buffer: f32 values (``is_f32``; count = elements)
    or packed quant bytes (count = bytes), seeded per buffer."""
    if is_f32:
        return unit_f32(nbytes_or_elems, SEED_W_F32 + BUFFER_STRIDE * buffer_id)
    return quant_bytes(nbytes_or_elems, SEED_QUANT + BUFFER_STRIDE * buffer_id)


def structured_exact(n: int, seed: int) -> np.ndarray:
    """Activations for zero-slack tests: integers in [-8, 8] over 16."""
    return grid_f32(n, seed, -8, 8, 16)
