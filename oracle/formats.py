"""Block formats of the packed weight matrix, decoded exactly to float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

Sizes (elements per block QK / bytes per block BB) are the packed sizes on the
pages: cera `wgpu_gemm_bench.rs`, the VARIANTS table (f32 4 B per element,
q4_0 e/32*18, q8_0 e/32*34, q4_k e/256*144, q6_k e/256*210) and memra
`moe_rows_ceiling_bench.rs`, synth_rows (NVFP4: in_f/64 groups of 36 B).
A weight matrix is m rows of row_bytes(k) = k/QK*BB bytes, blocks along k,
rows contiguous, no padding.

The byte layouts inside a block are not printed on the pages; the pages name
them by family (llama.cpp/ggml block quantization).  The readings used here:

  f16       IEEE binary16 little-endian, subnormals decoded, never flushed.
  Q4_0      d:f16@0, qs[16]@2.  elem j<16: d*((qs[j]&15)-8); elem j+16: d*((qs[j]>>4)-8).
  Q8_0      d:f16@0, int8 q[32]@2.  elem j: d*q[j].
  Q4_K      d:f16@0, dmin:f16@2, sc[12]@4, qs[128]@16.  Eight 6-bit (scale, min)
            pairs; chunk c<4 covers elems 64c..64c+63: low nibbles of
            qs[32c..32c+31] with pair 2c, high nibbles with pair 2c+1;
            elem = d*scale*q - dmin*min.
  Q6_K      ql[128]@0, qh[64]@128, int8 scales[16]@192, d:f16@208.  6-bit codes
            built from a low nibble of ql and two bits of qh (see _q6k_codes);
            elem e = d*scales[e/16]*(q(e)-32).
  NVFP4     s[4] E4M3FN@0, qs[32]@4 per 64 elems.  Half h covers elems
            32h..32h+31: elem 32h+j (j<16) = E2M1(qs[16h+j]&15)*E4M3(s[2h]);
            elem 32h+16+j = E2M1(qs[16h+j]>>4)*E4M3(s[2h+1]).
  NVFP4_V2  the same values with quants and scales in separate streams (memra
            `moe_rows_ceiling_bench.rs`: 18 bytes per 32-element group, 16 of
            quants and 2 of scales, the scales contiguous; the pages print no
            byte order, so this is a reading): a row of k elems is the k/2
            quant bytes, then the k/16 scale bytes.  Group g (elems 32g..32g+31):
            elem 32g+j (j<16) = E2M1(q[16g+j]&15)*E4M3(s[2g]);
            elem 32g+16+j = E2M1(q[16g+j]>>4)*E4M3(s[2g+1]).  Rows are whole
            NVFP4 groups (k a multiple of 64), so a row is the V1 row with each
            36-byte group split into its 32 quant bytes and its scale word.
"""

from __future__ import annotations

import numpy as np

# name -> (id, elements per block, bytes per block)
QTYPES = {
    "f32": (0, 1, 4),
    "q4_0": (1, 32, 18),
    "q8_0": (2, 32, 34),
    "q4_k": (3, 256, 144),
    "q6_k": (4, 256, 210),
    "nvfp4": (5, 64, 36),
    "nvfp4_v2": (6, 64, 36),   # not a contiguous block: see the module docstring
}


def qtype_id(name: str) -> int:
    return QTYPES[name][0]


def block_elems(name: str) -> int:
    return QTYPES[name][1]


def block_bytes(name: str) -> int:
    return QTYPES[name][2]


def row_bytes(name: str, k: int) -> int:
    _, qk, bb = QTYPES[name]
    if k % qk:
        raise ValueError(f"k={k} is not a multiple of the {name} block size {qk}")
    return k // qk * bb


# ---------------------------------------------------------------- element codecs


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE 754 binary16 from its definition: sign, 5-bit exponent (bias 15),
    10-bit fraction; exponent 0 is subnormal (f * 2^-24); exponent 31 is
    Inf (f == 0) or NaN.  (Same decode as hrx-rs `patch_bench.rs`, `float`,
    except that Inf is kept distinct from NaN.)"""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int64))
    sub = np.ldexp(f, -24)
    v = np.where(e == 0, sub, normal)
    v = np.where(e == 31, np.where(f == 0, np.inf, np.nan), v)
    return sign * v


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """OCP FP8 E4M3FN: sign bit 7, 4-bit exponent (bias 7), 3-bit mantissa;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no Inf."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    mant = (b & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + mant / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(mant / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & ((b & 7) == 7), np.nan, v)
    return sign * v


def e2m1_bits_to_f64(bits) -> np.ndarray:
    """OCP MX FP4 E2M1: sign bit 3, 2-bit exponent (bias 1), 1-bit mantissa;
    exponent 0 is subnormal (m * 0.5).  Magnitudes 0,0.5,1,1.5,2,3,4,6."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x8, -1.0, 1.0)
    e = (b >> 1) & 0x3
    mant = (b & 0x1).astype(np.float64)
    normal = np.ldexp(1.0 + mant / 2.0, (e - 1).astype(np.int64))
    sub = mant * 0.5
    return sign * np.where(e == 0, sub, normal)


def _le16(lo, hi) -> np.ndarray:
    return np.asarray(lo).astype(np.int64) | (np.asarray(hi).astype(np.int64) << 8)


# ---------------------------------------------------------------- block decoders


def _blocks(data, m: int, k: int, name: str) -> np.ndarray:
    _, qk, bb = QTYPES[name]
    rb = row_bytes(name, k)
    buf = np.ascontiguousarray(np.asarray(data).reshape(-1).view(np.uint8))
    if buf.size != m * rb:
        raise ValueError(f"{name}: expected {m * rb} bytes for m={m} k={k}, got {buf.size}")
    return buf.reshape(m, k // qk, bb)


def _decode_f32(data, m, k):
    a = np.asarray(data)
    if a.dtype == np.uint8:
        a = a.view(np.float32)
    a = a.reshape(-1).astype(np.float32)
    if a.size != m * k:
        raise ValueError("f32 weights: wrong element count")
    return a.astype(np.float64).reshape(m, k)


def _decode_q4_0(data, m, k):
    blk = _blocks(data, m, k, "q4_0")
    d = f16_bits_to_f64(_le16(blk[..., 0], blk[..., 1]))          # [m, nb]
    qs = blk[..., 2:18].astype(np.int64)                           # [m, nb, 16]
    q = np.concatenate([qs & 0xF, qs >> 4], axis=-1) - 8           # elems 0..15, 16..31
    return (d[..., None] * q).reshape(m, k)


def _decode_q8_0(data, m, k):
    blk = _blocks(data, m, k, "q8_0")
    d = f16_bits_to_f64(_le16(blk[..., 0], blk[..., 1]))
    q = blk[..., 2:34].view(np.int8).astype(np.int64)
    return (d[..., None] * q).reshape(m, k)


def _q4k_scale_min(sc: np.ndarray):
    """Eight 6-bit (scale, min) pairs from the 12 packed bytes (last axis)."""
    sc = sc.astype(np.int64)
    scales = np.empty(sc.shape[:-1] + (8,), dtype=np.int64)
    mins = np.empty_like(scales)
    for j in range(4):
        scales[..., j] = sc[..., j] & 63
        mins[..., j] = sc[..., j + 4] & 63
    for j in range(4, 8):
        scales[..., j] = (sc[..., j + 4] & 0xF) | ((sc[..., j - 4] >> 6) << 4)
        mins[..., j] = (sc[..., j + 4] >> 4) | ((sc[..., j] >> 6) << 4)
    return scales, mins


def _decode_q4_k(data, m, k):
    blk = _blocks(data, m, k, "q4_k")
    d = f16_bits_to_f64(_le16(blk[..., 0], blk[..., 1]))
    dmin = f16_bits_to_f64(_le16(blk[..., 2], blk[..., 3]))
    scales, mins = _q4k_scale_min(blk[..., 4:16])                 # [m, nb, 8]
    qs = blk[..., 16:144].astype(np.int64).reshape(m, -1, 4, 32)   # chunk c, byte l
    out = np.empty((m, qs.shape[1], 4, 2, 32), dtype=np.float64)
    for c in range(4):
        for half, q in ((0, qs[:, :, c, :] & 0xF), (1, qs[:, :, c, :] >> 4)):
            j = 2 * c + half
            out[:, :, c, half, :] = (d * scales[..., j])[..., None] * q - (dmin * mins[..., j])[..., None]
    return out.reshape(m, k)


def _q6k_codes(ql: np.ndarray, qh: np.ndarray) -> np.ndarray:
    """6-bit codes q(e), e = 0..255, for ql [..,128] and qh [..,64]."""
    ql = ql.astype(np.int64)
    qh = qh.astype(np.int64)
    q = np.empty(ql.shape[:-1] + (256,), dtype=np.int64)
    for h in range(2):
        L = ql[..., 64 * h:64 * h + 64]
        H = qh[..., 32 * h:32 * h + 32]
        base = 128 * h
        q[..., base + 0:base + 32] = (L[..., 0:32] & 0xF) | ((H & 3) << 4)
        q[..., base + 32:base + 64] = (L[..., 32:64] & 0xF) | (((H >> 2) & 3) << 4)
        q[..., base + 64:base + 96] = (L[..., 0:32] >> 4) | (((H >> 4) & 3) << 4)
        q[..., base + 96:base + 128] = (L[..., 32:64] >> 4) | (((H >> 6) & 3) << 4)
    return q


def _decode_q6_k(data, m, k):
    blk = _blocks(data, m, k, "q6_k")
    q = _q6k_codes(blk[..., 0:128], blk[..., 128:192])             # [m, nb, 256]
    sc = blk[..., 192:208].view(np.int8).astype(np.int64)          # [m, nb, 16]
    d = f16_bits_to_f64(_le16(blk[..., 208], blk[..., 209]))
    scale = d[..., None] * np.repeat(sc, 16, axis=-1)              # elem e -> sc[e/16]
    return (scale * (q - 32)).reshape(m, k)


# The FP8 / FP4 codecs above evaluated once on every code; the NVFP4
# decoders index these tables (the same values, element by element).
_E4M3 = e4m3_bits_to_f64(np.arange(256))
_E2M1 = e2m1_bits_to_f64(np.arange(16))


def _decode_nvfp4(data, m, k):
    blk = _blocks(data, m, k, "nvfp4")
    s = _E4M3[blk[..., 0:4]]                                       # [m, ng, 4]
    qs = blk[..., 4:36].reshape(m, -1, 2, 16)                      # half h, byte j
    out = np.empty((m, qs.shape[1], 2, 2, 16), dtype=np.float64)
    for h in range(2):
        out[:, :, h, 0, :] = _E2M1[qs[:, :, h, :] & 0xF] * s[..., 2 * h, None]
        out[:, :, h, 1, :] = _E2M1[qs[:, :, h, :] >> 4] * s[..., 2 * h + 1, None]
    return out.reshape(m, k)


def _decode_nvfp4_v2(data, m, k):
    rows = np.asarray(data).reshape(-1).view(np.uint8).reshape(m, row_bytes("nvfp4_v2", k))
    q = rows[:, :k // 2].reshape(m, k // 32, 16)                      # group g, byte j
    s = _E4M3[rows[:, k // 2:].reshape(m, k // 32, 2)]                # group g, run i
    out = np.empty((m, k // 32, 2, 16), dtype=np.float64)
    out[:, :, 0, :] = _E2M1[q & 0xF] * s[:, :, 0, None]
    out[:, :, 1, :] = _E2M1[q >> 4] * s[:, :, 1, None]
    return out.reshape(m, k)


def repack_nvfp4_v2(data, m: int, k: int) -> np.ndarray:
    """NVFP4 rows (V1) -> the same values in the V2 layout (uint8 [m*row_bytes]):
    per 36-byte group G of a row, bytes 4..35 go to quant bytes 32G..32G+31 and
    the scale word (bytes 0..3) to the row's scale bytes 4G..4G+3."""
    blk = _blocks(data, m, k, "nvfp4")                    # [m, k/64, 36]
    quants = blk[..., 4:36].reshape(m, -1)
    scales = blk[..., 0:4].reshape(m, -1)
    return np.concatenate([quants, scales], axis=1).reshape(-1).copy()


_DECODERS = {
    "f32": _decode_f32,
    "q4_0": _decode_q4_0,
    "q8_0": _decode_q8_0,
    "q4_k": _decode_q4_k,
    "q6_k": _decode_q6_k,
    "nvfp4": _decode_nvfp4,
    "nvfp4_v2": _decode_nvfp4_v2,
}


def decode(name: str, data, m: int, k: int) -> np.ndarray:
    """Decode an m x k weight matrix of format ``name`` to float64 [m, k]."""
    if name not in _DECODERS:
        raise ValueError(f"unknown qtype {name!r}")
    return _DECODERS[name](data, m, k)
