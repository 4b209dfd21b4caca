"""A literal, per-element decoder in pure Python.  TEST INFRASTRUCTURE.

Written independently of ``oracle.formats`` (no shared helper): each call
reads the bytes of one block and evaluates one element's formula with Python
ints and floats.  It exists so that the vectorized decoder can be checked
against a second reading of the same definitions on small random inputs, and
for brute-force GEMMs of tiny shapes.
"""

from __future__ import annotations

import math

_SIZES = {"f32": (1, 4), "q4_0": (32, 18), "q8_0": (32, 34), "q4_k": (256, 144),
          "q6_k": (256, 210), "nvfp4": (64, 36), "nvfp4_v2": (64, 36)}


def half(lo: int, hi: int) -> float:
    v = lo | (hi << 8)
    s = -1.0 if v & 0x8000 else 1.0
    e = (v >> 10) & 31
    f = v & 1023
    if e == 0:
        return s * f * 2.0 ** -24
    if e == 31:
        return s * math.inf if f == 0 else math.nan
    return s * (1024 + f) * 2.0 ** (e - 25)


def fp8_e4m3(b: int) -> float:
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 15
    mnt = b & 7
    if e == 15 and mnt == 7:
        return math.nan
    if e == 0:
        return s * mnt * 2.0 ** -9
    return s * (8 + mnt) * 2.0 ** (e - 10)


def fp4_e2m1(c: int) -> float:
    mag = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)[c & 7]
    return -mag if c & 8 else mag


def int8(b: int) -> int:
    return b - 256 if b >= 128 else b


def element(name: str, row: bytes, e: int) -> float:
    """Weight number ``e`` of one packed row."""
    qk, bb = _SIZES[name]
    if name == "f32":
        import struct
        return struct.unpack_from("<f", row, 4 * e)[0]
    blk = row[(e // qk) * bb:(e // qk + 1) * bb]
    i = e % qk
    if name == "q4_0":
        d = half(blk[0], blk[1])
        byte = blk[2 + (i % 16)]
        q = (byte & 15) if i < 16 else (byte >> 4)
        return d * (q - 8)
    if name == "q8_0":
        return half(blk[0], blk[1]) * int8(blk[2 + i])
    if name == "q4_k":
        d = half(blk[0], blk[1])
        dmin = half(blk[2], blk[3])
        sc = blk[4:16]
        chunk, r = divmod(i, 64)
        j = 2 * chunk + (1 if r >= 32 else 0)
        if j < 4:
            scale, mn = sc[j] & 63, sc[j + 4] & 63
        else:
            scale = (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4)
            mn = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4)
        byte = blk[16 + 32 * chunk + (r % 32)]
        q = (byte & 15) if r < 32 else (byte >> 4)
        return d * scale * q - dmin * mn
    if name == "q6_k":
        h, r = divmod(i, 128)
        quarter, l = divmod(r, 32)
        ql = blk[64 * h + l + (32 if quarter in (1, 3) else 0)]
        low = (ql & 15) if quarter < 2 else (ql >> 4)
        qh = blk[128 + 32 * h + l]
        high = (qh >> (2 * quarter)) & 3
        q = low | (high << 4)
        d = half(blk[208], blk[209])
        return d * int8(blk[192 + i // 16]) * (q - 32)
    if name == "nvfp4_v2":
        # row = k/2 quant bytes, then k/16 scale bytes (two per 32-element group)
        k = len(row) // 18 * 32
        g, r = divmod(e, 32)
        byte = row[16 * g + (r % 16)]
        code = (byte & 15) if r < 16 else (byte >> 4)
        return fp4_e2m1(code) * fp8_e4m3(row[k // 2 + 2 * g + (1 if r >= 16 else 0)])
    if name == "nvfp4":
        h, r = divmod(i, 32)
        byte = blk[4 + 16 * h + (r % 16)]
        code = (byte & 15) if r < 16 else (byte >> 4)
        scale = fp8_e4m3(blk[2 * h + (1 if r >= 16 else 0)])
        return fp4_e2m1(code) * scale
    raise ValueError(name)


def decode_matrix(name: str, data: bytes, m: int, k: int):
    qk, bb = _SIZES[name]
    rb = k // qk * bb
    return [[element(name, data[i * rb:(i + 1) * rb], c) for c in range(k)] for i in range(m)]


def gemm(name: str, data: bytes, x, m: int, k: int, n: int):
    """Brute force dst[j][i] = fsum_c W[i][c] * x[j][c] (exactly rounded sum)."""
    W = decode_matrix(name, data, m, k)
    return [[math.fsum(W[i][c] * float(x[j][c]) for c in range(k)) for i in range(m)]
            for j in range(n)]
