"""Test-only block ENCODERS: pack chosen field values into block bytes.

They are written in the packing direction from the same layout readings the
oracle's decoders follow (ggml-family block layouts, named by the pages; see
``oracle/formats.py``), share no code with either decoder, and let the tests
check decode(encode(fields)) == the closed-form value of every element.  A
transposed index, a dropped term or a wrong sign in a decoder breaks the round
trip.
"""

from __future__ import annotations

import numpy as np


def f16_bytes(value: float) -> tuple[int, int]:
    b = int(np.array([value], dtype=np.float16).view(np.uint16)[0])
    return b & 0xFF, b >> 8


def f16_of_bits(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def q4_0(d_bits: int, q) -> bytes:
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    out = bytearray([d_bits & 0xFF, d_bits >> 8])
    out += bytes(q[j] | (q[j + 16] << 4) for j in range(16))
    return bytes(out)


def q8_0(d_bits: int, q) -> bytes:
    q = [int(v) for v in q]
    assert len(q) == 32 and all(-128 <= v < 128 for v in q)
    return bytes([d_bits & 0xFF, d_bits >> 8] + [v & 0xFF for v in q])


def q4_k(d_bits: int, dmin_bits: int, scales, mins, q) -> bytes:
    scales = [int(v) for v in scales]
    mins = [int(v) for v in mins]
    q = [int(v) for v in q]
    assert len(scales) == 8 and len(mins) == 8 and len(q) == 256
    sc = [0] * 12
    for j in range(8):
        s, mn = scales[j], mins[j]
        assert 0 <= s < 64 and 0 <= mn < 64
        if j < 4:
            sc[j] |= s
            sc[j + 4] |= mn
        else:
            sc[j + 4] = (s & 0xF) | ((mn & 0xF) << 4)
            sc[j - 4] |= (s >> 4) << 6
            sc[j] |= (mn >> 4) << 6
    qs = [0] * 128
    for c in range(4):
        for l in range(32):
            lo, hi = q[64 * c + l], q[64 * c + 32 + l]
            assert 0 <= lo < 16 and 0 <= hi < 16
            qs[32 * c + l] = lo | (hi << 4)
    return bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8] + sc + qs)


def q6_k(d_bits: int, scales, q) -> bytes:
    scales = [int(v) for v in scales]
    q = [int(v) for v in q]
    assert len(scales) == 16 and len(q) == 256
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        v = q[e]
        assert 0 <= v < 64
        h, r = divmod(e, 128)
        quarter, l = divmod(r, 32)
        li = 64 * h + l + (32 if quarter & 1 else 0)
        if quarter < 2:
            ql[li] |= v & 0xF
        else:
            ql[li] |= (v & 0xF) << 4
        qh[32 * h + l] |= (v >> 4) << (2 * quarter)
    return bytes(ql + qh + [s & 0xFF for s in scales] + [d_bits & 0xFF, d_bits >> 8])


def nvfp4(scale_bytes, codes) -> bytes:
    scale_bytes = [int(v) for v in scale_bytes]
    codes = [int(v) for v in codes]
    assert len(scale_bytes) == 4 and len(codes) == 64
    qs = [0] * 32
    for e in range(64):
        h, r = divmod(e, 32)
        j = 16 * h + (r % 16)
        if r < 16:
            qs[j] |= codes[e] & 0xF
        else:
            qs[j] |= (codes[e] & 0xF) << 4
    return bytes(scale_bytes + qs)


def nvfp4_v2(scale_bytes, codes) -> bytes:
    """One V2 row of k = len(codes) elements: the quant bytes (group g's
    element 32g+j in the low nibble of byte 16g+j, element 32g+16+j in its
    high nibble), then the scale bytes (2g covers 32g..32g+15, 2g+1 the next 16)."""
    codes = [int(v) for v in codes]
    scale_bytes = [int(v) for v in scale_bytes]
    k = len(codes)
    assert k % 64 == 0 and len(scale_bytes) == k // 16
    qs = [0] * (k // 2)
    for e in range(k):
        g, r = divmod(e, 32)
        qs[16 * g + r % 16] |= (codes[e] & 0xF) << (4 if r >= 16 else 0)
    return bytes(qs + scale_bytes)


E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code: int) -> float:
    v = E2M1_MAG[code & 7]
    return -v if code & 8 else v
