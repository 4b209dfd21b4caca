"""Pins for the oracle's element codecs (f16, E4M3FN, E2M1) and packed sizes.

Each codec is checked against (a) the golden fixtures under tests/golden and
(b) an independent library routine over every code.
"""

import os

import numpy as np
import pytest

from oracle import formats
from oracle import scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_packed_sizes_match_pages():
    for qt, qk, bb in _rows("packed_sizes.txt"):
        assert formats.block_elems(qt) == int(qk)
        assert formats.block_bytes(qt) == int(bb)
    # LFM2 shapes: packed bytes of a 4608x1024 matrix per format
    e = 4608 * 1024
    assert formats.row_bytes("f32", 1024) * 4608 == e * 4
    assert formats.row_bytes("q4_0", 1024) * 4608 == e // 32 * 18 == 2654208
    assert formats.row_bytes("q8_0", 1024) * 4608 == e // 32 * 34 == 5013504
    assert formats.row_bytes("q4_k", 1024) * 4608 == e // 256 * 144 == 2654208
    assert formats.row_bytes("q6_k", 1024) * 4608 == e // 256 * 210 == 3870720
    assert formats.row_bytes("nvfp4", 4096) == 4096 // 64 * 36 == 2304
    with pytest.raises(ValueError):
        formats.row_bytes("q4_k", 1000)


def test_f16_golden():
    for hx, val in _rows("f16_hand.txt"):
        got = float(formats.f16_bits_to_f64(int(hx, 16)))
        assert got == float(val) and np.signbit(got) == np.signbit(float(val)), hx
        lo, hi = int(hx, 16) & 0xFF, int(hx, 16) >> 8
        assert scalar.half(lo, hi) == float(val)


def test_f16_all_codes_vs_numpy():
    codes = np.arange(65536, dtype=np.uint32)
    ours = formats.f16_bits_to_f64(codes)
    lib = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))
    # the literal decoder agrees on every code too
    sc = np.array([scalar.half(c & 0xFF, c >> 8) for c in range(65536)])
    assert np.array_equal(np.isnan(sc), nan)
    assert np.array_equal(sc[~nan], lib[~nan])


def test_e4m3_all_codes_vs_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.e4m3_bits_to_f64(codes)
    nan = np.isnan(lib)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    lit = np.array([scalar.fp8_e4m3(int(c)) for c in codes])
    assert np.array_equal(lit[~nan], lib[~nan])


def test_e4m3_generator_scale_bytes():
    for hx, val in _rows("e4m3_scale_bytes.txt"):
        assert float(formats.e4m3_bits_to_f64(int(hx, 16))) == float(val)


def test_e2m1_golden_and_torch():
    torch = pytest.importorskip("torch")
    rows = _rows("e2m1_codes.txt")
    for code, val in rows:
        assert float(formats.e2m1_bits_to_f64(int(code))) == float(val)
        assert scalar.fp4_e2m1(int(code)) == float(val)
    # torch has no float4 -> float copy kernel here, so widen each E2M1 code
    # into the E4M3FN byte with the same sign, exponent and mantissa (exponent
    # bias 1 -> 7, mantissa bit -> the top mantissa bit) and let torch's
    # float8_e4m3fn decode it.  Subnormal E2M1 (exponent 0) is m * 0.5, which
    # is the normal E4M3 code with exponent 2^-1 when m = 1.
    wide = []
    for c in range(16):
        s_, e, m_ = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e == 0:
            byte = (s_ << 7) | ((0x30) if m_ else 0)
        else:
            byte = (s_ << 7) | ((e - 1 + 7) << 3) | (m_ << 2)
        wide.append(byte)
    lib = torch.tensor(wide, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.e2m1_bits_to_f64(np.arange(16))
    assert np.array_equal(lib, ours)
    assert np.array_equal(np.signbit(lib), np.signbit(ours))
