"""Pins for the oracle's block decoders.

- golden hand-built blocks (tests/golden/q4_0_ramp.txt, q8_0_half.txt)
- decode(encode(fields)) == closed form, for every format, with random and
  exhaustive field values (test-only encoders in tests/encoders.py)
- one-hot scales identify exactly which elements each scale covers
- the literal scalar decoder equals the vectorized one byte for byte
"""

import os

import numpy as np
import pytest

import encoders as enc
from oracle import formats, scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, *vals = ln.split()
                out[key] = vals
    return out


def test_q4_0_golden_ramp_and_sign():
    g = _golden("q4_0_ramp.txt")
    for blk in ("A", "B"):
        data = np.array([int(h, 16) for h in g[blk]], dtype=np.uint8)
        want = np.array([float(v) for v in g[blk + "_values"]])
        got = formats.decode("q4_0", data, 1, 32)[0]
        assert np.array_equal(got, want)
        assert [scalar.element("q4_0", bytes(data), e) for e in range(32)] == list(want)
    # the encoder reproduces the golden bytes from the stated fields
    q = [j for j in range(16)] + [15 - j for j in range(16)]
    assert list(enc.q4_0(0x3C00, q)) == [int(h, 16) for h in g["A"]]


def test_q8_0_golden_half_scale():
    g = _golden("q8_0_half.txt")
    d = int(g["d"][0], 16)
    qs = np.arange(int(g["q_first"][0]), int(g["q_last"][0]) + 1)
    data = b"".join(enc.q8_0(d, qs[32 * b:32 * b + 32]) for b in range(8))
    got = formats.decode("q8_0", np.frombuffer(data, np.uint8), 1, 256)[0]
    assert np.array_equal(got, 0.5 * qs)


def _rand_f16_bits(rng, size, allow_sub=True):
    # finite f16 codes with random sign; optionally include subnormals
    e = rng.integers(0 if allow_sub else 1, 31, size=size)
    f = rng.integers(0, 1024, size=size)
    s = rng.integers(0, 2, size=size)
    return (s << 15) | (e << 10) | f


@pytest.mark.parametrize("seed", range(5))
def test_q4_0_q8_0_roundtrip(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        d = int(_rand_f16_bits(rng, 1)[0])
        dv = enc.f16_of_bits(d)
        q4 = rng.integers(0, 16, 32)
        got = formats.decode("q4_0", np.frombuffer(enc.q4_0(d, q4), np.uint8), 1, 32)[0]
        assert np.array_equal(got, dv * (q4 - 8.0))
        q8 = rng.integers(-128, 128, 32)
        got = formats.decode("q8_0", np.frombuffer(enc.q8_0(d, q8), np.uint8), 1, 32)[0]
        assert np.array_equal(got, dv * q8.astype(np.float64))


@pytest.mark.parametrize("seed", range(5))
def test_q4_k_roundtrip(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(10):
        d, dmin = (int(v) for v in _rand_f16_bits(rng, 2))
        sc = rng.integers(0, 64, 8)
        mn = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        blk = np.frombuffer(enc.q4_k(d, dmin, sc, mn, q), np.uint8)
        got = formats.decode("q4_k", blk, 1, 256)[0]
        dv, mv = enc.f16_of_bits(d), enc.f16_of_bits(dmin)
        j = np.arange(256) // 32                      # sub-block of each element
        want = dv * sc[j] * q - mv * mn[j]
        assert np.array_equal(got, want)


def test_q4_k_scale_min_packing_exhaustive():
    # every (scale, min) value in every one of the 8 slots, other slots zero
    d = 0x3C00  # 1.0
    dmin = 0x3C00
    for slot in range(8):
        blocks = []
        wants = []
        for s in range(64):
            for mval in range(64):
                sc = [0] * 8
                mn = [0] * 8
                sc[slot], mn[slot] = s, mval
                q = [1] * 256
                blocks.append(enc.q4_k(d, dmin, sc, mn, q))
                wants.append((s, mval))
        data = np.frombuffer(b"".join(blocks), np.uint8)
        got = formats.decode("q4_k", data, len(blocks), 256)
        want = np.zeros_like(got)
        for r, (s, mval) in enumerate(wants):
            want[r, 32 * slot:32 * slot + 32] = s * 1 - mval
        assert np.array_equal(got, want), slot


@pytest.mark.parametrize("seed", range(5))
def test_q6_k_roundtrip(seed):
    rng = np.random.default_rng(200 + seed)
    for _ in range(10):
        d = int(_rand_f16_bits(rng, 1)[0])
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        blk = np.frombuffer(enc.q6_k(d, sc, q), np.uint8)
        got = formats.decode("q6_k", blk, 1, 256)[0]
        want = enc.f16_of_bits(d) * sc[np.arange(256) // 16].astype(np.float64) * (q - 32)
        assert np.array_equal(got, want)


def test_q6_k_scale_index_one_hot():
    q = list(range(64)) * 4
    for i in range(16):
        sc = [0] * 16
        sc[i] = 1
        got = formats.decode("q6_k", np.frombuffer(enc.q6_k(0x3C00, sc, q), np.uint8), 1, 256)[0]
        nz = np.nonzero(got != 0)[0]
        assert set(nz) <= set(range(16 * i, 16 * i + 16))
        assert np.array_equal(got[16 * i:16 * i + 16], np.array(q[16 * i:16 * i + 16]) - 32.0)


@pytest.mark.parametrize("seed", range(5))
def test_nvfp4_roundtrip(seed):
    rng = np.random.default_rng(300 + seed)
    for _ in range(10):
        sbytes = rng.integers(0, 256, 4)
        sbytes[(sbytes & 0x7F) == 0x7F] = 0x38  # keep scales finite
        codes = rng.integers(0, 16, 64)
        blk = np.frombuffer(enc.nvfp4(sbytes, codes), np.uint8)
        got = formats.decode("nvfp4", blk, 1, 64)[0]
        sv = formats.e4m3_bits_to_f64(sbytes)
        want = np.array([enc.e2m1_value(codes[e]) * sv[e // 16] for e in range(64)])
        assert np.array_equal(got, want)


def test_nvfp4_scale_coverage_one_hot():
    codes = [2] * 64  # E2M1 code 2 = 1.0
    for g in range(4):
        sb = [0] * 4
        sb[g] = 0x38  # 1.0
        got = formats.decode("nvfp4", np.frombuffer(enc.nvfp4(sb, codes), np.uint8), 1, 64)[0]
        want = np.zeros(64)
        want[16 * g:16 * g + 16] = 1.0
        assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(3))
def test_nvfp4_v2_roundtrip(seed):
    """V2 rows built by the test encoder from chosen (scale, code) values
    decode to exactly those values."""
    rng = np.random.default_rng(400 + seed)
    k = 192
    sbytes = rng.integers(0, 256, k // 16)
    sbytes[(sbytes & 0x7F) == 0x7F] = 0x38
    codes = rng.integers(0, 16, k)
    row = np.frombuffer(enc.nvfp4_v2(sbytes, codes), np.uint8)
    assert row.size == formats.row_bytes("nvfp4_v2", k) == k // 32 * 18
    got = formats.decode("nvfp4_v2", row, 1, k)[0]
    sv = formats.e4m3_bits_to_f64(sbytes)
    assert np.array_equal(got, [enc.e2m1_value(codes[e]) * sv[e // 16] for e in range(k)])


def test_nvfp4_v2_scale_coverage_one_hot():
    """Scale byte g of a V2 row scales exactly elements 16g..16g+15."""
    k = 128
    for g in range(k // 16):
        sb = [0] * (k // 16)
        sb[g] = 0x40  # 2.0
        got = formats.decode("nvfp4_v2", np.frombuffer(enc.nvfp4_v2(sb, [2] * k), np.uint8), 1, k)[0]
        want = np.zeros(k)
        want[16 * g:16 * g + 16] = 2.0
        assert np.array_equal(got, want)


def test_nvfp4_v2_repack_keeps_values_and_matches_encoders():
    """The oracle's V1 -> V2 repack: decoded values are unchanged, and a V1
    row built by the V1 encoder repacks to the V2 encoder's bytes for the
    same (scale, code) values."""
    from synth import gen
    m, k = 5, 256
    v1 = gen.nvfp4_rows(m, k, 0x8181)
    v2 = formats.repack_nvfp4_v2(v1, m, k)
    assert v2.size == v1.size
    assert np.array_equal(formats.decode("nvfp4_v2", v2, m, k), formats.decode("nvfp4", v1, m, k))
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, k)
    sbytes = (rng.integers(0, 8, k // 16) | 0x38)
    v1_row = b"".join(enc.nvfp4(sbytes[4 * G:4 * G + 4], codes[64 * G:64 * G + 64]) for G in range(k // 64))
    got = formats.repack_nvfp4_v2(np.frombuffer(v1_row, np.uint8), 1, k)
    assert bytes(got) == enc.nvfp4_v2(sbytes, codes)


@pytest.mark.parametrize("qt", ["f32", "q4_0", "q8_0", "q4_k", "q6_k", "nvfp4", "nvfp4_v2"])
def test_scalar_equals_vectorized_random(qt):
    from synth import gen
    qk = formats.block_elems(qt)
    m, k = 3, max(2 * qk, 64)
    if qt == "f32":
        data = gen.unit_f32(m * k, 7).view(np.uint8)
    elif qt == "nvfp4":
        data = gen.nvfp4_rows(m, k, 11)
    elif qt == "nvfp4_v2":
        data = formats.repack_nvfp4_v2(gen.nvfp4_rows(m, k, 11), m, k)
    else:
        data = gen.quant_bytes(m * formats.row_bytes(qt, k), 13)
    vec = formats.decode(qt, data, m, k)
    lit = np.array(scalar.decode_matrix(qt, bytes(data), m, k))
    assert np.array_equal(vec, lit)


def test_generated_scales_finite_and_signed():
    """With the odd-byte mask every f16 scale is finite and both signs occur;
    without it about 1/32 of Q4_0 scales are Inf/NaN (cera wgpu_gemm_bench.rs,
    fill_quant_bytes doc comment: ~3% of Q4_0 blocks)."""
    from synth import gen
    nb = 20000
    for mask in (True, False):
        data = gen.quant_bytes(nb * 18, mask_odd=mask)
        d = formats.f16_bits_to_f64(data[0::18].astype(np.int64) | (data[1::18].astype(np.int64) << 8))
        bad = ~np.isfinite(d)
        if mask:
            assert not bad.any()
            assert 0.4 < (d < 0).mean() < 0.6
            sub = (data[1::18] & 0x7C) == 0
            assert 0.03 < sub.mean() < 0.10      # subnormal scales do occur
            assert np.abs(d).max() < 2.0
        else:
            assert 0.02 < bad.mean() < 0.045


def test_generators_deterministic_and_distinct():
    from synth import gen
    a = gen.quant_bytes(1000, 5)
    assert np.array_equal(a, gen.quant_bytes(1000, 5))
    assert not np.array_equal(a, gen.quant_bytes(1000, 6))
    x = gen.unit_f32(100000)
    assert x.min() >= -1.0 and x.max() < 1.0
    assert np.all((x * 32768.0) == np.round(x * 32768.0))
    v = gen.xorshift_f32(1000, 91)
    assert v.min() >= -1.0 and v.max() < 1.0
    ids = gen.expert_ids(16, 8, 64)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert len(np.unique(ids)) == 56
    rows = gen.nvfp4_rows(4, 128, 0x8181).reshape(-1, 36)
    assert np.all((rows[:, :4] & 0xF8) == 0x38)
