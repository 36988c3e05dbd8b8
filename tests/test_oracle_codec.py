"""Pins of the oracle's code decoder and dequantization (CPU only)."""
import json
import os

import numpy as np
import pytest

import gen
import oracle



def _np_int4_pairs(b):
    """Independent decode with numpy's arithmetic shifts on int8."""
    b = np.asarray(b, dtype=np.uint8)
    lo = ((b << 4).astype(np.int8) >> 4).astype(np.int8)
    hi = (b.astype(np.int8) >> 4).astype(np.int8)
    return lo, hi


def _np_int2_quads(b):
    b = np.asarray(b, dtype=np.uint8)
    return [((b << (6 - 2 * j)).astype(np.int8) >> 6).astype(np.int8) for j in range(4)]


def test_worked_bytes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "codec_worked_bytes.json")))
    for case in g["int4"]:
        got = oracle.decode_codes(oracle.I4, np.array([int(case["byte"], 16)], np.uint8), 2)
        assert got.tolist() == case["codes"], case
    for case in g["int2"]:
        got = oracle.decode_codes(oracle.I2, np.array([int(case["byte"], 16)], np.uint8), 4)
        assert got.tolist() == case["codes"], case


def test_int4_exhaustive():
    allb = np.arange(256, dtype=np.uint8)
    got = oracle.decode_codes(oracle.I4, allb, 512).reshape(256, 2)
    lo, hi = _np_int4_pairs(allb)
    assert np.array_equal(got[:, 0], lo) and np.array_equal(got[:, 1], hi)
    # bijection onto [-8, 7]^2
    pairs = {(int(a), int(b)) for a, b in got}
    assert len(pairs) == 256 and min(got.ravel()) == -8 and max(got.ravel()) == 7


def test_int2_exhaustive():
    allb = np.arange(256, dtype=np.uint8)
    got = oracle.decode_codes(oracle.I2, allb, 1024).reshape(256, 4)
    quads = _np_int2_quads(allb)
    for j in range(4):
        assert np.array_equal(got[:, j], quads[j])
    assert len({tuple(r) for r in got.tolist()}) == 256
    assert got.min() == -2 and got.max() == 1


def test_generator_codes_roundtrip():
    """gen's packer emits symmetric codes on [-7, 7], roughly uniform; the
    oracle's decoder reads back exactly what numpy's shifts read."""
    packed = gen.int4_codes(seed=11, layer=0, tensor=gen.T_GU_CODES, expert=3, rows=64, cols=512)
    dec = oracle.decode_codes(oracle.I4, packed, packed.size * 2)
    lo, hi = _np_int4_pairs(packed.ravel())
    assert np.array_equal(dec[0::2], lo) and np.array_equal(dec[1::2], hi)
    assert dec.min() == -7 and dec.max() == 7
    counts = np.bincount(dec.astype(np.int64) + 7, minlength=15)
    exp = dec.size / 15
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 60, chi2   # 14 dof; p ~ 1e-7


def test_int2_variant_of_int4():
    cols = 256
    c4 = gen.int4_codes(seed=4, layer=1, tensor=gen.T_DN_CODES, expert=5, rows=16, cols=cols)
    s4 = gen.scales(4, 1, gen.T_DN_SCALES, 5, 16, 1.0)
    c2, s2 = gen.int2_from_int4(c4, s4, cols)
    q4 = oracle.decode_codes(oracle.I4, c4, c4.size * 2).reshape(16, cols).astype(np.int64)
    q2 = oracle.decode_codes(oracle.I2, c2, c2.size * 4).reshape(16, cols).astype(np.int64)
    m = np.abs(q4).max(axis=1)
    # round-half-even of q4/m clamped to [-1, 1], by exact rational comparison
    want = np.where(2 * np.abs(q4) > m[:, None], np.sign(q4), 0)
    assert np.array_equal(q2, want)
    assert np.array_equal(s2, (s4.astype(np.float64) * m).astype(np.float32))


def test_dequant_integer_and_pow2_scales():
    rng = np.random.default_rng(0)
    cols = 64
    packed = rng.integers(0, 256, size=(8, cols // 2), dtype=np.uint8)
    lo, hi = _np_int4_pairs(packed)
    q = np.empty((8, cols), np.int8)
    q[:, 0::2], q[:, 1::2] = lo, hi
    ones = np.ones(8, np.float32)
    assert np.array_equal(oracle.dequant_rows(oracle.I4, packed, ones, cols, 0, 8), q.astype(np.float32))
    pow2 = (2.0 ** rng.integers(-20, 5, size=8)).astype(np.float32)
    got = oracle.dequant_rows(oracle.I4, packed, pow2, cols, 2, 5)
    assert np.array_equal(got, q[2:7].astype(np.float32) * pow2[2:7, None])
    # a general scale: one correctly rounded float multiply
    s = rng.uniform(0.01, 0.05, size=8).astype(np.float32)
    got = oracle.dequant_rows(oracle.I4, packed, s, cols, 0, 8)
    exact = q.astype(np.float64) * s.astype(np.float64)[:, None]
    assert np.array_equal(got, exact.astype(np.float32))


def test_int8_exhaustive():
    """The int8 container: every byte decodes to its two's-complement value."""
    allb = np.arange(256, dtype=np.uint8)
    got = oracle.decode_codes(oracle.I8, allb, 256)
    assert np.array_equal(got, allb.view(np.int8))
    assert got.min() == -128 and got.max() == 127


def test_int8_dequant_exact():
    """q * s in float for int8 codes: integer and power-of-two scales make
    every product exact, so the oracle's float multiply must reproduce them."""
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    scales = np.array([1.0, 0.5, 3.0, 2.0 ** -10], dtype=np.float32)
    got = oracle.dequant_rows(oracle.I8, codes, scales, 64, 0, 4)
    want = codes.view(np.int8).astype(np.float64) * scales.astype(np.float64)[:, None]
    assert np.array_equal(got.astype(np.float64), want)


def test_int8_widening_of_int4_codes():
    """gen's int4 -> int8 re-packing keeps every code: decoding the int8
    container gives the int4 container's codes."""
    packed = gen.int4_codes(seed=5, layer=1, tensor=gen.T_DN_CODES, expert=2, rows=16, cols=256)
    wide = gen.int8_from_int4(packed, 256)
    assert wide.shape == (16, 256)
    d4 = oracle.decode_codes(oracle.I4, packed, packed.size * 2)
    d8 = oracle.decode_codes(oracle.I8, wide, wide.size)
    assert np.array_equal(d4, d8)


def test_int8_generator_range():
    """Full-range int8 codes: symmetric on [-127, 127], every value drawn."""
    c = gen.int8_codes(seed=3, layer=0, tensor=gen.T_GU_I8, expert=1, rows=64, cols=1024)
    v = oracle.decode_codes(oracle.I8, c, c.size).astype(np.int64)
    assert v.min() == -127 and v.max() == 127
    assert len(np.unique(v)) == 255
    assert abs(v.mean()) < 1.0
