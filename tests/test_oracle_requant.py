"""Pins of the oracle's FP8 -> int4 requantizer (CPU only).

FP8 here is OCP E4M3 without infinities (torch's float8_e4m3fn); the
checkpoint's 128x128 block scales multiply it; the int4 container takes one
fp32 scale per row, m / 7 for the row's absolute maximum m, and codes
rounded to nearest even and clamped to [-7, 7] (our reading: the pages fix
neither).  The decoder is checked against torch's conversion of every byte;
the requantizer against cases whose answer is exact by construction and
against the rounding bound.
"""
import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _torch_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _unpack(codes, cols):
    b = np.asarray(codes, np.uint8)
    out = np.empty((b.shape[0], cols), np.int64)
    out[:, 0::2] = (b << 4).astype(np.int8) >> 4
    out[:, 1::2] = b.astype(np.int8) >> 4
    return out


def _e4m3_of(values):
    """FP8 bytes of float values that E4M3 holds exactly (via torch)."""
    t = torch.tensor(np.asarray(values, np.float32)).to(torch.float8_e4m3fn)
    back = t.float().numpy()
    assert np.array_equal(back, np.asarray(values, np.float32)), "value not exact in E4M3"
    return t.view(torch.uint8).numpy()


def test_decode_every_byte_against_torch():
    allb = np.arange(256, dtype=np.uint8)
    got = oracle.decode_e4m3(allb)
    want = _torch_e4m3(allb)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_worked_values():
    b = np.array([0x00, 0x01, 0x08, 0x38, 0xB8, 0x7E, 0x40, 0x3C], np.uint8)
    assert oracle.decode_e4m3(b).tolist() == [0.0, 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 448.0, 2.0, 1.5]


def test_integer_multiples_round_trip():
    """A row of k * u (k in [-7, 7], the absmax 7u present) with u = 1/4 and
    block scale 1 requantizes to scale u and codes k exactly."""
    rng = np.random.default_rng(0)
    k = rng.integers(-7, 8, size=(3, 256))
    k[:, 5] = 7
    k[1, 9] = -7
    fp8 = _e4m3_of(k * 0.25)
    codes, scales = oracle.requant_fp8_int4(fp8, np.ones((1, 2), np.float32))
    assert (scales == np.float32(0.25)).all()
    assert np.array_equal(_unpack(codes, 256), k)


def test_block_scales_apply_per_block():
    """Two row blocks and three column blocks (ragged at both ends) with
    distinct power-of-two scales: w = e4m3 * scale of the element's block."""
    rows, cols, blk = 200, 300, 128
    rng = np.random.default_rng(1)
    vals = rng.integers(-6, 7, size=(rows, cols)).astype(np.float32)
    bs = np.array([[1.0, 2.0, 0.5], [4.0, 0.25, 8.0]], np.float32)
    codes, scales = oracle.requant_fp8_int4(_e4m3_of(vals), bs, blk)
    w = vals.astype(np.float64) * np.repeat(np.repeat(bs, blk, 0), blk, 1)[:rows, :cols]
    m = np.abs(w).max(axis=1)
    assert np.array_equal(scales, (m / 7.0).astype(np.float32))
    q = _unpack(codes, cols)
    s = scales.astype(np.float64)[:, None]
    assert (np.abs(q * s - w) <= s / 2 + 0 * s).all()
    assert (np.abs(q) <= 7).all()
    assert (np.abs(q)[np.arange(rows), np.abs(w).argmax(axis=1)] == 7).all()


def test_rounding_bound_and_absmax_on_random_fp8():
    rng = np.random.default_rng(2)
    raw = rng.integers(0, 256, size=(64, 512)).astype(np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x10   # no NaN codes
    bs = rng.uniform(0.001, 0.01, size=(1, 4)).astype(np.float32)
    codes, scales = oracle.requant_fp8_int4(raw, bs)
    w = _torch_e4m3(raw) * np.repeat(bs.astype(np.float64), 128, 1)
    s = scales.astype(np.float64)[:, None]
    q = _unpack(codes, 512)
    # nearest: the error is at most half a step (one more step only where the
    # fp32 scale rounded m / 7 down and the absmax element would exceed 7)
    assert (np.abs(q * s - w) <= s / 2 * (1 + 1e-6)).all()
    assert (np.abs(q)[np.arange(64), np.abs(w).argmax(axis=1)] == 7).all()


def test_ties_to_even_and_zero_rows():
    # w / s = k + 1/2 exactly: scale 2 (m = 14), values 5 (2.5 -> 2), 7 (3.5 -> 4), -3 (-1.5 -> -2)
    row = np.array([14.0, 5.0, 7.0, -3.0, 1.0, 0.0, -14.0, 3.0], np.float32)
    codes, scales = oracle.requant_fp8_int4(_e4m3_of(row[None, :]), np.ones((1, 1), np.float32))
    assert scales[0] == 2.0
    assert _unpack(codes, 8)[0].tolist() == [7, 2, 4, -2, 0, 0, -7, 2]
    zc, zs = oracle.requant_fp8_int4(np.zeros((2, 16), np.uint8), np.ones((1, 1), np.float32))
    assert (zs == 0).all() and (zc == 0).all()


def test_nan_code_is_an_error():
    b = np.zeros((1, 8), np.uint8)
    b[0, 3] = 0x7F
    with pytest.raises(Exception):
        oracle.requant_fp8_int4(b, np.ones((1, 1), np.float32))
