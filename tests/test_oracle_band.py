"""Pins of the oracle's bf16 rounding band (orc_layer_band), the tolerance
helper of the bf16-activation parity tests.

The band bounds how much the layer output can move when an h whose float value
lies within a relative window of a bf16 rounding midpoint takes the other
rounding.  Pinned here: zero for f32 activations, monotone in the window, and
at a window wide enough to make every h ambiguous it equals the sum over all h
of |w_j| * |down| * (bf16 spacing at h), with h rebuilt from the oracle's
decoded codes and the scales.
"""
import numpy as np
import pytest

import gen
import oracle


def _bf16_layer(seed=5):
    return gen.shrink(gen.get_config("c0"), act_dtype=gen.BF16, seed=seed)


def test_band_is_zero_for_f32_activations():
    cfg = gen.get_config("c0")
    hl = gen.host_layer(cfg, 0, experts="all")
    x = gen.x_tokens(cfg, 5, batch_id=3)
    assert not oracle.layer_band_host(hl, x, 1.0).any()


def test_band_is_monotone_in_the_window():
    cfg = _bf16_layer()
    hl = gen.host_layer(cfg, 0, experts="all")
    x = gen.x_tokens(cfg, 9, batch_id=4)
    prev = None
    for w in (0.0, 2.0 ** -20, 2.0 ** -12, 2.0 ** -6, 1.0):
        b = oracle.layer_band_host(hl, x, w)
        assert (b >= 0).all()
        if prev is not None:
            assert (b >= prev).all()
        prev = b


def _bf16_spacing(h):
    """Distance between the two bf16 values around the float h."""
    f = np.float32(h)
    bits = np.array([f], np.float32).view(np.uint32)[0]
    lo = np.array([bits & 0xFFFF0000], np.uint32).view(np.float32)[0]
    hi = np.array([(bits & 0xFFFF0000) + 0x10000], np.uint32).view(np.float32)[0]
    return abs(float(hi) - float(lo))


def test_widest_window_sums_every_h():
    cfg = _bf16_layer(seed=6)
    hl = gen.host_layer(cfg, 0, experts="all")
    T = 3
    x = gen.x_tokens(cfg, T, batch_id=5)
    band = oracle.layer_band_host(hl, x, 4.0)
    d = oracle.Desc.from_config(cfg)
    idx, _, w64 = oracle.route(d, hl.w_router, hl.bias, x, T)
    xv = gen.bf16_bits_to_f32(x).astype(np.float64)
    H, I = cfg.hidden, cfg.inter

    def dense(ex, rows, cols, which):
        # int codes times float scales, exact in double
        codes = oracle.decode_codes(ex["dtype"], np.ascontiguousarray(ex[which]), rows * cols)
        return codes.reshape(rows, cols).astype(np.float64) * \
            ex[which + "_scale"].astype(np.float64)[:, None]

    def term(ex, inter, t, weight):
        gu = dense(ex, 2 * inter, H, "gate_up")
        dn = dense(ex, H, inter, "down")
        g, u = gu[:inter] @ xv[t], gu[inter:] @ xv[t]
        h = g / (1.0 + np.exp(-g)) * u
        sp = np.array([_bf16_spacing(v) for v in h])
        return weight * (np.abs(dn) @ sp)

    for t in range(T):
        want = np.zeros(H)
        for j in range(cfg.top_k):
            want += term(hl.get(int(idx[t, j])), I, t, abs(float(w64[t, j])))
        if cfg.n_shared:
            want += term(hl.shared, I * cfg.n_shared, t, 1.0)
        np.testing.assert_allclose(band[t], want, rtol=1e-9, atol=0)
