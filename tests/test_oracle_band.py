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


# ------------------------------------------------------------------------
# The window test of the band, pinned at its operating width: a hand-built
# layer (one int4 expert, H = 2, I = 2, weight 1) whose SwiGLU output h0 is
# placed just inside or just outside window * e0 of a bf16 rounding midpoint,
# on both sides of it and at several magnitudes.  g0 = 1 (gate codes (1, 0),
# scale 1, x = (1, 0)), u0 = s_u (up codes (1, 0), scale s_u), so
# h0 = silu(1) s_u with s_u a float chosen to put h0 where wanted, and its
# error scale is e0 = |silu'(1) u0| * |1| + |silu(1)| * |u0| (the sums of g0
# and u0 have one term each), silu'(v) = s (1 + v (1 - s)), s = logistic(v).
# Down rows (1, 0) and (2, 0) with unit scales: an ambiguous h0 gives band =
# (1, 2) * (bf16 spacing at h0); otherwise the band is 0 (h1 = 0 is never
# ambiguous).

WINDOW = 2.0 ** -18
SIG1 = 1.0 / (1.0 + np.exp(-1.0))            # logistic(1)
DSILU1 = SIG1 * (1.0 + 1.0 * (1.0 - SIG1))   # silu'(1)


def _pinned_layer(s_u):
    d = oracle.Desc(hidden=2, inter=2, n_experts=1, top_k=1, n_group=1, topk_group=1,
                    routed_scaling=1.0, expert_dtype=oracle.I4, act_bf16=1)
    pack = lambda rows: np.array([[(a & 0xF) | ((b & 0xF) << 4)] for a, b in rows], np.uint8)
    ex = dict(gate_up=pack([(1, 0), (0, 0), (1, 0), (0, 0)]),
              gate_up_scale=np.array([1.0, 1.0, s_u, 1.0], np.float32),
              down=pack([(1, 0), (2, 0)]), down_scale=np.array([1.0, 1.0], np.float32))
    routed = oracle.ExpertSet(oracle.I4, [ex])
    w_router = np.ones((1, 2), np.float32)
    x = np.array([[0x3F80, 0x0000]], np.uint16)   # bf16 (1, 0)
    return d, w_router, routed, x


def _e0(u):
    return abs(DSILU1 * u) + abs(SIG1 * u)


@pytest.mark.parametrize("mid", [1.0 + 2.0 ** -8, 96.25, 0.010772705078125, -3.0390625])
@pytest.mark.parametrize("side", [-1.0, 1.0])
@pytest.mark.parametrize("rel,inside", [(0.5, True), (0.9, True), (1.1, False), (2.0, False)])
def test_band_window_around_a_midpoint(mid, side, rel, inside):
    # mid lies halfway between two adjacent bf16 values (checked here)
    spacing = _bf16_spacing(mid)
    lo = np.floor(abs(mid) / spacing) * spacing
    assert abs(abs(mid) - (lo + spacing / 2)) == 0.0
    u_mid = mid / SIG1
    s_u = np.float32((mid + side * rel * WINDOW * _e0(u_mid)) / SIG1)
    h0 = np.float32(SIG1 * float(s_u))
    dist = abs(float(h0) - mid) / (WINDOW * _e0(float(s_u)))
    assert (dist <= 1.0) == inside, (dist, inside)
    d, w_router, routed, x = _pinned_layer(s_u)
    # the oracle's error scale of h0 is the closed form above
    h, e = oracle.expert_h(d, routed, 0, x, n_rows=1, with_scale=True)
    assert h[0, 0] == SIG1 * float(s_u)
    np.testing.assert_allclose(e[0, 0], _e0(float(s_u)), rtol=1e-14)
    band = oracle.layer_band(d, w_router, None, routed, None, x, 1, WINDOW)
    want = np.array([1.0, 2.0]) * _bf16_spacing(h0) if inside else np.zeros(2)
    np.testing.assert_array_equal(band[0], want)
