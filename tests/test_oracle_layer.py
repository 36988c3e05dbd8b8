"""Pins of the oracle's whole layer (CPU only): a dense evaluation of every
expert for every token, written independently with numpy, must agree with
the oracle's sparse batch-union evaluation."""
import numpy as np
import pytest
from scipy.special import expit

import gen
import oracle


def _np_codes(packed, cols, dtype):
    packed = np.asarray(packed, np.uint8)
    out = np.empty((packed.shape[0], cols), np.int64)
    if dtype == gen.I4:
        out[:, 0::2] = (packed << 4).astype(np.int8) >> 4
        out[:, 1::2] = packed.astype(np.int8) >> 4
    elif dtype == gen.I8:
        out[:] = packed.view(np.int8)
    else:
        for j in range(4):
            out[:, j::4] = (packed << (6 - 2 * j)).astype(np.int8) >> 6
    return out


def _np_matrix(ex, key, cols):
    if ex["dtype"] == gen.BF16:
        return gen.bf16_bits_to_f32(ex[key]).astype(np.float64)
    q = _np_codes(ex[key], cols, ex["dtype"]).astype(np.float64)
    return q * ex[key + "_scale"].astype(np.float64)[:, None]


def _bf16_round(h):
    """Nearest bf16 of float32(h), ties to even, by comparing the two
    neighbouring bf16 values (independent of the bit-add trick)."""
    f = h.astype(np.float32)
    u = f.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    fd = f.astype(np.float64)
    dlo, dhi = np.abs(fd - lo), np.abs(hi - fd)
    lo_even = ((u >> 16) & 1) == 0
    pick_lo = (dlo < dhi) | ((dlo == dhi) & lo_even)
    return np.where(pick_lo, lo, hi)


def _np_ffn(ex, x, H, I, act_bf16):
    W = _np_matrix(ex, "gate_up", H)
    D = _np_matrix(ex, "down", I)
    g, u = x @ W[:I].T, x @ W[I:].T
    h = g * expit(g) * u
    if act_bf16:
        h = _bf16_round(h)
    return h @ D.T


def _dense_layer(cfg, hl, x64, idx, w64):
    """All experts on all tokens, combined with a dense weight matrix that is
    zero for unselected experts."""
    T = x64.shape[0]
    wfull = np.zeros((T, cfg.n_experts))
    for t in range(T):
        wfull[t, idx[t]] = w64[t]
    out = np.zeros((T, cfg.hidden))
    for e in range(cfg.n_experts):
        out += wfull[:, e:e + 1] * _np_ffn(hl.get(e), x64, cfg.hidden, cfg.inter,
                                          cfg.act_dtype == gen.BF16)
    if cfg.n_shared:
        out += _np_ffn(hl.shared, x64, cfg.hidden, cfg.inter * cfg.n_shared,
                       cfg.act_dtype == gen.BF16)
    return out


SMALL = [
    dict(base="c0"),
    dict(base="c0", expert_dtype=gen.I2, hidden=128, inter=64),
    dict(base="c0", expert_dtype=gen.I8, shared_dtype=gen.I8, hidden=128, inter=64),
    dict(base="c2", hidden=128, inter=64, n_experts=16, n_group=4, topk_group=2, top_k=4),
    dict(base="c3", hidden=128, inter=64, n_experts=16, n_group=4, topk_group=2, top_k=4),
    dict(base="c1", hidden=64, inter=32, n_experts=8, top_k=3),
    dict(base="c2", hidden=64, inter=64, n_experts=6, n_group=1, topk_group=1, top_k=6,
         shared_dtype=gen.I4),
]


def _small_cfg(spec):
    spec = dict(spec)
    base = gen.get_config(spec.pop("base"))
    return gen.shrink(base, **spec)


def _x_as_f64(cfg, x):
    return gen.bf16_bits_to_f32(x).astype(np.float64) if cfg.act_dtype == gen.BF16 else x.astype(np.float64)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_sparse_equals_dense(spec):
    cfg = _small_cfg(spec)
    hl = gen.host_layer(cfg, 0, experts="all")
    T = 5
    x = gen.x_tokens(cfg, T)
    d = oracle.Desc.from_config(cfg)
    out, idx, w = oracle.layer_forward_host(hl, x)
    _, _, w64 = oracle.route(d, hl.w_router, hl.bias, x, T)
    dense = _dense_layer(cfg, hl, _x_as_f64(cfg, x), idx, w64)
    rms = np.sqrt((dense ** 2).mean())
    assert np.abs(out - dense).max() <= 1e-12 * rms


@pytest.mark.parametrize("spec", SMALL[:4], ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_batch_union_equals_per_token(spec):
    cfg = _small_cfg(spec)
    hl = gen.host_layer(cfg, 0, experts="all")
    T = 9
    x = gen.x_tokens(cfg, T, batch_id=1)
    d = oracle.Desc.from_config(cfg)
    routed = oracle.expert_set_from_host_layer(hl)
    shared = oracle.shared_set_from_host_layer(hl)
    bu, _, _ = oracle.layer_forward(d, hl.w_router, hl.bias, routed, shared, x, T)
    pt = oracle.layer_forward_per_token(d, hl.w_router, hl.bias, routed, shared, x, T)
    assert np.array_equal(bu, pt)
    # token permutation equivariance, bitwise
    perm = np.random.default_rng(0).permutation(T)
    bp, _, _ = oracle.layer_forward(d, hl.w_router, hl.bias, routed, shared,
                                    np.ascontiguousarray(x[perm]), T)
    assert np.array_equal(bp, bu[perm])


def test_zero_input_gives_zero():
    cfg = gen.get_config("c0")
    hl = gen.host_layer(cfg, 0, experts="all")
    out, idx, w = oracle.layer_forward_host(hl, np.zeros((2, cfg.hidden), np.float32))
    assert (out == 0).all()


def test_single_expert_layer():
    cfg = gen.shrink(gen.get_config("c0"), n_experts=1, top_k=1, n_group=1, topk_group=1)
    hl = gen.host_layer(cfg, 0, experts="all")
    x = gen.x_tokens(cfg, 3)
    d = oracle.Desc.from_config(cfg)
    out, idx, w = oracle.layer_forward_host(hl, x)
    assert (idx == 0).all() and (w == np.float32(cfg.routed_scaling)).all()
    f = oracle.expert_ffn(d, oracle.ExpertSet(gen.I4, [hl.get(0)]), 0, x, n_rows=3)
    s = oracle.expert_ffn(d, oracle.shared_set_from_host_layer(hl), 0, x, n_rows=3)
    assert np.array_equal(out, cfg.routed_scaling * f + s)


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(6, 1024)).astype(np.float32) * np.array([1, 10, 1e-3, 3, 0.5, 100],
                                                                  np.float32)[:, None]
    eps = 1e-6
    y = oracle.rmsnorm(x, eps)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    rms_out = np.sqrt((y.astype(np.float64) ** 2).mean(axis=1))
    assert np.allclose(rms_out, 1.0 / np.sqrt(1.0 + eps / ms), rtol=1e-6)
    c = np.full((1, 64), 3.0, np.float32)   # constant row: value 3/sqrt(9+eps)
    assert abs(float(oracle.rmsnorm(c, eps)[0, 0]) - 3.0 / np.sqrt(9.0 + eps)) < 1e-7
    assert (oracle.rmsnorm(np.zeros((1, 8), np.float32), eps) == 0).all()


def test_residual_add_is_float_addition():
    x = np.array([1.0, 1e8, -2.5, 3.0], np.float32)
    y = np.array([2.0 ** -30, 1.0, 2.5, 0.1], np.float64)
    got = oracle.residual_add(x, y)
    want = x + y.astype(np.float32)
    assert np.array_equal(got, want)


def widened_layer(hl4):
    """The same layer with every int4 expert re-packed into the int8 container."""
    cfg = hl4.cfg
    hl8 = gen.HostLayer(cfg=cfg, layer=hl4.layer, w_router=hl4.w_router, bias=hl4.bias,
                        dtype=gen.I8)
    for e in range(cfg.n_experts):
        hl8.experts[e] = gen.expert_i8_from_i4(hl4.get(e), cfg.hidden, cfg.inter)
    hl8.shared = hl4.shared
    return hl8


@pytest.mark.parametrize("spec", [SMALL[0], SMALL[3]], ids=["c0", "c2small"])
def test_int8_container_of_int4_codes_is_bitwise_identical(spec):
    """The int8 container holding int4 codes (the pages validate the int4
    packing bit-identical to the int8 container) defines the same layer: the
    oracle's outputs agree bit for bit."""
    cfg = _small_cfg(spec)
    hl4 = gen.host_layer(cfg, 0, experts="all")
    hl8 = widened_layer(hl4)
    x = gen.x_tokens(cfg, 6, batch_id=2)
    o4, i4, w4 = oracle.layer_forward_host(hl4, x)
    o8, i8, w8 = oracle.layer_forward_host(hl8, x)
    assert np.array_equal(i4, i8) and np.array_equal(w4, w8)
    assert np.array_equal(o4.view(np.uint64), o8.view(np.uint64))
